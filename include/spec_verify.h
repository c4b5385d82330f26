/*
 * spec_verify.h -- C ABI of the target-model verification step of
 * speculative decoding, for one AMD Instinct MI355X (gfx950) GPU.
 *
 * What the step computes (one call of spec_verify_step):
 *   One target pass over the block [pending, d_1 .. d_k] at cache positions
 *   L .. L+k gives k+1 rows of logits; row j is what the target would write
 *   after block token j.  (Essay "LLM Inference: Speculative Decoding",
 *   section "The loop", step 2; why one pass answers every prefix: section
 *   "The four sentences are already inside one sentence".)
 *   Greedy acceptance keeps the longest prefix of drafts that agrees with the
 *   row-wise argmax and returns the target's own token after it (same
 *   section, steps 3-4).  Stochastic acceptance applies the rule of Leviathan
 *   et al. that the essay names in "What is not here": accept d_i with
 *   probability min(1, p/q), otherwise resample from the normalized positive
 *   part of p - q; a bonus token is drawn from the last row when all drafts
 *   pass.  Only accepted entries stay in the KV cache (essay "The loop",
 *   step 5; S2-MoE section 4.3, where the cache shared by drafting and
 *   verification keeps the entries of accepted tokens alone).
 *
 * Conventions
 *   - Every function returns a spec_status (0 = SPEC_OK) unless stated.
 *     On error the handle's state is unchanged and spec_last_error()
 *     describes the failure.  A GPU runtime failure in the middle of a step
 *     (SPEC_EHIP) leaves the handle unusable: later calls return
 *     SPEC_ESTATE.
 *   - "host" pointers are ordinary CPU memory; "device" pointers are GPU
 *     memory on the device that was current at spec_verify_create (for
 *     example a torch tensor's data_ptr()).  The caller owns every pointer
 *     it passes; the library keeps none of them after the call returns.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream);
 *     all work of a handle is enqueued on it.  Streams must have the
 *     default priority.
 *   - A handle is not thread-safe; calls on one handle must not overlap.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct spec_verify spec_verify_t;   /* opaque: device weights + KV pages */

typedef enum {
  SPEC_OK = 0,
  SPEC_EINVAL = -1,     /* invalid argument */
  SPEC_ENOMEM = -2,     /* device or pinned-host allocation failed */
  SPEC_ECAPACITY = -3,  /* block does not fit in max_ctx */
  SPEC_EHIP = -4,       /* GPU runtime error */
  SPEC_ESTATE = -5      /* handle unusable after an earlier GPU error */
} spec_status;

typedef enum { SPEC_DT_F32 = 0, SPEC_DT_BF16 = 1, SPEC_DT_INT4G128 = 2 } spec_dtype;

typedef enum {
  SPEC_ACCEPT_GREEDY = 0,
  SPEC_ACCEPT_STOCHASTIC = 1,
  /* commit the whole block (append / chunked prefill / resync):
     n_accepted = k, kv_len = L+k+1, next_token = argmax of row k */
  SPEC_ACCEPT_NONE = 2
} spec_accept_mode;

/* Model shape and capacity.  fp32 weights go with an fp32 KV cache, bf16 and
 * int4 weights with a bf16 cache.  Decoder-only LM: RMSNorm (gain), rotate-half
 * rotary embedding, causal attention with n_kv_heads groups (query head h
 * reads KV head h*n_kv_heads/n_q_heads), SwiGLU FFN.  n_experts > 0 selects
 * a MoE FFN: softmax router with bias over n_experts, each token keeps its
 * top_k experts by probability (weights = those probabilities, not
 * renormalized), plus n_shared always-on experts of width d_ff_expert
 * (S2-MoE section 2.1 and Table 1 give the family).  vocab is at most
 * 262144. */
typedef struct {
  int32_t n_layers, d_model, n_q_heads, n_kv_heads, head_dim, d_ff, vocab;
  int32_t n_experts, top_k, n_shared, d_ff_expert;
  int32_t weight_dtype;  /* spec_dtype of matmul weights (embedding: bf16 unless F32) */
  int32_t kv_dtype;      /* SPEC_DT_F32 or SPEC_DT_BF16 */
  float rope_theta, rms_eps;
  int32_t max_ctx;       /* KV capacity in positions */
  int32_t max_k;         /* largest k per step, 0..15 */
  int32_t gemm_k_split;  /* K elements per staged activation window of the weight-streaming
                            phases (multiple of 128, at most 2048); 0 = 2048.  Smaller windows
                            split every output over more partial sums (a test knob). */
  int32_t kv_page_seed;  /* 0: cache page i holds positions 64i .. 64i+63 (identity page
                            table); otherwise the logical pages are mapped to physical pages
                            by a permutation drawn from this seed (results are identical;
                            a test knob for the page indirection). */
  int32_t n_seqs;        /* sequences the handle holds (0 or 1: one), at most 64.  Each has
                            its own cache of max_ctx positions and committed length;
                            sequence 0 is the one the single-sequence calls work on, the
                            others are stepped by spec_verify_batch. */
  int32_t attn_group_pages; /* cache pages per attention work item: 0 = chosen per pass (3,
                            or 5 or 6 when fewer, longer items fit the grid in one round);
                            3, 5 or 6 = fixed (bf16 / int4 models; fp32 models take 3).
                            Results agree to rounding; a test knob. */
  int32_t reserved[4];   /* must be zero */
} spec_config;

/* Weight tensor kinds.  Matrices are row-major [K][N] with y = x . W. */
typedef enum {
  SPEC_T_EMBED = 0,       /* [vocab][d_model] */
  SPEC_T_FINAL_NORM = 1,  /* [d_model] fp32 gain */
  SPEC_T_LM_HEAD = 2,     /* [d_model][vocab] */
  SPEC_T_ATTN_NORM = 3,   /* [d_model] fp32 gain, per layer */
  SPEC_T_WQ = 4,          /* [d_model][n_q_heads*head_dim] */
  SPEC_T_WK = 5,          /* [d_model][n_kv_heads*head_dim] */
  SPEC_T_WV = 6,          /* [d_model][n_kv_heads*head_dim] */
  SPEC_T_WO = 7,          /* [n_q_heads*head_dim][d_model] */
  SPEC_T_FFN_NORM = 8,    /* [d_model] fp32 gain */
  SPEC_T_W_GATE = 9,      /* [d_model][d_ff] (expert: [d_model][d_ff_expert]) */
  SPEC_T_W_UP = 10,       /* same shape as gate */
  SPEC_T_W_DOWN = 11,     /* [d_ff][d_model] */
  SPEC_T_ROUTER = 12,     /* [d_model][n_experts], MoE only */
  SPEC_T_ROUTER_BIAS = 13 /* [n_experts] fp32, MoE only */
} spec_tensor_kind;

/* One host weight buffer.  Element types: SPEC_DT_F32 models use fp32 for
 * everything; otherwise the embedding is bf16 (uint16 bit patterns), gains
 * and the router bias are fp32, and matrices are bf16 (weight_dtype BF16)
 * or int4 (INT4G128): part 0 = packed nibbles uint8 [K/2][N] (even k in the
 * low nibble, two's complement), part 1 = fp16 scales [K/128][N], value =
 * nibble * scale.  expert = -1 except for MoE FFN matrices, where experts
 * 0..n_experts-1 are routed and n_experts..n_experts+n_shared-1 shared.
 * layer = -1 for embed / final norm / lm head. */
typedef struct {
  int32_t kind, layer, expert, part;
  const void* data;   /* host */
  uint64_t bytes;     /* must equal the size implied by the shape */
} spec_tensor;

typedef struct {
  int32_t n_accepted;  /* accepted drafts, 0..k */
  int32_t next_token;  /* new pending token (correction or bonus); its KV is not cached */
  int32_t kv_len;      /* committed cache length after the step = L + 1 + n_accepted */
} spec_step_result;

/* Checks a configuration without touching the GPU.  Returns SPEC_OK or
 * SPEC_EINVAL; a description of the first problem goes to `msg` (host
 * buffer of msg_len bytes, may be NULL). */
int spec_config_check(const spec_config* cfg, char* msg, int32_t msg_len);

/* Host-only diagnostic of the work split: builds the weight-streaming plan
 * a verifier of this configuration would use on a grid of n_wg workgroups
 * (one per compute unit, 1 <= n_wg <= 4096) and replays every workgroup's
 * walk over every weight matrix, checking each index it would form against
 * the buffer sizes it would allocate.  spec_verify_create runs the same
 * check for the device's compute-unit count.  Returns SPEC_OK, or
 * SPEC_EINVAL with the first problem in `msg` (host buffer, may be NULL). */
int spec_plan_check(const spec_config* cfg, int32_t n_wg, char* msg, int32_t msg_len);

/* Creates a verifier: copies every weight to device memory (re-tiled for
 * the GPU kernels), allocates KV pages for max_ctx positions and copies the
 * prompt cache in.  prompt_k / prompt_v: host [n_layers][n_kv_heads]
 * [prompt_len][head_dim] in the KV dtype (bf16 bit patterns or fp32), keys
 * already rotated; NULL when prompt_len == 0.  Every tensor the config
 * needs must appear exactly once in `tensors`.  Blocks until the copies are
 * done.  On success *out owns all device memory until spec_verify_destroy. */
int spec_verify_create(const spec_config* cfg, const spec_tensor* tensors, int32_t n_tensors,
                       const void* prompt_k, const void* prompt_v, int32_t prompt_len,
                       void* stream, spec_verify_t** out);

/* One verification step.
 *   tokens:  host int32 [k+1] = pending, d_1..d_k; every id in [0, vocab).
 *   k:       0..max_k (k = 0 is one autoregressive step).
 *   mode:    spec_accept_mode.
 *   q_dev:   device fp32 [k][vocab], q_dev[i-1] = draft distribution of d_i
 *            (STOCHASTIC only; else NULL).  Rows need not be normalized
 *            beyond what the draft produced; q(d_i) must be > 0.
 *   u_dev:   device fp32 [k+1] uniforms in [0,1): u_1..u_k for the tests,
 *            u_{k+1} for the final draw (STOCHASTIC only; else NULL).
 *   out:     host result.
 *   logits_dev: NULL or device fp32 [k+1][vocab] receiving the block's logits.
 * Requires kv_len + k + 1 <= max_ctx (else SPEC_ECAPACITY).  Enqueues the
 * pass on the handle's stream and returns after the 12-byte result has
 * reached the host (one stream synchronization).  No copy runs in either
 * direction: the ids are staged in pinned host memory of the handle, which
 * the kernels read through its device mapping, and the acceptance kernel
 * writes the result into pinned host memory of the handle.  The caller's
 * tokens array is copied before any work is enqueued.  The committed length
 * becomes out->kv_len; cache entries at or beyond it are dead. */
int spec_verify_step(spec_verify_t* h, const int32_t* tokens, int32_t k, int32_t mode,
                     const float* q_dev, const float* u_dev, spec_step_result* out,
                     float* logits_dev);

/* For callers that cannot allocate device memory while stepping (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same step as spec_verify_step, with the same arguments and results,
 * and it allocates nothing.  The pass kernel's split-K partial tiles and
 * their arrival tickets go to a fixed device scratch array of the library
 * (64 MiB, reserved on every device the library runs on until the process
 * ends) instead of the handle's workspace; the tickets are cleared by a
 * small kernel on the handle's stream before the pass.  SPEC_ECAPACITY if
 * this model's workspace (two banks of partials plus tickets) exceeds the
 * scratch.  All calls on one device share that device's scratch: calls
 * that overlap in time on one device (several handles or streams) race. */
int spec_verify_step_noalloc(spec_verify_t* h, const int32_t* tokens, int32_t k, int32_t mode,
                             const float* q_dev, const float* u_dev, spec_step_result* out,
                             float* logits_dev);

/* Verification of a token tree (S2-MoE section 4.1: drafts expanded as a
 * tree, each candidate verified in the same pass).  Row 0 is the pending
 * token (the root, parents[0] = -1); row i > 0 is a draft token whose parent
 * row parents[i] precedes it (0 <= parents[i] < i).  One target pass scores
 * every row: row i sits at position kv_len + depth(i) and attends to the
 * committed cache and to its ancestors (and itself) only, so its logits are
 * those the target writes after the path root..i.  Greedy acceptance walks
 * down from the root: while the argmax of the current row (lowest id on
 * ties) is the token of one of its children (the lowest-numbered such child
 * if several), that child is accepted and becomes current; next_token is
 * the argmax of the last current row (a correction, or the bonus token at a
 * leaf).  The cache keeps the pending token and the accepted path at
 * positions kv_len .. kv_len + n_accepted (their entries are moved there
 * from the rows' block slots); everything after is dead.
 *   tokens, parents: host int32 [m], 1 <= m <= max_k + 1.
 *   out:   n_accepted = length of the accepted path, next_token, kv_len =
 *          old kv_len + 1 + n_accepted.
 *   path:  host int32 [m] receiving the accepted rows in order (root
 *          excluded; n_accepted entries).
 *   logits_dev: NULL or device fp32 [m][vocab].
 * Errors as in spec_verify_step (SPEC_EINVAL for a malformed tree). */
int spec_verify_tree(spec_verify_t* h, const int32_t* tokens, const int32_t* parents, int32_t m,
                     spec_step_result* out, int32_t* path, float* logits_dev);

/* Several sequences verified in one pass: their blocks share one stream
 * of the weights (the essay's "What is not here" sets batching aside; the
 * rows of the pass are what batching spends).  Sequence i of the call is
 * seqs[i] (distinct, in [0, n_seqs)), with block tokens[r_i .. r_i + ks[i]]
 * = [pending_i, d_1 .. d_k] (r_i = sum of ks[j] + 1 over j < i); the
 * blocks' rows sum(ks[i] + 1) must not exceed max_k + 1.  Each row attends
 * to its own sequence's committed cache and earlier rows only, at that
 * sequence's positions, so every sequence gets the result a step of its
 * own block would give (up to summation order).
 *   mode: SPEC_ACCEPT_GREEDY or SPEC_ACCEPT_NONE (commit every row, e.g.
 *         to append a sequence's prompt).
 *   out:  host [n], one result per sequence in call order.
 *   logits_dev: NULL or device fp32 [sum(ks[i] + 1)][vocab], rows in call
 *         order.
 * Errors as in spec_verify_step, plus SPEC_EINVAL for a bad or repeated
 * sequence id; nothing changes on an error. */
int spec_verify_batch(spec_verify_t* h, int32_t n, const int32_t* seqs, const int32_t* tokens, const int32_t* ks,
                      int32_t mode, spec_step_result* out, float* logits_dev);

/* Debugging aid for the error paths (callers: tests): from now on, the
 * n-th device allocation the library makes (0 = the next one) fails as if
 * the device were out of memory; n < 0 switches this off.  Process-wide.
 * Returns the previous setting: the allocations that were still left
 * before the failure (-1 if none was armed or it has fired).  A failed
 * spec_verify_create frees everything it allocated and returns
 * SPEC_ENOMEM. */
int64_t spec_debug_fail_alloc(int64_t n);

/* Committed length of sequence seq (-1 for a bad handle or id). */
int32_t spec_seq_kv_len(const spec_verify_t* h, int32_t seq);

/* Commit / rollback for sequence seq (new_kv_len <= its length), as
 * spec_kv_commit_rollback does for sequence 0. */
int spec_seq_rollback(spec_verify_t* h, int32_t seq, int32_t new_kv_len);

/* Replaces sequence seq's cache with a prompt cache: host arrays laid out
 * as spec_verify_create's prompt_k / prompt_v, prompt_len <= max_ctx (else
 * SPEC_ECAPACITY); the sequence's committed length becomes prompt_len.
 * Allocates and frees a device staging buffer. */
int spec_seq_import(spec_verify_t* h, int32_t seq, const void* prompt_k, const void* prompt_v, int32_t prompt_len);

/* Self-speculative draft of a MoE target by expert sparsity (S2-MoE,
 * section 2.3 and section 5 "Draft configuration", Table 1: the draft is
 * the target itself with fewer routed experts per token; section 4.3: the
 * draft reads the target's cache, its own cache writes are temporary and
 * only verified tokens are kept).  Runs n autoregressive single-token passes
 * of this handle's model with draft_top_k routed experts per token (the
 * router's top draft_top_k by probability, weights the unrenormalized
 * probabilities, shared experts as in the target): pass i at position
 * kv_len + i takes token pending (i = 0) or d_i, attends to the committed
 * cache and the draft's own earlier entries, and d_{i+1} is the argmax of
 * its logits (lowest id on ties).  The passes are chained on the device (no
 * host round trip between tokens); the call returns after the n ids have
 * reached the host.
 *   pending:     the pending token (host), in [0, vocab).
 *   n:           1..16 draft tokens.
 *   draft_top_k: 1..top_k routed experts per draft token (MoE models only;
 *                SPEC_EINVAL for dense models).
 *   drafts:      host int32 [n] receiving d_1..d_n.
 *   logits_dev:  NULL or device fp32 [n][vocab] receiving each draft pass's
 *                logits (the draft distributions for stochastic acceptance
 *                are their softmax).
 *   route_dev:   NULL or device int32 [n][n_layers][draft_top_k] receiving
 *                the experts each draft pass routed its token to, per
 *                layer, in rank order (probability descending, lower id
 *                first on ties).
 * Requires kv_len + n <= max_ctx (else SPEC_ECAPACITY).  The committed
 * length does not change: the draft's cache entries at kv_len .. kv_len+n-1
 * are dead, and the verification step that follows overwrites them. */
int spec_draft(spec_verify_t* h, int32_t pending, int32_t n, int32_t draft_top_k, int32_t* drafts,
               float* logits_dev, int32_t* route_dev);

/* Routing-aware adaptive expansion of a draft tree (S2-MoE section 4.1;
 * host policy, no device work).  Candidate i (0 <= i < n) has a parent
 * parents[i] (-1: a child of the root, else an earlier candidate), the draft
 * probability p[i] in [0, 1] of its token given its parent, a drafting cost
 * c_draft[i] >= 0, and the experts verifying it would activate: ids
 * exp_ids[exp_offsets[i] .. exp_offsets[i+1]) (any non-negative ids, e.g.
 * layer * n_experts + expert; duplicates count once).  Its prefix
 * confidence P_i is the product of p along its path from the root, its
 * expected benefit P_i * t_ar (t_ar: one target decoding step), its cost
 * the number of its experts not yet active times t_exp (one expert's
 * verification cost) plus c_draft[i], and its utility U_i = benefit / cost
 * (infinite for a zero cost and positive benefit, 0 for a zero benefit).
 * Starting from the active set base_ids [n_base], each round admits the
 * candidate of highest U_i (lowest index on ties) among those whose parent
 * is the root or already admitted, provided U_i >= 1, and adds its experts
 * to the active set; it stops when the best U_i < 1 or max_nodes are
 * admitted.  Writes the admitted candidates in admission order to order
 * [max_nodes] and, when row_parents [max_nodes + 1] is not NULL, the parent
 * rows of the verification tree whose row 0 is the root and row r the
 * candidate admitted r-th (ready for spec_verify_tree).  Returns the
 * number admitted, or -1 for invalid arguments. */
int32_t spec_tree_expand(int32_t n, const int32_t* parents, const double* p, const int32_t* exp_offsets,
                         const int32_t* exp_ids, int32_t n_base, const int32_t* base_ids, double t_ar, double t_exp,
                         const double* c_draft, int32_t max_nodes, int32_t* order, int32_t* row_parents);

/* Lossy variant of spec_verify_step with reuse-aware expert gating (S2-MoE
 * section 4.2): in every MoE layer the block's rows steer their routing
 * towards shared experts, so the union of experts the pass loads shrinks.
 * For block rows b with gating logits l_b (router logits plus bias):
 * importance g_e = sum_b w_b l_{b,e} with w_b = conf_dev[b] (device fp32
 * [k+1], non-negative; NULL: all 1); the `cap` experts of largest importance
 * (ties to the lower id) are preferred; row b adds alpha * (l_b(1) -
 * l_b(top_k+1)) -- its first minus its (top_k+1)-th logit -- to the preferred
 * experts' logits, and top_k routing (selection and weights) runs on the
 * biased logits.  alpha = 0, or cap = n_experts (the same shift for every
 * expert of a row), gives the exact target.  The outputs are those of the
 * modified model: acceptance no longer reproduces the target's own decode.
 * MoE models with top_k < n_experts only; cap in [top_k, n_experts],
 * alpha >= 0.  union_dev / route_dev as in spec_verify_step_debug (may be
 * NULL).  Other arguments, results and errors as in spec_verify_step. */
int spec_verify_step_reuse(spec_verify_t* h, const int32_t* tokens, int32_t k, int32_t mode,
                           const float* q_dev, const float* u_dev, const float* conf_dev, int32_t cap,
                           float alpha, spec_step_result* out, float* logits_dev, int32_t* union_dev,
                           int32_t* route_dev);

/* Lookahead schedule for the next round (host policy, no device work): the
 * adaptive schedule the essay "LLM Inference: Speculative Decoding"
 * attributes to HuggingFace in "And the checking stops being free" -- raise
 * the lookahead by 2 after a round whose whole block was accepted, back off
 * otherwise.  Returns min(k + 2, max_k) if n_accepted == k, else
 * max(1, k - 1); -1 if k is outside [1, max_k], max_k < 1 or n_accepted is
 * outside [0, k]. */
int32_t spec_adaptive_k(int32_t k, int32_t n_accepted, int32_t max_k);

/* Truncates the committed cache to new_kv_len (0 <= new_kv_len <= kv_len):
 * entries at or beyond it become dead and are overwritten by later blocks.
 * Metadata only; no device work. */
int spec_kv_commit_rollback(spec_verify_t* h, int32_t new_kv_len);

/* Committed cache length, or -1 for a NULL handle. */
int32_t spec_kv_len(const spec_verify_t* h);

/* Last error message of the handle ("" if none); a static message for a
 * NULL handle.  Valid until the next call on the handle. */
const char* spec_last_error(const spec_verify_t* h);

/* Frees all device and pinned memory of the handle (synchronizes its
 * stream first).  NULL is allowed. */
void spec_verify_destroy(spec_verify_t* h);

/* ---------------------------------------------------------------------
 * Measurement and debugging hooks (same error conventions).
 * ------------------------------------------------------------------- */

/* Kernel classes timed by the profiling mode. */
/* The pass runs as one persistent kernel made of phases separated by grid
 * barriers; classes name the phases, plus the whole pass kernel and the
 * acceptance kernel. */
typedef enum {
  SPEC_K_EMBED = 0, SPEC_K_QKV = 1, SPEC_K_ATTN = 2, SPEC_K_ATTN_COMBINE = 3,
  SPEC_K_O = 4, SPEC_K_GATEUP = 5, SPEC_K_DOWN = 6, SPEC_K_ROUTER = 7,
  SPEC_K_ROUTE = 8, SPEC_K_EXPERT_GATEUP = 9, SPEC_K_EXPERT_DOWN = 10,
  SPEC_K_MOE_COMBINE = 11, SPEC_K_LMHEAD = 12, SPEC_K_ACCEPT = 13,
  SPEC_K_PASS = 14,
  SPEC_K_NCLASSES = 15
} spec_kernel_class;

/* on = 1: every following step times the pass kernel and the acceptance
 * kernel with HIP events recorded on the handle's stream, and each phase of
 * the pass with device wall-clock stamps taken by workgroup 0 after every
 * grid barrier (a phase's time includes its barrier); it accumulates per-
 * class counts, elapsed milliseconds and algorithmic bytes (weights, KV and
 * activations each phase must move).  SPEC_K_ATTN_COMBINE is the merge of
 * the attention groups (no algorithmic bytes of its own: its partials are
 * an artefact of the split); SPEC_K_ROUTE stays zero (routing runs inside
 * SPEC_K_EXPERT_GATEUP).  on = 2: only the HIP events around the pass and
 * acceptance kernels (no per-phase stamps, so the pass runs exactly as
 * unprofiled).  In both modes SPEC_K_PASS accumulates the bytes of
 * spec_pass_bytes for each step (MoE: with the experts the step loaded).
 * on = 0 turns profiling off.  Enabling resets the counters. */
int spec_profile_enable(spec_verify_t* h, int32_t on);

/* Reads the accumulated per-class figures since the last enable.
 * launches / ms / bytes: host arrays of SPEC_K_NCLASSES entries (any may
 * be NULL). */
int spec_profile_read(const spec_verify_t* h, int64_t* launches, double* ms, double* bytes);

/* Per-workgroup split of each class's phases while profiling is on (device
 * wall-clock stamps taken by every workgroup), summed over launches, in ms.
 * For class c, out[8*c + j] is the mean over workgroups and out[8*c + 4 + j]
 * the maximum of: j = 0 activation staging, 1 weight stream, 2 flush
 * (split-K tickets, reductions, epilogues), 3 the whole work.  Attention:
 * j = 0 operand loads and query set-up, 1 the position walk, 2 partials
 * and merges (of a workgroup's last item).  Other phases that stream no
 * weights: their whole work in j = 2.  A phase's time
 * (spec_profile_read) minus the maximum whole work is its grid-barrier
 * wait.  out: host array of 8 * SPEC_K_NCLASSES doubles. */
int spec_profile_detail(const spec_verify_t* h, double* out);

/* The per-workgroup stamps of the last profiled step (device wall clock,
 * 100 MHz on MI355X): out[(phase * n_wg + wg) * 4 + j] for j = 0 start,
 * 1 after staging, 2 after the stream, 3 end of work (same meaning as in
 * spec_profile_detail; phases in program order).  *count (host, may be
 * NULL) receives phases * n_wg * 4; out (host array of n uint64) may be
 * NULL to ask for the count only; SPEC_ECAPACITY if n is smaller. */
int spec_profile_raw(const spec_verify_t* h, uint64_t* out, int64_t n, int64_t* count);

/* Like spec_verify_step, and additionally copies the residual stream after
 * every layer into trace_dev (device fp32 [n_layers][k+1][d_model], may be
 * NULL) and, for MoE models, the number of routed experts loaded by each
 * layer into union_dev (device int32 [n_layers], may be NULL) and the
 * experts each block row selected into route_dev (device int32
 * [n_layers][k+1][top_k], in rank order: probability descending, lower
 * expert id first on ties; may be NULL; ignored for dense models). */
int spec_verify_step_debug(spec_verify_t* h, const int32_t* tokens, int32_t k, int32_t mode,
                           const float* q_dev, const float* u_dev, spec_step_result* out,
                           float* logits_dev, float* trace_dev, int32_t* union_dev,
                           int32_t* route_dev);

/* Debugging aid for the rollback rule (essay "The loop", step 5: entries
 * of rejected drafts must never influence later steps): overwrites every
 * cache entry at positions kv_len .. max_ctx-1 (keys and values of every
 * layer and KV head) with NaN, on the handle's stream, and waits for it.
 * A later step that read any of them would produce NaN logits. */
int spec_kv_poison_dead(spec_verify_t* h);

/* Algorithmic bytes one verification pass must move for this handle's
 * model at committed length L with block size k+1 and (MoE) `experts_loaded`
 * routed experts summed over layers: every weight once, live KV once, new
 * KV rows, logits (and the draft distributions for stochastic mode). */
double spec_pass_bytes(const spec_verify_t* h, int32_t L, int32_t k, int32_t mode,
                       int64_t experts_loaded);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
