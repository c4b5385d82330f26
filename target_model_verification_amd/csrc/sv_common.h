// Shared declarations of the HIP device code and the host runtime.
// Device code targets gfx950 (CDNA4, wave64) only.
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace sv {

// ---------------------------------------------------------------- geometry
// The verification pass runs as one persistent cooperative kernel: one
// workgroup of kWaves waves per compute unit (one per SIMD, so a wave may
// hold up to 512 registers), each wave streaming its weights in batches of
// kRing 1 KB fragments (128 KB in flight per CU).  Work of every weight-
// streaming phase is split over the workgroups in equal runs of
// (supergroup, K chunk) units ("stream-K"); a supergroup is kWaves output
// units, one per wave, so the kWaves waves of a workgroup read one
// contiguous block of kWaves x 1 KB fragments per K chunk.
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kTileN = 16;            // output columns per MFMA tile
constexpr int kChunkK = 32;           // k per bf16 / fp32 fragment
constexpr int kGroupK = 128;          // int4: k per fragment (= scale group)
constexpr int kMaxRows = 16;          // block rows (k+1) per pass
constexpr int kPage = 64;             // KV page (positions); attention sub-chunk
constexpr int kGroupPages = 3;        // pages per attention work item: the smallest group size
constexpr int kGroupPos = kPage * kGroupPages;
constexpr int kMaxGroupPages = 6;     // the largest (a pass takes 3, 5 or 6, see group_pages)
constexpr int kMaxAttnRows = 128;     // (k+1) * (n_q_heads / n_kv_heads) per KV head
constexpr int kAttnRT = kMaxAttnRows / 16;   // attention row tiles per KV head at most
constexpr long long kInlineMergeElems = 16384;   // rows * head_dim * groups merged by one workgroup
constexpr int kRing = 32;             // weight fragments per prefetch batch (per wave)
constexpr int kAWindowBytes = 128 * 1024;  // LDS bytes of the staged A window (2048 k of hi/lo rows)
constexpr int kMaxLds = 160 * 1024;

enum WFmt : int { W_BF16 = 0, W_INT4 = 1, W_F32 = 2 };

// One weight matrix, or a stack of expert matrices of one shape, in the
// streaming layout: fragment (expert, supergroup, chunk, wave, half) at
// ((((e * n_sg + sg) * nkc + c) * kWaves + w) * tpu + half) KB, where the
// output unit of (sg, w) is sg * kWaves + w and a unit is one 16-column
// tile (tpu = 1) or a gate tile and its up tile (tpu = 2).
struct Mat {
  const void* w;          // fragments (bf16, int4, or the bf16 "hi" part of fp32)
  const void* w2;         // fp32: "lo" fragments; int4: fp16 scales [..][16]; else null
  long long w_stride;     // bytes per expert (w)
  long long w2_stride;    // bytes per expert (w2)
  int n_units;            // units per expert
  int n_sg;               // supergroups per expert = ceil(n_units / kWaves)
  int nkc;                // fragments along K (32 k each; 128 k for int4)
  int win;                // chunks per staged A window
  int n_win;              // ceil(nkc / win)
  int K, N;               // logical shape (N: output columns; SwiGLU: activation columns)
  int max_seg;            // workspace slots per unit block (split-K partials)
  int U;                  // chunks per weight batch of one wave (a piece of the work split)
};

// One phase of the pass program (a grid barrier separates consecutive
// phases).  GEMM phases stream M; the other fields are what the phase kind
// reads or writes.
enum PhKind : int {
  PH_EMBED = 0,        // embedding gather + first norm's A operand
  PH_STORE = 1,        // Y = (A W) [* row scale] -> out (QKV, router, expert down)
  PH_RESID = 2,        // x += A W -> next A operand (x * gain), sum-of-squares
  PH_SWIGLU = 3,       // silu(s * A Wg) * (s * A Wu) -> next A operand
  PH_LOGITS = 4,       // logits = s * A W and per-tile (max, argmax, sum-exp)
  PH_ATTN = 5,         // causal attention over the paged cache -> per-group partials
  PH_ROUTE_SWIGLU = 6, // MoE routing of the block, then SWIGLU over the union
  PH_COMBINE = 7,      // MoE weighted combine -> x, next A operand
  PH_ATTN_MERGE = 8,   // merge of the attention partials -> A operand of O
  PH_QKV = 9           // Q/K/V projection: rotary, queries -> fragments, keys / values -> cache
};

struct Phase {
  int kind, layer;
  int slot_mode;          // 0 dense; 1 MoE slots sharing A; 2 MoE slot-major (A per slot)
  int trace;              // RESID / COMBINE: this phase finishes the layer's residual
  Mat M;
  const uint4* a; long long a_slot;
  float* out; int ldo; long long out_slot; int scale;
  const float* gain;      // RESID / COMBINE: gain of the next norm
  uint4* a_out; long long a_out_slot;
  const float* bias;      // ROUTE: router bias
  void* kv;               // QKV / ATTN: the layer's KV pages
  Mat Mr;                 // ROUTE: router matrix computed in the phase (Mr.w null: read the router phase's logits)
  int next_gemm;          // index of the next weight-streaming phase (n_prog if none)
  int dep;                // inputs: 0 after a grid barrier; else waits on this layer's
                          // ready counters (kDepHeads / kDepOWin)
  int notify;             // outputs announced on ready counters (kDepHeads)
  const float* ss_in;     // sum-of-squares partials of the input's norm (row scales)
  float* ss_out;          // EMBED / RESID / COMBINE: partials of the next norm
  float* ws;              // split-K workspace bank (GEMM phases; a phase that may
  unsigned* tickets;      // overlap its predecessor's reductions uses the other bank)
  int ws_bank;            // which of the two banks (0 / 1) ws and tickets are
};
// Ready counters per layer (64-bit, monotonic: pass e waits for e times the
// expected count): KV heads' query / key / value blocks, and windows of the
// O projection's input (merged heads).  Edges whose consumers depend on
// many producers (a normalised row, a gate/up window) keep grid barriers.
enum DepKind : int { kDepNone = 0, kDepHeads = 1, kDepOWin = 2 };
constexpr int kReadyStride = 512;   // counters per layer: [0,256) KV heads, [256,512) O windows
constexpr int kRdyOWin = 256;

// Everything one pass needs; passed by value to the pass kernel.
struct PassP {
  int m, L, n_layers, d, Hq, Hkv, D, V, G, E, top_k, n_shared, F;
  int n_groups;              // attention position groups covering [0, L+m)
  int n_ss;                  // d / 16: sum-of-squares partials per row
  int lds_bytes;             // dynamic LDS of the launch (control area at its end)
  float eps, inv_d, attn_scale;
  const Phase* prog; int n_prog;   // device array: the phases of one pass
  const void* embed;         // [V][d] bf16 bits (fp32 for fp32 models)
  const float* gain0;        // attention-norm gain of layer 0
  const int* tokens;         // [m]
  const int* page_table;
  const float* rope_cs;      // [max_ctx][D/2][2]
  // activations (A operands and norm partials are per phase, in the program)
  float* x; int ldx;         // residual stream [16][ldx]
  float* logits; int ldl;    // [16][ldl]
  float* st_max; float* st_sum; int* st_idx; int n_stat;   // per 16-column tile of the LM head
  float* pm; float* ps; float* pacc;                      // attention partials
  float* rlog; int ldr;      // MoE router logits [16][ldr]
  float* ey; long long ey_slot; int ldy;                  // expert outputs [slot][16][ldy]
  int* route;                // MoE routing record (route_words)
  unsigned* attn_tickets;     // [Hkv] groups finished per KV head (inline merge)
  unsigned long long* ready;  // [n_layers][kReadyStride] ready counters
  unsigned long long epoch;   // passes run by this handle, this one included
  int o_wcols;                // input columns per window of the O projection
  int qf_rt;                  // row tiles per KV head in the query fragments
  int attn_inline;           // 1: attention's last arrivers merge, the merge phase is skipped
  // split-K banks replacing the program's own (null: use the program's):
  // bank b at ws_alt + b * ws_bank_floats, tickets_alt + b * tickets_bank
  float* ws_alt; unsigned* tickets_alt; long long ws_bank_floats, tickets_bank;
  // grid barrier
  unsigned long long* bar; unsigned long long bar_base;
  int* err;                  // set to 1 by a grid-barrier wait that ran out
  // debug / profiling (nullable)
  float* trace;              // [n_layers][m][d]
  int* union_hist;           // [n_layers]
  int* route_hist;           // [n_layers][m][top_k] experts selected by each row, in rank order
  // reuse-aware gating (lossy; reuse_cap 0 = off): per layer the cap experts
  // with the largest confidence-weighted sum of the block's gating logits
  // get a per-row bias reuse_alpha * (top-1 logit - (top_k+1)-th logit)
  int reuse_cap; float reuse_alpha;
  const float* reuse_w;      // [m] row confidences (null: 1)
  // Per-row placement (each null: one sequence, row j at cache slot L + j,
  // rotary position L + j, causal over slots 0 .. L + j):
  //   row_slot[j]  cache slot of row j's new key and value;
  //   row_rope[j]  its rotary position;
  //   row_lo/hi[j] the slots it attends to, lo .. hi (several sequences in
  //                one slot space: each row sees its own sequence only);
  //   page_live[p] live slots of page p (the rest are another sequence's
  //                padding: their keys and values are never used).
  // A token tree: rows attend to the committed cache and to the block rows
  // whose bits are set in tree_anc[j] (ancestors and itself).
  const int* row_slot;
  const int* row_rope;
  const int* row_lo;
  const int* row_hi;
  const int* page_live;
  const unsigned* tree_anc;
  int T;                     // slots the attention reads: L + m (one sequence) or the batch's extent
  int group_pages;           // pages per attention group (3, 5 or 6; the host picks it per pass)
  unsigned long long* stamps;   // [n_phases + 1] wall clock at phase ends (workgroup 0)
  unsigned long long* wstamps;  // [n_phases][n_wg][4] per-workgroup phase stamps (nullable)
};

struct AcceptParams {
  int k, V, L, mode, n_stat;
  int n_seq;                 // several sequences (mode kAcceptBatch*): their count
  const int* seq_info;       // [n_seq][3]: first row, k, committed length
  const int* tokens;
  const int* parents;   // token tree: parent row of every row (mode kAcceptTree)
  int* path;            // token tree: accepted rows, root excluded
  const float* st_max; const float* st_sum; const int* st_idx;
  const float* logits; int ldl;
  const float* q; const float* u;
  int* result;          // [3]
  float* acc_ws;        // kAccFloats words, tickets zero at first use
  int* result_mirror;   // single-sequence step: result[0..3] also here (pinned host memory), else null
};

// Acceptance workspace (words): the decision of the stochastic tests (row of
// the draw, residual flag, that row's max logit and softmax sum), the arrival
// tickets of the statistics grid and of the draw grid, then per 64-id tile
// the residual weight sums and the plain p weight sums, then the row
// statistics' per-chunk partials [16 rows][kAccMaxChunks][3].
constexpr int kAccTiles = 4 * 1024;      // 64-id tiles: vocabularies up to 262144 ids
constexpr int kAccMaxChunks = 4;         // statistics chunks per row (4096 partials each)
constexpr int kDrawRow = 0, kDrawResid = 1, kDrawM = 2, kDrawS = 3, kDrawTicket = 4, kAccTicket = 5;
constexpr int kDrawHead = 16;
constexpr int kAccPart = kDrawHead + 2 * kAccTiles;
constexpr int kAccFloats = kAccPart + 16 * kAccMaxChunks * 3;

// Acceptance kernel mode for a token tree (greedy; the C ABI's modes are
// 0..2).
constexpr int kAcceptTree = 3;
// Several sequences in one block: greedy per sequence, or every row
// committed (results [n_seq][4]: n_accepted, next token, new length).
constexpr int kAcceptBatchGreedy = 4;
constexpr int kAcceptBatchNone = 5;

// MoE routing record in global memory (int32 words):
//   [0] union size U; [1 .. E] union list (ascending expert id);
//   [1+E .. 2E] slot of each expert (-1 if unused);
//   [1+2E ..) sel [16][top_k] expert ids; then selw [16][top_k] fp32 bits.
__host__ __device__ inline int route_words(int E, int top_k) { return 1 + 2 * E + 2 * 16 * top_k; }

// ---------------------------------------------------------------- launchers
// One pass executes n_prog - 1 grid barriers (the host advances the barrier
// generation by that much per launch).  fp32 weights imply an fp32 KV cache;
// bf16 / int4 weights a bf16 cache.
hipError_t launch_pass(int wfmt, bool moe, const PassP& p, int n_wg, size_t lds, hipStream_t s);
hipError_t pass_occupancy(int wfmt, bool moe, size_t lds, int* blocks_per_cu);
// split units one workgroup may flush per phase (control-area capacity)
constexpr int kMaxPending = 512;
hipError_t launch_accept(const AcceptParams& p, hipStream_t s);
// Fixed device scratch (file-scope array) for steps that allocate nothing:
// its device address on `device` (which must be current); looked up once per
// device.
constexpr size_t kScratchBytes = size_t(64) << 20;
hipError_t scratch_setup(int device, void** out);
hipError_t launch_zero_u32(unsigned* p, long long n, hipStream_t s);
hipError_t launch_retile(int wfmt, const void* src, const void* src_scales, int K, int N, void* dst,
                         void* dst2, int nkc, int tpu, int tile_off, int tile_stride, int pair_dim, hipStream_t s);
hipError_t launch_kv_import(int kv_f32, const void* src, int P, int Hkv, int D, void* layer_base,
                            const int* page_table, hipStream_t s);
hipError_t launch_kv_poison(int kv_f32, void* base, long long layer_elems, int n_layers, int Hkv, int D,
                            const int* page_table, int from, int to, hipStream_t s);
// After a token-tree step: moves the cache entries of the accepted rows
// (path, count in result[0]) from slots L + path[j] to L + 1 + j.
hipError_t launch_tree_commit(int kv_f32, void* base, long long layer_elems, int n_layers, int Hkv, int D,
                              const int* page_table, int L, const int* result, const int* path, hipStream_t s);


// ------------------------------------------------------------ LDS plan of the pass
// [0, kAWindowBytes): the staged A window (GEMM phases) / attention working
// set; [kAWindowBytes, +1 KB) int4 row sums; then the routing scratch (MoE);
// a control area at the end.
constexpr int kCtlBytes = 4096;
constexpr int kPsStride = kPage + 4;         // floats per attention score row in LDS (two-pass path)

// LDS of the attention phase: Q fragments [RT][D/32][hi|lo][64 lanes],
// scores / probabilities [RT*16][kPsStride], running max / sum / rescale.
// (two-pass path; the one-row-tile path needs 16 rows of a whole group of
// the largest size + 4)
__host__ __device__ constexpr size_t attn_lds_bytes(int rt, int D) {
  return (size_t)rt * (D / 32) * 2 * 1024 + (size_t)rt * 16 * kPsStride * 4 + (size_t)3 * rt * 16 * 4 +
         (size_t)16 * (kPage * kMaxGroupPages + 4) * 4;
}

// LDS of routing, after the A window (which stays staged for the routed
// gate/up phase, whose A operand is the router's): used / slot of each
// expert [256], sel [16][16], selw [16][16], reuse-gating scratch, then one
// [16][E] float area that holds the block's router logits (when computed in
// the phase), then the reuse-gating logits, then the probabilities (rows
// padded to a multiple of 4).
constexpr int kRouteBase = kAWindowBytes + 1024;   // after the int4 row sums
constexpr int kRouteZl = kRouteBase + 6 * 1024;
constexpr int kRouteBytes = 6 * 1024 + 16 * 256 * 4;
// The expert phases' fixed-order split keeps each segment's running chain
// (kWaves waves x up to 2 tiles x 64 lanes x 16 bytes) in the routing
// scratch, which is free once the union is built.
constexpr int kChainBase = kRouteBase;
static_assert(kWaves * 2 * 64 * 16 <= kRouteBytes, "chain area exceeds the routing scratch");

inline size_t pass_lds_bytes(int wfmt, int max_rows_attn, int D) {
  const size_t gemm = (size_t)kAWindowBytes + (wfmt == W_INT4 ? 16 * 16 * 4 : 0);   // + int4 row sums
  const size_t attn = attn_lds_bytes((max_rows_attn + 15) / 16, D);
  const size_t route = (size_t)kRouteBase + kRouteBytes;   // after the A window
  size_t b = gemm > attn ? gemm : attn;
  if (route > b) b = route;
  return b + kCtlBytes;
}

}  // namespace sv
