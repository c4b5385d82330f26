// Host runtime of the verification-step library: configuration checks,
// weight upload into the streaming layout, the paged KV cache, the phase
// program of one pass, the cooperative launch, acceptance readback and KV
// commit / rollback.
#include "../../include/spec_verify.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <iterator>
#include <map>
#include <string>
#include <tuple>
#include <vector>

#include "sv_common.h"
#include "stream_plan.h"

using namespace sv;

namespace {

inline int rup(int a, int b) { return ((a + b - 1) / b) * b; }
inline int cdiv(int a, int b) { return (a + b - 1) / b; }

struct HostMat {
  Mat m{};
  int tpu = 1, n_stack = 1;
  double alg_bytes = 0;   // logical weight bytes per expert
};

struct HostLayer {
  HostMat qkv, o, gateup, down, router, ex_gateup, ex_down;
  float* attn_norm = nullptr;
  float* ffn_norm = nullptr;
  float* router_bias = nullptr;
  void* kv = nullptr;
};

}  // namespace

struct spec_verify {
  spec_config cfg{};
  hipStream_t stream = nullptr;
  int device = 0;
  int wfmt = W_BF16;
  int n_wg = 0;                 // workgroups of the pass (one per CU)
  size_t lds = 0;
  double wall_khz = 0;          // device wall clock rate (kHz)
  std::vector<HostLayer> layers;
  void* embed = nullptr;
  HostMat lm_head;
  float* final_norm = nullptr;
  // KV cache
  void* kv = nullptr;
  long long kv_layer_elems = 0;
  int n_pages = 0;              // all sequences' pages
  int* page_table = nullptr;    // [n_seqs][pps]: sequence s's logical page i -> physical page
  std::vector<int> pt_host;     // host copy of the page table
  int n_seqs = 1, pps = 0;      // sequences, pages per sequence
  std::vector<int> seq_len;     // committed lengths of sequences 1.. (sequence 0: kv_len)
  int* batch_dev = nullptr;     // several sequences: row placement, sequence records, virtual page table
  int* batch_host = nullptr;    // pinned staging of batch_dev
  int* batch_res = nullptr;     // [kMaxRows][4] per-sequence outcomes (device)
  int* batch_res_host = nullptr;
  float* rope_cs = nullptr;
  // activations / scratch
  int ldx = 0, ldl = 0, n_ss = 0, n_stat = 0, ldr = 0;
  float *x = nullptr, *ss = nullptr, *logits = nullptr;
  uint4* qf = nullptr;     // attention query fragments
  uint4 *a_norm = nullptr, *a_o = nullptr, *a_act = nullptr;
  long long a_act_slot = 0, a_act_layer = 0;   // uint4 per slot / per layer
  long long a_norm_site = 0, ss_site = 0;       // uint4 / floats per norm site
  float *st_max = nullptr, *st_sum = nullptr;
  int* st_idx = nullptr;
  float *pm = nullptr, *ps = nullptr, *pacc = nullptr;
  float *rlog = nullptr, *ey = nullptr;
  long long ey_slot = 0;
  int* route = nullptr;
  float* ws = nullptr;
  unsigned* tickets = nullptr;
  size_t ws_bank_floats = 0, tickets_bank = 0;   // per split-K bank
  void* scratch = nullptr;      // the fixed device scratch of this device (no-alloc steps)
  bool scratch_fits = false;    // both split-K banks and their tickets fit in it
  unsigned* attn_tickets = nullptr;
  unsigned long long* bar = nullptr;
  unsigned long long bar_gen = 0;
  int n_barriers_inline = 0, n_barriers_merge = 0;   // grid barriers per pass
  unsigned long long epoch = 0;        // passes run (ready counters count up by pass)
  unsigned long long* ready = nullptr; // [n_layers][kReadyStride]
  int qf_rt = 1, o_wcols = 0;
  long long qf_layer = 0, a_o_layer = 0;   // uint4 per layer
  int* tokens_dev = nullptr;
  int* result_dev = nullptr;
  float* acc_ws = nullptr;      // acceptance: tickets, partial statistics, draw tile sums
  int* tokens_host = nullptr;   // pinned
  int* tokens_mapped = nullptr;   // device view of tokens_host (the step's kernels read the ids there), or null
  int* result_host = nullptr;   // pinned
  int* result_mirror = nullptr;   // device view of result_host (the step's acceptance writes it), or null
  int* draft_res = nullptr;     // self-speculative draft: [kMaxRows][4] acceptance records (device)
  int* tree_dev = nullptr;      // token tree: parents [16], depths [16], ancestor masks [16], path [16]
  int* tree_host = nullptr;     // pinned staging of the tree arrays and the returned path
  int* draft_host = nullptr;    // pinned copy of draft_res and the error flag
  // the pass program
  Phase* prog = nullptr;
  int n_prog = 0;
  std::vector<int> prog_cls;    // profiling class of each phase
  std::vector<int> prog_layer;  // layer of each phase (-1: none)
  std::vector<int> prog_kind;   // PhKind of each phase
  std::vector<double> prog_bytes_fixed;   // weight bytes of each phase (MoE experts: per expert)
  std::vector<void*> allocs;
  // state
  int kv_len = 0;
  bool broken = false;
  std::string err;
  // profiling (0 off, 1 events + per-phase stamps, 2 events only)
  int prof_mode = 0;
  bool profiling = false;
  hipEvent_t ev[4] = {nullptr, nullptr, nullptr, nullptr};
  unsigned long long* stamps_dev = nullptr;
  std::vector<unsigned long long> stamps_host;
  unsigned long long* wstamps_dev = nullptr;    // [n_prog][n_wg][4]
  std::vector<unsigned long long> wstamps_host;
  std::vector<int> union_host;                  // MoE: union sizes of the last profiled step
  double prof_detail[SPEC_K_NCLASSES][8] = {};
  int* union_dev_prof = nullptr;
  int64_t prof_launches[SPEC_K_NCLASSES] = {};
  double prof_ms[SPEC_K_NCLASSES] = {};
  double prof_bytes[SPEC_K_NCLASSES] = {};
};

namespace {

const char* kNullMsg = "null handle";

// Several sequences in one pass, device words: row slots, rotary positions,
// slot intervals [4][kMaxRows], sequence records [kMaxRows][3], then the
// virtual page table and the live slots of each virtual page.
constexpr int kBatchSlot = 0, kBatchRope = kMaxRows, kBatchLo = 2 * kMaxRows, kBatchHi = 3 * kMaxRows,
              kBatchSeq = 4 * kMaxRows, kBatchPages = 7 * kMaxRows;
size_t batch_words(const spec_verify* h) { return kBatchPages + 2 * (size_t)h->n_pages; }

int fail(spec_verify* h, int code, const std::string& msg) {
  if (h) h->err = msg;
  return code;
}

#define HIPCHK(expr)                                                              \
  do {                                                                            \
    hipError_t e_ = (expr);                                                       \
    if (e_ != hipSuccess) {                                                       \
      h->err = std::string(#expr) + ": " + hipGetErrorString(e_);                 \
      return SPEC_EHIP;                                                           \
    }                                                                             \
  } while (0)

// Debugging aid (spec_debug_fail_alloc): the number of device allocations
// left before one fails as if the device were out of memory (-1: off).
std::atomic<long long> g_fail_alloc{-1};

int dalloc(spec_verify* h, void** p, size_t bytes) {
  if (bytes == 0) bytes = 16;
  for (long long n = g_fail_alloc.load(); n >= 0;) {
    if (g_fail_alloc.compare_exchange_weak(n, n - 1)) {
      if (n == 0) {
        *p = nullptr;
        h->err = "hipMalloc(" + std::to_string(bytes) + "): injected failure";
        return SPEC_ENOMEM;
      }
      break;
    }
  }
  hipError_t e = hipMalloc(p, bytes);
  if (e != hipSuccess) {
    *p = nullptr;
    h->err = "hipMalloc(" + std::to_string(bytes) + "): " + hipGetErrorString(e);
    return e == hipErrorOutOfMemory ? SPEC_ENOMEM : SPEC_EHIP;
  }
  h->allocs.push_back(*p);
  return SPEC_OK;
}

template <typename T>
int dalloc_t(spec_verify* h, T** p, size_t count) {
  void* q = nullptr;
  int rc = dalloc(h, &q, count * sizeof(T));
  *p = static_cast<T*>(q);
  return rc;
}

// zero-filled allocation (at least 16 bytes, all of them zeroed)
template <typename T>
int dalloc_z(spec_verify* h, T** p, size_t count) {
  const size_t bytes = std::max<size_t>(count * sizeof(T), 16);
  void* q = nullptr;
  int rc = dalloc(h, &q, bytes);
  *p = static_cast<T*>(q);
  if (rc) return rc;
  hipError_t e = hipMemsetAsync(*p, 0, bytes, h->stream);
  if (e != hipSuccess) return fail(h, SPEC_EHIP, std::string("memset: ") + hipGetErrorString(e));
  return SPEC_OK;
}

double elem_bytes(int dt) { return dt == SPEC_DT_F32 ? 4.0 : dt == SPEC_DT_BF16 ? 2.0 : 0.5; }

int max_rows_attn(const spec_config* c) { return (c->max_k + 1) * (c->n_q_heads / c->n_kv_heads); }

bool check_cfg(const spec_config* c, std::string& msg) {
  auto bad = [&](const char* m) {
    msg = m;
    return false;
  };
  if (!c) return bad("null config");
  if (c->n_layers < 1 || c->d_model < 1 || c->n_q_heads < 1 || c->n_kv_heads < 1 || c->vocab < 2)
    return bad("n_layers, d_model, heads must be >= 1 and vocab >= 2");
  if (c->vocab > 262144) return bad("vocab must be <= 262144 (on-device acceptance works in 4096 tiles of 64 ids)");
  if (c->n_q_heads % c->n_kv_heads != 0) return bad("n_q_heads must be a multiple of n_kv_heads");
  if (c->n_kv_heads > 256) return bad("n_kv_heads must be at most 256");
  if (c->head_dim != 64 && c->head_dim != 128) return bad("head_dim must be 64 or 128");
  if (c->weight_dtype < SPEC_DT_F32 || c->weight_dtype > SPEC_DT_INT4G128) return bad("bad weight_dtype");
  if (c->kv_dtype != SPEC_DT_F32 && c->kv_dtype != SPEC_DT_BF16) return bad("kv_dtype must be F32 or BF16");
  if ((c->weight_dtype == SPEC_DT_F32) != (c->kv_dtype == SPEC_DT_F32))
    return bad("fp32 weights need an fp32 KV cache and bf16/int4 weights a bf16 cache");
  if (c->max_k < 0 || c->max_k > 15) return bad("max_k must be in [0, 15]");
  if (c->max_ctx < 1 || c->max_ctx > (1 << 22)) return bad("max_ctx out of range");
  if (!(c->rope_theta > 0.f) || !(c->rms_eps >= 0.f)) return bad("rope_theta must be > 0 and rms_eps >= 0");
  if (c->gemm_k_split < 0 || c->gemm_k_split % 128 != 0 || c->gemm_k_split > 2048)
    return bad("gemm_k_split must be a multiple of 128 in [0, 2048]");
  for (int i = 0; i < 4; ++i)
    if (c->reserved[i] != 0) return bad("reserved fields must be zero");
  if (c->attn_group_pages != 0 && c->attn_group_pages != 3 && c->attn_group_pages != 5 && c->attn_group_pages != 6)
    return bad("attn_group_pages must be 0, 3, 5 or 6");
  if (c->weight_dtype == SPEC_DT_F32 && c->attn_group_pages > 3) return bad("fp32 models take 3-page groups");
  if (c->n_seqs < 0 || c->n_seqs > 64) return bad("n_seqs must be in [0, 64]");
  const bool moe = c->n_experts > 0;
  if (moe) {
    if (c->n_experts > 256) return bad("n_experts must be <= 256");
    if (c->top_k < 1 || c->top_k > c->n_experts || c->top_k > 16) return bad("top_k must be in [1, min(16, n_experts)]");
    if (c->n_shared < 0 || c->n_shared > 8) return bad("n_shared must be in [0, 8]");
    if (c->d_ff_expert < 1) return bad("d_ff_expert must be >= 1");
  } else {
    if (c->n_experts < 0) return bad("n_experts must be >= 0");
    if (c->d_ff < 1) return bad("d_ff must be >= 1");
  }
  if (c->weight_dtype == SPEC_DT_INT4G128) {
    const int F = moe ? c->d_ff_expert : c->d_ff;
    if (c->d_model % 128 || (c->n_q_heads * c->head_dim) % 128 || F % 128)
      return bad("int4 weights need d_model, n_q_heads*head_dim and the FFN width divisible by 128");
  }
  if (c->d_model % 16) return bad("d_model must be a multiple of 16");
  if (max_rows_attn(c) > kMaxAttnRows)
    return bad("(max_k+1) * (n_q_heads/n_kv_heads) must be at most 128 (attention rows per KV head)");
  const size_t lds = pass_lds_bytes(W_BF16, max_rows_attn(c), c->head_dim);
  if (lds > (size_t)kMaxLds) return bad("the pass does not fit in LDS for this configuration");
  return true;
}

// ------------------------------------------------------------------ stream-K plan
// Geometry of every weight-streaming phase, the split-K workspace and
// ticket counts they need on a grid of G workgroups, and a host replay of
// every workgroup's walk (check_gemm_walk) before anything is allocated.
struct PassPlan {
  GemmShape qkv{}, o{}, gateup{}, down{}, router{}, ex_gateup{}, ex_down{}, lm_head{};
  std::vector<GemmShape*> used;
  size_t ws_floats = 16, n_tickets = 16;
  long long a_norm = 0, a_o = 0, a_act_slot = 0;   // A operand sizes (uint4)
};

bool build_plan(const spec_config& c, int wf, int G, PassPlan& P, std::string& err) {
  const int d = c.d_model, Hq = c.n_q_heads, Hkv = c.n_kv_heads, D = c.head_dim, V = c.vocab;
  const bool moe = c.n_experts > 0;
  const int E = c.n_experts, S = c.n_shared, F = moe ? c.d_ff_expert : c.d_ff;
  const int window_k = c.gemm_k_split > 0 ? c.gemm_k_split : 2048;
  const int n_slots_max = moe ? E + S : 1;
  P.a_norm = (long long)cdiv(d, 32) * 128;
  P.a_o = (long long)cdiv(Hq * D, 32) * 128;
  P.a_act_slot = (long long)cdiv(F, 32) * 128;
  auto shape = [&](GemmShape& s, const char* name, int K, int N, int tpu, int n_stack, bool slot_major,
                   long long a_slot, long long a_size) {
    s.name = name;
    mat_geometry(s.M, wf, K, N, cdiv(N, 16), tpu, window_k);
    s.wf = wf;
    s.tpu = tpu;
    s.n_stack = n_stack;
    s.n_experts = E;
    s.n_shared = S;
    s.max_slots = n_stack;
    s.slot_major = slot_major;
    s.fixed = false;
    s.a_slot = a_slot;
    s.a_size = a_size;
    P.used.push_back(&s);
  };
  shape(P.qkv, "qkv", d, (Hq + 2 * Hkv) * D, 1, 1, false, 0, P.a_norm);
  shape(P.o, "o", Hq * D, d, 1, 1, false, 0, P.a_o);
  if (!moe) {
    shape(P.gateup, "gate/up", d, F, 2, 1, false, 0, P.a_norm);
    shape(P.down, "down", F, d, 1, 1, false, 0, P.a_act_slot);
  } else {
    shape(P.router, "router", d, E, 1, 1, false, 0, P.a_norm);
    shape(P.ex_gateup, "expert gate/up", d, F, 2, n_slots_max, false, 0, P.a_norm);
    shape(P.ex_down, "expert down", F, d, 1, n_slots_max, true, P.a_act_slot, P.a_act_slot * n_slots_max);
    // the expert phases' split follows the routed union: fixed summation
    // order (the router shares the pass kernel's code path with the expert
    // down projection)
    P.router.fixed = P.ex_gateup.fixed = P.ex_down.fixed = true;
  }
  shape(P.lm_head, "lm_head", d, V, 1, 1, false, 0, P.a_norm);
  for (GemmShape* s : P.used) {
    int ms = 1, mp = 0;
    const int lo = s->max_slots > 1 ? std::max(1, S) : 1;
    for (int ns = lo; ns <= s->max_slots; ++ns) {
      int a = 0, b = 0;
      seg_bounds(s->M, ns, s->slot_major, s->fixed, G, a, b);
      ms = std::max(ms, a);
      mp = std::max(mp, b);
    }
    if (mp > kMaxPending) {
      err = std::string(s->name) + ": matrix too long for the split-K bookkeeping";
      return false;
    }
    s->M.max_seg = ms;
    P.ws_floats = std::max(P.ws_floats, (size_t)s->max_slots * s->M.n_sg * ms * kWaves * s->tpu * 256);
    P.n_tickets = std::max(P.n_tickets, (size_t)s->max_slots * s->M.n_sg);
  }
  for (GemmShape* s : P.used)
    if (s->M.n_win > 256) {   // ready counters per layer
      err = std::string(s->name) + ": too many activation windows";
      return false;
    }
  for (GemmShape* s : P.used)
    if (!check_gemm_walk(*s, G, P.ws_floats, P.n_tickets, err)) return false;
  return true;
}

// ------------------------------------------------------------------ weights
using TKey = std::tuple<int, int, int, int>;

struct Uploader {
  spec_verify* h;
  std::map<TKey, const spec_tensor*> idx;
  void* staging = nullptr;
  size_t staging_bytes = 0;

  const spec_tensor* get(int kind, int layer, int expert, int part, uint64_t bytes) {
    auto it = idx.find(TKey(kind, layer, expert, part));
    if (it == idx.end()) {
      h->err = "missing tensor kind=" + std::to_string(kind) + " layer=" + std::to_string(layer) +
               " expert=" + std::to_string(expert) + " part=" + std::to_string(part);
      return nullptr;
    }
    if (it->second->bytes != bytes || it->second->data == nullptr) {
      h->err = "tensor kind=" + std::to_string(kind) + " layer=" + std::to_string(layer) + " has " +
               std::to_string(it->second->bytes) + " bytes, expected " + std::to_string(bytes);
      return nullptr;
    }
    return it->second;
  }

  // allocate a (possibly stacked) matrix of the planned shape
  int alloc_mat(HostMat& H, const GemmShape& s) {
    Mat& M = H.m;
    M = s.M;
    H.tpu = s.tpu;
    H.n_stack = s.n_stack;
    void* w = nullptr;
    int rc = dalloc_z(h, reinterpret_cast<char**>(&w), (size_t)M.w_stride * s.n_stack);
    if (rc) return rc;
    M.w = w;
    M.w2 = nullptr;
    if (M.w2_stride) {
      void* w2 = nullptr;
      rc = dalloc_z(h, reinterpret_cast<char**>(&w2), (size_t)M.w2_stride * s.n_stack);
      if (rc) return rc;
      M.w2 = w2;
    }
    return SPEC_OK;
  }

  // upload host matrix [K][N] into tiles tile_off + t * tile_stride of stack slot e
  // (pair_dim > 0: columns of every pair_dim-wide head interleaved as rotary
  // pairs, see k_retile)
  int put(HostMat& H, int kind, int layer, int expert, int K, int N, int tile_off, int tile_stride, int e,
          int pair_dim = 0) {
    const int wf = h->wfmt;
    Mat& M = H.m;
    char* wdst = const_cast<char*>(static_cast<const char*>(M.w)) + (long long)e * M.w_stride;
    char* w2dst = M.w2 ? const_cast<char*>(static_cast<const char*>(M.w2)) + (long long)e * M.w2_stride : nullptr;
    hipError_t he;
    if (wf == W_INT4) {
      const spec_tensor* tq = get(kind, layer, expert, 0, (uint64_t)K / 2 * N);
      const spec_tensor* ts = get(kind, layer, expert, 1, (uint64_t)(K / 128) * N * 2);
      if (!tq || !ts) return SPEC_EINVAL;
      const size_t qb = (size_t)K / 2 * N;
      const size_t sb = (size_t)(K / 128) * N * 2;
      const size_t soff = (qb + 255) / 256 * 256;
      he = hipMemcpyAsync(staging, tq->data, qb, hipMemcpyHostToDevice, h->stream);
      if (he == hipSuccess)
        he = hipMemcpyAsync(static_cast<char*>(staging) + soff, ts->data, sb, hipMemcpyHostToDevice, h->stream);
      if (he == hipSuccess)
        he = launch_retile(wf, staging, static_cast<char*>(staging) + soff, K, N, wdst, w2dst, M.nkc, H.tpu,
                           tile_off, tile_stride, pair_dim, h->stream);
    } else {
      const size_t eb = wf == W_F32 ? 4 : 2;
      const spec_tensor* t = get(kind, layer, expert, 0, (uint64_t)K * N * eb);
      if (!t) return SPEC_EINVAL;
      he = hipMemcpyAsync(staging, t->data, (size_t)K * N * eb, hipMemcpyHostToDevice, h->stream);
      if (he == hipSuccess)
        he = launch_retile(wf, staging, nullptr, K, N, wdst, w2dst, M.nkc, H.tpu, tile_off, tile_stride, pair_dim,
                           h->stream);
    }
    if (he == hipSuccess) he = hipStreamSynchronize(h->stream);
    if (he != hipSuccess) return fail(h, SPEC_EHIP, std::string("weight upload: ") + hipGetErrorString(he));
    H.alg_bytes += (double)K * N * elem_bytes(h->cfg.weight_dtype) +
                   (wf == W_INT4 ? (double)(K / 128) * N * 2 : 0.0);
    return SPEC_OK;
  }

  int put_vec(float** dst, int kind, int layer, int n) {
    const spec_tensor* t = get(kind, layer, -1, 0, (uint64_t)n * 4);
    if (!t) return SPEC_EINVAL;
    int rc = dalloc_t(h, dst, n);
    if (rc) return rc;
    hipError_t e = hipMemcpy(*dst, t->data, (size_t)n * 4, hipMemcpyHostToDevice);
    if (e != hipSuccess) return fail(h, SPEC_EHIP, std::string("vector copy: ") + hipGetErrorString(e));
    return SPEC_OK;
  }
};

struct Req {
  int kind, layer, expert, part;
  uint64_t bytes;
};

// Every tensor a configuration needs, with its exact byte size.
std::vector<Req> required_tensors(const spec_config& c) {
  std::vector<Req> r;
  const uint64_t d = c.d_model, V = c.vocab, Hq = c.n_q_heads, Hkv = c.n_kv_heads, D = c.head_dim;
  const bool f32 = c.weight_dtype == SPEC_DT_F32, i4 = c.weight_dtype == SPEC_DT_INT4G128;
  auto mat = [&](int kind, int layer, int expert, uint64_t K, uint64_t N) {
    if (i4) {
      r.push_back({kind, layer, expert, 0, K / 2 * N});
      r.push_back({kind, layer, expert, 1, K / 128 * N * 2});
    } else {
      r.push_back({kind, layer, expert, 0, K * N * (f32 ? 4 : 2)});
    }
  };
  r.push_back({SPEC_T_EMBED, -1, -1, 0, V * d * (f32 ? 4 : 2)});
  r.push_back({SPEC_T_FINAL_NORM, -1, -1, 0, d * 4});
  mat(SPEC_T_LM_HEAD, -1, -1, d, V);
  for (int l = 0; l < c.n_layers; ++l) {
    r.push_back({SPEC_T_ATTN_NORM, l, -1, 0, d * 4});
    r.push_back({SPEC_T_FFN_NORM, l, -1, 0, d * 4});
    mat(SPEC_T_WQ, l, -1, d, Hq * D);
    mat(SPEC_T_WK, l, -1, d, Hkv * D);
    mat(SPEC_T_WV, l, -1, d, Hkv * D);
    mat(SPEC_T_WO, l, -1, Hq * D, d);
    if (c.n_experts > 0) {
      mat(SPEC_T_ROUTER, l, -1, d, c.n_experts);
      r.push_back({SPEC_T_ROUTER_BIAS, l, -1, 0, (uint64_t)c.n_experts * 4});
      for (int e = 0; e < c.n_experts + c.n_shared; ++e) {
        mat(SPEC_T_W_GATE, l, e, d, c.d_ff_expert);
        mat(SPEC_T_W_UP, l, e, d, c.d_ff_expert);
        mat(SPEC_T_W_DOWN, l, e, c.d_ff_expert, d);
      }
    } else {
      mat(SPEC_T_W_GATE, l, -1, d, c.d_ff);
      mat(SPEC_T_W_UP, l, -1, d, c.d_ff);
      mat(SPEC_T_W_DOWN, l, -1, c.d_ff, d);
    }
  }
  return r;
}

// Host-only check of the tensor list: no duplicates, nothing missing or
// extra, exact sizes, non-null data.
bool check_tensors(const spec_config& c, const spec_tensor* t, int n, std::string& msg) {
  std::map<TKey, const spec_tensor*> idx;
  for (int i = 0; i < n; ++i) {
    TKey key(t[i].kind, t[i].layer, t[i].expert, t[i].part);
    if (idx.count(key)) {
      msg = "duplicate tensor kind=" + std::to_string(t[i].kind) + " layer=" + std::to_string(t[i].layer);
      return false;
    }
    idx[key] = &t[i];
  }
  const std::vector<Req> req = required_tensors(c);
  for (const Req& q : req) {
    auto it = idx.find(TKey(q.kind, q.layer, q.expert, q.part));
    const std::string what = "kind=" + std::to_string(q.kind) + " layer=" + std::to_string(q.layer) +
                             " expert=" + std::to_string(q.expert) + " part=" + std::to_string(q.part);
    if (it == idx.end()) {
      msg = "missing tensor " + what;
      return false;
    }
    if (it->second->bytes != q.bytes || !it->second->data) {
      msg = "tensor " + what + " has " + std::to_string(it->second->bytes) + " bytes (expected " +
            std::to_string(q.bytes) + ") or no data";
      return false;
    }
  }
  if (idx.size() != req.size()) {
    msg = "unexpected extra tensors for this configuration";
    return false;
  }
  return true;
}

bool prog_kind_is_gemm(int kind) {
  return kind == PH_STORE || kind == PH_RESID || kind == PH_SWIGLU || kind == PH_LOGITS || kind == PH_ROUTE_SWIGLU ||
         kind == PH_QKV;
}

Phase gemm_phase_desc(int kind, int layer, const HostMat& H) {
  Phase p{};
  p.kind = kind;
  p.layer = layer;
  p.M = H.m;
  return p;
}

int create_impl(spec_verify* h, const spec_tensor* tensors, int32_t n_tensors, const void* prompt_k,
                const void* prompt_v, int32_t prompt_len) {
  const spec_config& c = h->cfg;
  const int d = c.d_model, Hq = c.n_q_heads, Hkv = c.n_kv_heads, D = c.head_dim, V = c.vocab;
  const bool moe = c.n_experts > 0;
  const int E = c.n_experts, S = c.n_shared;
  const int F = moe ? c.d_ff_expert : c.d_ff;
  h->wfmt = c.weight_dtype == SPEC_DT_F32 ? W_F32 : c.weight_dtype == SPEC_DT_BF16 ? W_BF16 : W_INT4;
  int rc;
  HIPCHK(hipGetDevice(&h->device));
  HIPCHK(hipDeviceGetAttribute(&h->n_wg, hipDeviceAttributeMultiprocessorCount, h->device));
  int coop = 0;
  HIPCHK(hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, h->device));
  if (!coop) return fail(h, SPEC_EHIP, "device does not support cooperative launches");
  int wclk = 0;
  HIPCHK(hipDeviceGetAttribute(&wclk, hipDeviceAttributeWallClockRate, h->device));
  h->wall_khz = wclk > 0 ? (double)wclk : 100000.0;
  h->lds = pass_lds_bytes(h->wfmt, max_rows_attn(&c), D);
  int per_cu = 0;
  HIPCHK(pass_occupancy(h->wfmt, c.n_experts > 0, h->lds, &per_cu));
  if (per_cu < 1) return fail(h, SPEC_EHIP, "the pass kernel does not fit on a compute unit");
  PassPlan plan;
  {
    std::string err;
    if (!build_plan(c, h->wfmt, h->n_wg, plan, err)) return fail(h, SPEC_EINVAL, "stream-K plan: " + err);
  }

  Uploader up{h};
  size_t max_bytes = 0;
  for (int i = 0; i < n_tensors; ++i) {
    const spec_tensor& t = tensors[i];
    TKey key(t.kind, t.layer, t.expert, t.part);
    if (up.idx.count(key)) return fail(h, SPEC_EINVAL, "duplicate tensor kind=" + std::to_string(t.kind));
    up.idx[key] = &t;
    max_bytes = std::max<size_t>(max_bytes, t.bytes);
  }
  max_bytes = max_bytes * 2 + 256;   // int4: nibbles and scales staged together
  const size_t kv_elem = c.kv_dtype == SPEC_DT_F32 ? 4 : 2;
  max_bytes = std::max(max_bytes, (size_t)2 * Hkv * std::max(prompt_len, 1) * D * kv_elem);
  if ((rc = dalloc(h, &up.staging, max_bytes))) return rc;
  up.staging_bytes = max_bytes;

  {
    const size_t eb = c.weight_dtype == SPEC_DT_F32 ? 4 : 2;
    const spec_tensor* t = up.get(SPEC_T_EMBED, -1, -1, 0, (uint64_t)V * d * eb);
    if (!t) return SPEC_EINVAL;
    if ((rc = dalloc(h, &h->embed, (size_t)V * d * eb))) return rc;
    HIPCHK(hipMemcpy(h->embed, t->data, (size_t)V * d * eb, hipMemcpyHostToDevice));
  }
  if ((rc = up.put_vec(&h->final_norm, SPEC_T_FINAL_NORM, -1, d))) return rc;
  h->layers.resize(c.n_layers);
  for (int l = 0; l < c.n_layers; ++l) {
    HostLayer& Lw = h->layers[l];
    if ((rc = up.put_vec(&Lw.attn_norm, SPEC_T_ATTN_NORM, l, d))) return rc;
    if ((rc = up.put_vec(&Lw.ffn_norm, SPEC_T_FFN_NORM, l, d))) return rc;
    if ((rc = up.alloc_mat(Lw.qkv, plan.qkv))) return rc;
    // query and key heads with rotary pairs side by side (the QKV epilogue
    // rotates with its neighbouring lane)
    if ((rc = up.put(Lw.qkv, SPEC_T_WQ, l, -1, d, Hq * D, 0, 1, 0, D))) return rc;
    if ((rc = up.put(Lw.qkv, SPEC_T_WK, l, -1, d, Hkv * D, Hq * D / 16, 1, 0, D))) return rc;
    if ((rc = up.put(Lw.qkv, SPEC_T_WV, l, -1, d, Hkv * D, (Hq + Hkv) * D / 16, 1, 0))) return rc;
    if ((rc = up.alloc_mat(Lw.o, plan.o))) return rc;
    if ((rc = up.put(Lw.o, SPEC_T_WO, l, -1, Hq * D, d, 0, 1, 0))) return rc;
    if (!moe) {
      if ((rc = up.alloc_mat(Lw.gateup, plan.gateup))) return rc;
      if ((rc = up.put(Lw.gateup, SPEC_T_W_GATE, l, -1, d, F, 0, 2, 0))) return rc;
      if ((rc = up.put(Lw.gateup, SPEC_T_W_UP, l, -1, d, F, 1, 2, 0))) return rc;
      if ((rc = up.alloc_mat(Lw.down, plan.down))) return rc;
      if ((rc = up.put(Lw.down, SPEC_T_W_DOWN, l, -1, F, d, 0, 1, 0))) return rc;
    } else {
      if ((rc = up.alloc_mat(Lw.router, plan.router))) return rc;
      if ((rc = up.put(Lw.router, SPEC_T_ROUTER, l, -1, d, E, 0, 1, 0))) return rc;
      if ((rc = up.put_vec(&Lw.router_bias, SPEC_T_ROUTER_BIAS, l, E))) return rc;
      if ((rc = up.alloc_mat(Lw.ex_gateup, plan.ex_gateup))) return rc;
      if ((rc = up.alloc_mat(Lw.ex_down, plan.ex_down))) return rc;
      for (int e = 0; e < E + S; ++e) {
        if ((rc = up.put(Lw.ex_gateup, SPEC_T_W_GATE, l, e, d, F, 0, 2, e))) return rc;
        if ((rc = up.put(Lw.ex_gateup, SPEC_T_W_UP, l, e, d, F, 1, 2, e))) return rc;
        if ((rc = up.put(Lw.ex_down, SPEC_T_W_DOWN, l, e, F, d, 0, 1, e))) return rc;
      }
      Lw.ex_gateup.alg_bytes /= (E + S);
      Lw.ex_down.alg_bytes /= (E + S);
    }
  }
  if ((rc = up.alloc_mat(h->lm_head, plan.lm_head))) return rc;
  if ((rc = up.put(h->lm_head, SPEC_T_LM_HEAD, -1, -1, d, V, 0, 1, 0))) return rc;

  // KV cache pages and the page table (identity, or a seeded permutation)
  h->n_seqs = c.n_seqs > 0 ? c.n_seqs : 1;
  h->pps = cdiv(c.max_ctx, kPage);
  h->n_pages = h->n_seqs * h->pps;
  h->kv_layer_elems = (long long)h->n_pages * Hkv * 2 * kPage * D;
  if ((rc = dalloc_z(h, reinterpret_cast<char**>(&h->kv), (size_t)h->kv_layer_elems * c.n_layers * kv_elem)))
    return rc;
  for (int l = 0; l < c.n_layers; ++l)
    h->layers[l].kv = static_cast<char*>(h->kv) + (long long)l * h->kv_layer_elems * (long long)kv_elem;
  {
    std::vector<int> pt(h->n_pages);
    for (int i = 0; i < h->n_pages; ++i) pt[i] = i;
    if (c.kv_page_seed != 0) {
      // Fisher-Yates with a splitmix64 stream seeded by kv_page_seed
      unsigned long long st = (unsigned long long)(unsigned)c.kv_page_seed;
      auto next = [&st]() {
        unsigned long long z = (st += 0x9E3779B97F4A7C15ull);
        z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
        z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
        return z ^ (z >> 31);
      };
      for (int i = h->n_pages - 1; i > 0; --i) std::swap(pt[i], pt[(int)(next() % (unsigned long long)(i + 1))]);
    }
    if ((rc = dalloc_t(h, &h->page_table, h->n_pages))) return rc;
    HIPCHK(hipMemcpy(h->page_table, pt.data(), sizeof(int) * h->n_pages, hipMemcpyHostToDevice));
    h->pt_host = pt;
  }
  h->seq_len.assign(h->n_seqs, 0);
  if (prompt_len > 0) {
    const size_t lb = (size_t)Hkv * prompt_len * D * kv_elem;
    for (int l = 0; l < c.n_layers; ++l) {
      HIPCHK(hipMemcpyAsync(up.staging, static_cast<const char*>(prompt_k) + l * lb, lb, hipMemcpyHostToDevice,
                            h->stream));
      HIPCHK(hipMemcpyAsync(static_cast<char*>(up.staging) + lb, static_cast<const char*>(prompt_v) + l * lb, lb,
                            hipMemcpyHostToDevice, h->stream));
      HIPCHK(launch_kv_import(c.kv_dtype == SPEC_DT_F32, up.staging, prompt_len, Hkv, D, h->layers[l].kv,
                              h->page_table, h->stream));
      HIPCHK(hipStreamSynchronize(h->stream));
    }
  }
  h->kv_len = prompt_len;
  // rotary table [max_ctx][D/2][2], angles in double
  {
    std::vector<float> cs((size_t)c.max_ctx * (D / 2) * 2);
    for (int pos = 0; pos < c.max_ctx; ++pos)
      for (int i = 0; i < D / 2; ++i) {
        const double inv = std::pow((double)c.rope_theta, -2.0 * i / D);
        const double a = (double)pos * inv;
        cs[((size_t)pos * (D / 2) + i) * 2 + 0] = (float)std::cos(a);
        cs[((size_t)pos * (D / 2) + i) * 2 + 1] = (float)std::sin(a);
      }
    if ((rc = dalloc_t(h, &h->rope_cs, cs.size()))) return rc;
    HIPCHK(hipMemcpy(h->rope_cs, cs.data(), cs.size() * 4, hipMemcpyHostToDevice));
  }
  // activations and scratch (zero-filled)
  h->ldx = rup(d, 32);
  h->ldl = rup(V, 32);
  h->n_ss = cdiv(d, 16);
  h->n_stat = cdiv(V, 16);
  h->ldr = rup(std::max(E, 1), 32);
  const int n_slots_max = moe ? E + S : 1;
  if ((rc = dalloc_z(h, &h->x, 16 * (size_t)h->ldx))) return rc;
  // per-layer buffers for data crossing a dataflow edge (each address is
  // written once per pass, so no cache can hold a stale copy of it)
  h->qf_rt = cdiv(max_rows_attn(&c), 16);
  h->qf_layer = (long long)Hkv * h->qf_rt * (D / 32) * 2 * 64;
  if ((rc = dalloc_z(h, &h->qf, (size_t)h->qf_layer * c.n_layers))) return rc;
  if ((rc = dalloc_z(h, &h->ready, (size_t)kReadyStride * c.n_layers))) return rc;
  h->o_wcols = plan.o.M.win * (h->wfmt == W_INT4 ? kGroupK : kChunkK);
  // norm sites: 2l = input of layer l's QKV, 2l+1 = input of its FFN /
  // router, 2L = input of the LM head; each site's A operand and
  // sum-of-squares partials are written once per pass
  const int n_sites = 2 * c.n_layers + 1;
  h->ss_site = 16LL * h->n_ss;
  if ((rc = dalloc_z(h, &h->ss, (size_t)h->ss_site * n_sites))) return rc;
  if ((rc = dalloc_z(h, &h->logits, 16 * (size_t)h->ldl))) return rc;
  h->a_norm_site = plan.a_norm;
  if ((rc = dalloc_z(h, &h->a_norm, (size_t)plan.a_norm * n_sites))) return rc;
  h->a_o_layer = plan.a_o;
  if ((rc = dalloc_z(h, &h->a_o, (size_t)plan.a_o * c.n_layers))) return rc;
  h->a_act_slot = plan.a_act_slot;
  h->a_act_layer = h->a_act_slot * n_slots_max;
  if ((rc = dalloc_z(h, &h->a_act, (size_t)h->a_act_layer * c.n_layers))) return rc;
  if ((rc = dalloc_z(h, &h->st_max, 16 * (size_t)h->n_stat))) return rc;
  if ((rc = dalloc_z(h, &h->st_sum, 16 * (size_t)h->n_stat))) return rc;
  if ((rc = dalloc_z(h, &h->st_idx, 16 * (size_t)h->n_stat))) return rc;
  const size_t Rmax = (size_t)max_rows_attn(&c);
  // (several sequences: one slot space of all of them, page-aligned)
  const size_t max_groups = cdiv((size_t)h->n_pages * kPage, (size_t)kGroupPos);
  if ((rc = dalloc_z(h, &h->pm, Hkv * max_groups * Rmax))) return rc;
  if ((rc = dalloc_z(h, &h->ps, Hkv * max_groups * Rmax))) return rc;
  if ((rc = dalloc_z(h, &h->pacc, Hkv * max_groups * Rmax * D))) return rc;
  // two split-K banks, alternating between consecutive weight-streaming
  // phases (a phase fed over ready counters may start while its
  // predecessor's reductions still run)
  if ((rc = dalloc_z(h, &h->ws, 2 * plan.ws_floats))) return rc;
  if ((rc = dalloc_z(h, &h->tickets, 2 * plan.n_tickets))) return rc;
  h->ws_bank_floats = plan.ws_floats;
  h->tickets_bank = plan.n_tickets;
  // the fixed scratch that spec_verify_step_noalloc uses in place of ws and
  // tickets: two banks of partials, then two banks of tickets
  if (scratch_setup(h->device, &h->scratch) != hipSuccess) h->scratch = nullptr;   // no-alloc steps then refuse
  h->scratch_fits = (2 * plan.ws_floats * 4 + 255) / 256 * 256 + 2 * plan.n_tickets * 4 <= kScratchBytes;
  if ((rc = dalloc_z(h, &h->attn_tickets, (size_t)Hkv + 16))) return rc;
  if ((rc = dalloc_z(h, &h->bar, 512))) return rc;
  if ((rc = dalloc_z(h, &h->tokens_dev, 16))) return rc;
  if ((rc = dalloc_z(h, &h->result_dev, 4))) return rc;
  if ((rc = dalloc_z(h, &h->acc_ws, (size_t)kAccFloats))) return rc;
  if (moe) {
    if ((rc = dalloc_z(h, &h->rlog, 16 * (size_t)h->ldr))) return rc;
    h->ey_slot = 16LL * h->ldx;
    if ((rc = dalloc_z(h, &h->ey, (size_t)h->ey_slot * n_slots_max))) return rc;
    if ((rc = dalloc_z(h, &h->route, (size_t)route_words(E, c.top_k)))) return rc;
  }
  HIPCHK(hipHostMalloc(reinterpret_cast<void**>(&h->tokens_host), 16 * sizeof(int), hipHostMallocDefault));
  if (hipHostGetDevicePointer(reinterpret_cast<void**>(&h->tokens_mapped), h->tokens_host, 0) != hipSuccess)
    h->tokens_mapped = nullptr;   // the step then uploads the ids
  HIPCHK(hipHostMalloc(reinterpret_cast<void**>(&h->result_host), 4 * sizeof(int), hipHostMallocDefault));
  if (hipHostGetDevicePointer(reinterpret_cast<void**>(&h->result_mirror), h->result_host, 0) != hipSuccess)
    h->result_mirror = nullptr;   // the step then copies the result back
  if ((rc = dalloc_z(h, &h->draft_res, (size_t)kMaxRows * 4))) return rc;
  if ((rc = dalloc_z(h, &h->tree_dev, (size_t)kMaxRows * 4))) return rc;
  if ((rc = dalloc_z(h, &h->batch_dev, (size_t)batch_words(h)))) return rc;
  if ((rc = dalloc_z(h, &h->batch_res, (size_t)kMaxRows * 4))) return rc;
  HIPCHK(hipHostMalloc(reinterpret_cast<void**>(&h->batch_host), batch_words(h) * sizeof(int), hipHostMallocDefault));
  HIPCHK(hipHostMalloc(reinterpret_cast<void**>(&h->batch_res_host), kMaxRows * 4 * sizeof(int), hipHostMallocDefault));
  HIPCHK(hipHostMalloc(reinterpret_cast<void**>(&h->tree_host), kMaxRows * 4 * sizeof(int), hipHostMallocDefault));
  HIPCHK(hipHostMalloc(reinterpret_cast<void**>(&h->draft_host), (kMaxRows * 4 + 4) * sizeof(int),
                       hipHostMallocDefault));

  // ---- the pass program
  std::vector<Phase> prog;
  std::vector<int> cls;
  std::vector<double> wbytes;
  auto add = [&](const Phase& p, int k, double b) {
    prog.push_back(p);
    cls.push_back(k);
    wbytes.push_back(b);
  };
  {
    Phase p{};
    p.kind = PH_EMBED;
    add(p, SPEC_K_EMBED, 0);
  }
  auto a_site = [&](int i) { return h->a_norm + (long long)i * h->a_norm_site; };
  auto ss_site = [&](int i) { return h->ss + (long long)i * h->ss_site; };
  prog[0].a_out = a_site(0);
  prog[0].ss_out = ss_site(0);
  for (int l = 0; l < c.n_layers; ++l) {
    HostLayer& Lw = h->layers[l];
    const float* next_gain = l + 1 < c.n_layers ? h->layers[l + 1].attn_norm : h->final_norm;
    uint4* act_l = h->a_act + (long long)l * h->a_act_layer;
    uint4* qf_l = h->qf + (long long)l * h->qf_layer;
    uint4* a_o_l = h->a_o + (long long)l * h->a_o_layer;
    Phase q = gemm_phase_desc(PH_QKV, l, Lw.qkv);
    q.a = a_site(2 * l); q.ss_in = ss_site(2 * l); q.kv = Lw.kv; q.a_out = qf_l; q.notify = kDepHeads;
    add(q, SPEC_K_QKV, Lw.qkv.alg_bytes);
    Phase at{};
    at.kind = PH_ATTN; at.layer = l; at.kv = Lw.kv; at.a = qf_l; at.a_out = a_o_l; at.dep = kDepHeads;
    add(at, SPEC_K_ATTN, 0);
    Phase mg{};
    mg.kind = PH_ATTN_MERGE; mg.layer = l; mg.a_out = a_o_l;
    add(mg, SPEC_K_ATTN_COMBINE, 0);
    Phase o = gemm_phase_desc(PH_RESID, l, Lw.o);
    o.a = a_o_l; o.gain = Lw.ffn_norm; o.a_out = a_site(2 * l + 1); o.ss_out = ss_site(2 * l + 1); o.dep = kDepOWin;
    add(o, SPEC_K_O, Lw.o.alg_bytes);
    if (!moe) {
      Phase g = gemm_phase_desc(PH_SWIGLU, l, Lw.gateup);
      g.a = a_site(2 * l + 1); g.ss_in = ss_site(2 * l + 1); g.a_out = act_l;
      add(g, SPEC_K_GATEUP, Lw.gateup.alg_bytes);
      Phase dn = gemm_phase_desc(PH_RESID, l, Lw.down);
      dn.a = act_l; dn.gain = next_gain; dn.a_out = a_site(2 * l + 2); dn.ss_out = ss_site(2 * l + 2); dn.trace = 1;
      add(dn, SPEC_K_DOWN, Lw.down.alg_bytes);
    } else {
      // bf16 routers with K in one A window are computed inside the routed
      // phase by every workgroup (no router phase, no barrier before routing)
      const bool fuse_router = h->wfmt == W_BF16 && Lw.router.m.n_win == 1;
      if (!fuse_router) {
        Phase r = gemm_phase_desc(PH_STORE, l, Lw.router);
        r.a = a_site(2 * l + 1); r.ss_in = ss_site(2 * l + 1); r.out = h->rlog; r.ldo = h->ldr; r.scale = 1;
        add(r, SPEC_K_ROUTER, Lw.router.alg_bytes);
      }
      Phase g = gemm_phase_desc(PH_ROUTE_SWIGLU, l, Lw.ex_gateup);
      g.slot_mode = 1; g.a = a_site(2 * l + 1); g.ss_in = ss_site(2 * l + 1); g.a_out = act_l;
      g.a_out_slot = h->a_act_slot; g.bias = Lw.router_bias;
      if (fuse_router) g.Mr = Lw.router.m;
      add(g, SPEC_K_EXPERT_GATEUP, Lw.ex_gateup.alg_bytes + (fuse_router ? Lw.router.alg_bytes : 0.0));
      Phase dn = gemm_phase_desc(PH_STORE, l, Lw.ex_down);
      dn.slot_mode = 2; dn.a = act_l; dn.a_slot = h->a_act_slot; dn.out = h->ey; dn.ldo = h->ldx;
      dn.out_slot = h->ey_slot; dn.scale = 0;
      add(dn, SPEC_K_EXPERT_DOWN, Lw.ex_down.alg_bytes);
      Phase cb{};
      cb.kind = PH_COMBINE; cb.layer = l; cb.gain = next_gain; cb.trace = 1;
      cb.a_out = a_site(2 * l + 2); cb.ss_out = ss_site(2 * l + 2);
      add(cb, SPEC_K_MOE_COMBINE, 0);
    }
  }
  {
    Phase lm = gemm_phase_desc(PH_LOGITS, -1, h->lm_head);
    lm.a = a_site(2 * c.n_layers); lm.ss_in = ss_site(2 * c.n_layers); lm.out = h->logits; lm.ldo = h->ldl;
    add(lm, SPEC_K_LMHEAD, h->lm_head.alg_bytes);
  }
  h->n_prog = (int)prog.size();
  // split-K banks alternate between consecutive weight-streaming phases
  for (int i = 0, ng = 0; i < h->n_prog; ++i) {
    if (!prog_kind_is_gemm(prog[i].kind)) continue;
    const int bank = ng++ & 1;
    prog[i].ws = h->ws + (size_t)bank * plan.ws_floats;
    prog[i].tickets = h->tickets + (size_t)bank * plan.n_tickets;
    prog[i].ws_bank = bank;
  }
  // grid barriers per pass (every phase but the first, except those fed by
  // ready counters and, with the inline merge, the merge phases)
  h->n_barriers_inline = h->n_barriers_merge = 0;
  for (int i = 1; i < h->n_prog; ++i) {
    const Phase& q = prog[i];
    const bool dep_inline = q.dep != kDepNone || q.kind == PH_ATTN_MERGE;
    const bool dep_merge = q.dep != kDepNone && q.dep != kDepOWin;
    h->n_barriers_inline += dep_inline ? 0 : 1;
    h->n_barriers_merge += dep_merge ? 0 : 1;
  }
  for (int i = h->n_prog - 1, nx = h->n_prog; i >= 0; --i) {
    prog[i].next_gemm = nx;
    if (prog_kind_is_gemm(prog[i].kind)) nx = i;
  }
  h->prog_layer.clear();
  h->prog_kind.clear();
  for (const Phase& q : prog) {
    h->prog_layer.push_back(q.layer);
    h->prog_kind.push_back(q.kind);
  }
  h->prog_cls = cls;
  h->prog_bytes_fixed = wbytes;
  if ((rc = dalloc_t(h, &h->prog, prog.size()))) return rc;
  HIPCHK(hipMemcpy(h->prog, prog.data(), prog.size() * sizeof(Phase), hipMemcpyHostToDevice));
  if ((rc = dalloc_z(h, &h->stamps_dev, (size_t)h->n_prog + 4))) return rc;
  h->stamps_host.assign((size_t)h->n_prog + 4, 0);
  if ((rc = dalloc_z(h, &h->wstamps_dev, (size_t)h->n_prog * h->n_wg * 4))) return rc;
  if (moe && (rc = dalloc_z(h, &h->union_dev_prof, (size_t)c.n_layers))) return rc;
  h->union_host.assign((size_t)std::max(c.n_layers, 1), 0);
  h->wstamps_host.assign((size_t)h->n_prog * h->n_wg * 4, 0);
  for (auto& e : h->ev) HIPCHK(hipEventCreate(&e));

  // the staging buffer is no longer needed
  HIPCHK(hipStreamSynchronize(h->stream));
  auto it = std::find(h->allocs.begin(), h->allocs.end(), up.staging);
  if (it != h->allocs.end()) {
    (void)hipFree(up.staging);
    h->allocs.erase(it);
  }
  return SPEC_OK;
}

void free_all(spec_verify* h) {
  if (h->stream) (void)hipStreamSynchronize(h->stream);
  for (void* p : h->allocs) (void)hipFree(p);
  h->allocs.clear();
  if (h->tokens_host) (void)hipHostFree(h->tokens_host);
  if (h->result_host) (void)hipHostFree(h->result_host);
  if (h->draft_host) (void)hipHostFree(h->draft_host);
  if (h->tree_host) (void)hipHostFree(h->tree_host);
  if (h->batch_host) (void)hipHostFree(h->batch_host);
  if (h->batch_res_host) (void)hipHostFree(h->batch_res_host);
  for (auto& e : h->ev)
    if (e) (void)hipEventDestroy(e);
}

// algorithmic bytes of one phase of the program (profiling)
double phase_bytes(const spec_verify* h, int i, int m, int L, int experts_loaded_layer) {
  const spec_config& c = h->cfg;
  const double kvb = c.kv_dtype == SPEC_DT_F32 ? 4.0 : 2.0;
  const int d = c.d_model, Hq = c.n_q_heads, Hkv = c.n_kv_heads, D = c.head_dim;
  const double w = h->prog_bytes_fixed[i];
  switch (h->prog_cls[i]) {
    case SPEC_K_EMBED: return (double)m * d * (c.weight_dtype == SPEC_DT_F32 ? 4 : 2) + (double)m * d * 4;
    case SPEC_K_QKV:   // weights, A operand, queries out (hi/lo), new keys and values into the cache
      return w + (double)m * d * 4 + (double)m * Hq * D * 4 + (double)m * Hkv * D * 2 * kvb;
    case SPEC_K_ATTN:  // the cache over L + m positions, queries in, attention output (hi/lo)
      return (double)(L + m) * Hkv * D * 2 * kvb + 2.0 * m * Hq * D * 4;
    case SPEC_K_O: return w + (double)m * Hq * D * 4 + 2.0 * m * d * 4;
    case SPEC_K_GATEUP: return w + (double)m * d * 4 + (double)m * c.d_ff * 4;
    case SPEC_K_DOWN: return w + (double)m * c.d_ff * 4 + 2.0 * m * d * 4;
    case SPEC_K_ROUTER: return w + (double)m * d * 4;
    case SPEC_K_EXPERT_GATEUP: return w * (experts_loaded_layer + c.n_shared);
    case SPEC_K_EXPERT_DOWN: return w * (experts_loaded_layer + c.n_shared);
    case SPEC_K_MOE_COMBINE: return (double)m * d * 4 * (2 + c.top_k + c.n_shared);
    case SPEC_K_LMHEAD: return w + (double)m * d * 4 + (double)m * c.vocab * 4;
    default: return 0;
  }
}

// Parameters of one pass over m block rows at committed length L, reading
// the block's token ids from tokens_dev, with top_k routed experts per token
// (MoE).
PassP pass_params(const spec_verify* h, int m, int L, const int* tokens_dev, int top_k, int T = -1) {
  const spec_config& c = h->cfg;
  const bool moe = c.n_experts > 0;
  PassP p{};
  p.m = m; p.L = L; p.n_layers = c.n_layers; p.d = c.d_model; p.Hq = c.n_q_heads; p.Hkv = c.n_kv_heads;
  p.D = c.head_dim; p.V = c.vocab; p.G = c.n_q_heads / c.n_kv_heads; p.E = c.n_experts; p.top_k = top_k;
  p.n_shared = c.n_shared; p.F = moe ? c.d_ff_expert : c.d_ff;
  p.T = T >= 0 ? T : L + m;
  // attention work items (KV head, group, 16-row tile): groups of 3 pages,
  // or of 5 or 6 when that is what keeps every item in one round over the
  // grid (more items than workgroups run in two rounds, each item waiting
  // on its loads); fp32 caches keep 3
  const int n_rt = cdiv(m * p.G, 16);
  p.group_pages = kGroupPages;
  if (c.attn_group_pages > 0)
    p.group_pages = c.attn_group_pages;
  else if (h->wfmt != W_F32)
    for (int gp : {kGroupPages, 5, 6}) {
      p.group_pages = gp;
      if ((long long)c.n_kv_heads * cdiv(p.T, gp * kPage) * n_rt <= h->n_wg) break;
    }
  p.n_groups = cdiv(p.T, p.group_pages * kPage);
  // heads whose merge is small are merged by their last attention item;
  // the merge phases (one per layer) then run without a barrier
  p.attn_inline = (long long)m * p.G * c.head_dim * p.n_groups <= kInlineMergeElems ? 1 : 0;
  p.attn_tickets = h->attn_tickets;
  p.n_ss = h->n_ss;
  p.lds_bytes = (int)h->lds;
  p.eps = c.rms_eps;
  p.inv_d = 1.0f / (float)c.d_model;
  p.attn_scale = 1.0f / std::sqrt((float)c.head_dim);
  p.prog = h->prog; p.n_prog = h->n_prog;
  p.embed = h->embed; p.gain0 = h->layers[0].attn_norm;
  p.tokens = tokens_dev; p.page_table = h->page_table; p.rope_cs = h->rope_cs;
  p.x = h->x; p.ldx = h->ldx;
  p.logits = h->logits; p.ldl = h->ldl;
  p.ready = h->ready; p.epoch = h->epoch + 1; p.qf_rt = h->qf_rt; p.o_wcols = h->o_wcols;
  p.st_max = h->st_max; p.st_sum = h->st_sum; p.st_idx = h->st_idx; p.n_stat = h->n_stat;
  p.pm = h->pm; p.ps = h->ps; p.pacc = h->pacc;
  p.rlog = h->rlog; p.ldr = h->ldr; p.ey = h->ey; p.ey_slot = h->ey_slot; p.ldy = h->ldx;
  p.route = h->route;
  p.bar = h->bar; p.bar_base = h->bar_gen; p.err = h->result_dev + 3;
  return p;
}

// Launches one pass and advances the handle's barrier generation and pass
// count (the device counters are monotonic over the handle's lifetime).
hipError_t launch_counted(spec_verify* h, const PassP& p) {
  const hipError_t he = launch_pass(h->wfmt, h->cfg.n_experts > 0, p, h->n_wg, h->lds, h->stream);
  if (he != hipSuccess) return he;
  h->bar_gen += (unsigned long long)(p.attn_inline ? h->n_barriers_inline : h->n_barriers_merge);
  h->epoch = p.epoch;
  return hipSuccess;
}

int step_impl(spec_verify* h, const int32_t* tokens, int32_t k, int32_t mode, const float* q_dev,
              const float* u_dev, spec_step_result* out, float* logits_dev, float* trace_dev,
              int32_t* union_dev, int32_t* route_dev, bool noalloc = false, int reuse_cap = 0,
              float reuse_alpha = 0.f, const float* reuse_w = nullptr) {
  if (!h) return SPEC_EINVAL;
  if (h->broken) return fail(h, SPEC_ESTATE, "handle unusable after an earlier GPU error");
  const spec_config& c = h->cfg;
  if (!tokens || !out) return fail(h, SPEC_EINVAL, "tokens and out must not be NULL");
  if (k < 0 || k > c.max_k) return fail(h, SPEC_EINVAL, "k out of range [0, max_k]");
  if (mode < SPEC_ACCEPT_GREEDY || mode > SPEC_ACCEPT_NONE) return fail(h, SPEC_EINVAL, "bad acceptance mode");
  for (int i = 0; i <= k; ++i)
    if (tokens[i] < 0 || tokens[i] >= c.vocab) return fail(h, SPEC_EINVAL, "token id out of range");
  if (mode == SPEC_ACCEPT_STOCHASTIC && (!q_dev || !u_dev))
    return fail(h, SPEC_EINVAL, "stochastic acceptance needs q_dev and u_dev");
  const int m = k + 1;
  const int L = h->kv_len;
  if ((long long)L + m > c.max_ctx) return fail(h, SPEC_ECAPACITY, "block exceeds max_ctx");
  if (noalloc && (!h->scratch || !h->scratch_fits))
    return fail(h, SPEC_ECAPACITY, "the split-K workspace of this model exceeds the fixed scratch (" +
                                       std::to_string(kScratchBytes >> 20) + " MiB)");
  const bool moe = c.n_experts > 0;
  int* union_rec = union_dev;
  if (!union_rec && h->profiling && moe) union_rec = h->union_dev_prof;   // allocated at create
  const bool stamps = h->prof_mode == 1;

  // the kernels read the ids from pinned host memory (no upload), unless
  // the device cannot map it
  std::memcpy(h->tokens_host, tokens, sizeof(int32_t) * m);
  const int* tok = h->tokens_mapped ? h->tokens_mapped : h->tokens_dev;
  hipError_t he = h->tokens_mapped ? hipSuccess
                                   : hipMemcpyAsync(h->tokens_dev, h->tokens_host, sizeof(int32_t) * m,
                                                    hipMemcpyHostToDevice, h->stream);
  PassP p = pass_params(h, m, L, tok, c.top_k);
  p.reuse_cap = reuse_cap;
  p.reuse_alpha = reuse_alpha;
  p.reuse_w = reuse_w;
  if (noalloc) {
    // partials in the fixed scratch; its tickets start at zero
    p.ws_alt = static_cast<float*>(h->scratch);
    p.ws_bank_floats = (long long)h->ws_bank_floats;
    p.tickets_alt = reinterpret_cast<unsigned*>(static_cast<char*>(h->scratch) +
                                                (2 * h->ws_bank_floats * 4 + 255) / 256 * 256);
    p.tickets_bank = (long long)h->tickets_bank;
    if (he == hipSuccess) he = launch_zero_u32(p.tickets_alt, 2 * (long long)h->tickets_bank, h->stream);
  }
  p.trace = trace_dev; p.union_hist = union_rec; p.route_hist = moe ? route_dev : nullptr;
  p.stamps = stamps ? h->stamps_dev : nullptr;
  p.wstamps = stamps ? h->wstamps_dev : nullptr;

  if (he == hipSuccess && h->profiling) he = hipEventRecord(h->ev[0], h->stream);
  if (he == hipSuccess) he = launch_counted(h, p);
  if (he != hipSuccess) {
    h->broken = true;
    return fail(h, SPEC_EHIP, std::string("pass launch: ") + hipGetErrorString(he));
  }
  if (h->profiling) he = hipEventRecord(h->ev[1], h->stream);
  AcceptParams a{};
  a.k = k; a.V = c.vocab; a.L = L; a.mode = mode; a.n_stat = h->n_stat;
  a.tokens = tok;
  a.st_max = h->st_max; a.st_sum = h->st_sum; a.st_idx = h->st_idx;
  a.logits = h->logits; a.ldl = h->ldl;
  a.q = q_dev; a.u = u_dev;
  a.result = h->result_dev;
  a.acc_ws = h->acc_ws;
  a.result_mirror = h->result_mirror;   // the acceptance writes the result to the host itself
  if (he == hipSuccess) he = launch_accept(a, h->stream);
  if (he == hipSuccess && h->profiling) he = hipEventRecord(h->ev[2], h->stream);
  if (he == hipSuccess && !a.result_mirror)
    he = hipMemcpyAsync(h->result_host, h->result_dev, 4 * sizeof(int), hipMemcpyDeviceToHost, h->stream);
  if (he == hipSuccess && logits_dev)
    he = hipMemcpy2DAsync(logits_dev, (size_t)c.vocab * 4, h->logits, (size_t)h->ldl * 4, (size_t)c.vocab * 4, m,
                          hipMemcpyDeviceToDevice, h->stream);
  if (he == hipSuccess && stamps)
    he = hipMemcpyAsync(h->stamps_host.data(), h->stamps_dev, sizeof(unsigned long long) * h->n_prog,
                        hipMemcpyDeviceToHost, h->stream);
  if (he == hipSuccess && stamps)
    he = hipMemcpyAsync(h->wstamps_host.data(), h->wstamps_dev, sizeof(unsigned long long) * h->wstamps_host.size(),
                        hipMemcpyDeviceToHost, h->stream);
  std::vector<int>& uh = h->union_host;
  if (he == hipSuccess && h->profiling && moe)
    he = hipMemcpyAsync(uh.data(), union_rec, sizeof(int) * c.n_layers, hipMemcpyDeviceToHost, h->stream);
  if (he == hipSuccess) he = hipStreamSynchronize(h->stream);
  if (he != hipSuccess) {
    h->broken = true;
    return fail(h, SPEC_EHIP, std::string("step completion: ") + hipGetErrorString(he));
  }
  if (h->result_host[3] != 0) {
    h->broken = true;
    return fail(h, SPEC_EHIP, "grid barrier wait timed out inside the pass");
  }
  if (h->profiling) {
    float pass_ms = 0.f, acc_ms = 0.f;
    (void)hipEventElapsedTime(&pass_ms, h->ev[0], h->ev[1]);
    (void)hipEventElapsedTime(&acc_ms, h->ev[1], h->ev[2]);
    long long experts_loaded = 0;
    if (moe)
      for (int l = 0; l < c.n_layers; ++l) experts_loaded += uh[l];
    const double tick_ms = 1.0 / h->wall_khz;
    double stamped = 0;
    for (int i = 0; i < h->n_prog && stamps; ++i) {
      double ms;
      if (i + 1 < h->n_prog) {
        ms = (double)(h->stamps_host[i + 1] - h->stamps_host[i]) * tick_ms;
        stamped += ms;
      } else {
        ms = std::max(0.0, (double)pass_ms - stamped);
      }
      const int layer = std::max(0, h->prog_layer[i]);
      const double b = phase_bytes(h, i, m, L, moe ? uh[layer] : 0);
      const int k2 = h->prog_cls[i];
      {
        // per-workgroup split of the phase: A staging, weight stream and
        // flush (GEMM phases; other phases: all in the third) and the whole
        // work, each as mean and max over workgroups
        const unsigned long long* w = h->wstamps_host.data() + (size_t)i * h->n_wg * 4;
        const bool gemm = prog_kind_is_gemm(h->prog_kind[i]) || h->prog_kind[i] == PH_ATTN;
        double sum[4] = {0, 0, 0, 0}, mx[4] = {0, 0, 0, 0};
        for (int g = 0; g < h->n_wg; ++g) {
          const unsigned long long* q = w + (size_t)g * 4;
          double v[4];
          v[0] = gemm ? (double)(q[1] - q[0]) * tick_ms : 0.0;
          v[1] = gemm ? (double)(q[2] - q[1]) * tick_ms : 0.0;
          v[2] = gemm ? (double)(q[3] - q[2]) * tick_ms : (double)(q[3] - q[0]) * tick_ms;
          v[3] = (double)(q[3] - q[0]) * tick_ms;
          for (int j = 0; j < 4; ++j) {
            sum[j] += v[j];
            mx[j] = std::max(mx[j], v[j]);
          }
        }
        for (int j = 0; j < 4; ++j) {
          h->prof_detail[k2][j] += sum[j] / h->n_wg;
          h->prof_detail[k2][4 + j] += mx[j];
        }
      }
      h->prof_launches[k2] += 1;
      h->prof_ms[k2] += ms;
      h->prof_bytes[k2] += b;
    }
    h->prof_launches[SPEC_K_PASS] += 1;
    h->prof_ms[SPEC_K_PASS] += pass_ms;
    h->prof_bytes[SPEC_K_PASS] += spec_pass_bytes(h, L, k, mode, experts_loaded);
    h->prof_launches[SPEC_K_ACCEPT] += 1;
    h->prof_ms[SPEC_K_ACCEPT] += acc_ms;
    h->prof_bytes[SPEC_K_ACCEPT] +=
        (double)m * h->n_stat * 12 + (mode == SPEC_ACCEPT_STOCHASTIC ? (double)c.vocab * 8 + (double)k * 8 : 0.0);
  }
  out->n_accepted = h->result_host[0];
  out->next_token = h->result_host[1];
  out->kv_len = h->result_host[2];
  h->kv_len = out->kv_len;
  h->err.clear();
  return SPEC_OK;
}

}  // namespace

// ====================================================================== C ABI

extern "C" {

int spec_config_check(const spec_config* cfg, char* msg, int32_t msg_len) {
  std::string m;
  const bool ok = check_cfg(cfg, m);
  if (msg && msg_len > 0) std::snprintf(msg, (size_t)msg_len, "%s", ok ? "" : m.c_str());
  return ok ? SPEC_OK : SPEC_EINVAL;
}

int spec_plan_check(const spec_config* cfg, int32_t n_wg, char* msg, int32_t msg_len) {
  std::string m;
  bool ok = n_wg >= 1 && n_wg <= 4096;
  if (!ok) m = "n_wg must be in [1, 4096]";
  if (ok) ok = check_cfg(cfg, m);
  if (ok) {
    PassPlan plan;
    const int wf = cfg->weight_dtype == SPEC_DT_F32 ? W_F32 : cfg->weight_dtype == SPEC_DT_BF16 ? W_BF16 : W_INT4;
    ok = build_plan(*cfg, wf, n_wg, plan, m);
  }
  if (msg && msg_len > 0) std::snprintf(msg, (size_t)msg_len, "%s", ok ? "" : m.c_str());
  return ok ? SPEC_OK : SPEC_EINVAL;
}

int spec_verify_create(const spec_config* cfg, const spec_tensor* tensors, int32_t n_tensors,
                       const void* prompt_k, const void* prompt_v, int32_t prompt_len, void* stream,
                       spec_verify_t** out) {
  if (!out) return SPEC_EINVAL;
  *out = nullptr;
  std::string m;
  if (!check_cfg(cfg, m)) return SPEC_EINVAL;
  if (!tensors || n_tensors <= 0) return SPEC_EINVAL;
  if (prompt_len < 0 || prompt_len > cfg->max_ctx) return SPEC_ECAPACITY;
  if (prompt_len > 0 && (!prompt_k || !prompt_v)) return SPEC_EINVAL;
  if (!check_tensors(*cfg, tensors, n_tensors, m)) {
    std::fprintf(stderr, "spec_verify_create: %s\n", m.c_str());
    return SPEC_EINVAL;
  }
  spec_verify* h = new (std::nothrow) spec_verify();
  if (!h) return SPEC_ENOMEM;
  h->cfg = *cfg;
  h->stream = static_cast<hipStream_t>(stream);
  int rc = create_impl(h, tensors, n_tensors, prompt_k, prompt_v, prompt_len);
  if (rc != SPEC_OK) {
    std::fprintf(stderr, "spec_verify_create: %s\n", h->err.c_str());
    free_all(h);
    delete h;
    return rc;
  }
  *out = h;
  return SPEC_OK;
}

int spec_verify_step(spec_verify_t* h, const int32_t* tokens, int32_t k, int32_t mode, const float* q_dev,
                     const float* u_dev, spec_step_result* out, float* logits_dev) {
  return step_impl(h, tokens, k, mode, q_dev, u_dev, out, logits_dev, nullptr, nullptr, nullptr);
}

int spec_verify_step_noalloc(spec_verify_t* h, const int32_t* tokens, int32_t k, int32_t mode,
                             const float* q_dev, const float* u_dev, spec_step_result* out, float* logits_dev) {
  return step_impl(h, tokens, k, mode, q_dev, u_dev, out, logits_dev, nullptr, nullptr, nullptr, true);
}

int spec_verify_step_reuse(spec_verify_t* h, const int32_t* tokens, int32_t k, int32_t mode, const float* q_dev,
                           const float* u_dev, const float* conf_dev, int32_t cap, float alpha,
                           spec_step_result* out, float* logits_dev, int32_t* union_dev, int32_t* route_dev) {
  if (!h) return SPEC_EINVAL;
  const spec_config& c = h->cfg;
  if (c.n_experts <= 0) return fail(h, SPEC_EINVAL, "reuse-aware gating needs a MoE model");
  if (c.top_k >= c.n_experts) return fail(h, SPEC_EINVAL, "reuse-aware gating needs top_k < n_experts");
  if (cap < c.top_k || cap > c.n_experts) return fail(h, SPEC_EINVAL, "cap must be in [top_k, n_experts]");
  if (!(alpha >= 0.f) || !(alpha <= 1e6f)) return fail(h, SPEC_EINVAL, "alpha must be finite and >= 0");
  return step_impl(h, tokens, k, mode, q_dev, u_dev, out, logits_dev, nullptr, union_dev, route_dev, false, cap,
                   alpha, conf_dev);
}

int spec_verify_step_debug(spec_verify_t* h, const int32_t* tokens, int32_t k, int32_t mode,
                           const float* q_dev, const float* u_dev, spec_step_result* out, float* logits_dev,
                           float* trace_dev, int32_t* union_dev, int32_t* route_dev) {
  return step_impl(h, tokens, k, mode, q_dev, u_dev, out, logits_dev, trace_dev, union_dev, route_dev);
}

int spec_verify_tree(spec_verify_t* h, const int32_t* tokens, const int32_t* parents, int32_t m,
                     spec_step_result* out, int32_t* path, float* logits_dev) {
  if (!h) return SPEC_EINVAL;
  if (h->broken) return fail(h, SPEC_ESTATE, "handle unusable after an earlier GPU error");
  const spec_config& c = h->cfg;
  if (!tokens || !parents || !out || !path) return fail(h, SPEC_EINVAL, "tokens, parents, out and path are required");
  if (m < 1 || m > c.max_k + 1) return fail(h, SPEC_EINVAL, "m must be in [1, max_k + 1]");
  for (int i = 0; i < m; ++i)
    if (tokens[i] < 0 || tokens[i] >= c.vocab) return fail(h, SPEC_EINVAL, "token id out of range");
  if (parents[0] != -1) return fail(h, SPEC_EINVAL, "row 0 (the pending token) is the root: parents[0] must be -1");
  int* depth = h->tree_host + kMaxRows;   // rotary positions L + depth
  unsigned* anc = reinterpret_cast<unsigned*>(h->tree_host + 2 * kMaxRows);
  depth[0] = h->kv_len;
  anc[0] = 1u;
  for (int i = 1; i < m; ++i) {
    if (parents[i] < 0 || parents[i] >= i) return fail(h, SPEC_EINVAL, "every parent must precede its row");
    depth[i] = depth[parents[i]] + 1;
    anc[i] = anc[parents[i]] | (1u << i);
  }
  const int L = h->kv_len;
  if ((long long)L + m > c.max_ctx) return fail(h, SPEC_ECAPACITY, "block exceeds max_ctx");
  std::memcpy(h->tree_host, parents, sizeof(int32_t) * m);
  std::memcpy(h->tokens_host, tokens, sizeof(int32_t) * m);
  hipError_t he = hipMemcpyAsync(h->tokens_dev, h->tokens_host, sizeof(int32_t) * m, hipMemcpyHostToDevice, h->stream);
  if (he == hipSuccess)
    he = hipMemcpyAsync(h->tree_dev, h->tree_host, sizeof(int) * 3 * kMaxRows, hipMemcpyHostToDevice, h->stream);
  PassP p = pass_params(h, m, L, h->tokens_dev, c.top_k);
  p.row_rope = h->tree_dev + kMaxRows;
  p.tree_anc = reinterpret_cast<const unsigned*>(h->tree_dev + 2 * kMaxRows);
  if (he == hipSuccess) he = launch_counted(h, p);
  AcceptParams a{};
  a.k = m - 1; a.V = c.vocab; a.L = L; a.mode = kAcceptTree; a.n_stat = h->n_stat;
  a.tokens = h->tokens_dev; a.parents = h->tree_dev; a.path = h->tree_dev + 3 * kMaxRows;
  a.st_max = h->st_max; a.st_sum = h->st_sum; a.st_idx = h->st_idx;
  a.logits = h->logits; a.ldl = h->ldl;
  a.result = h->result_dev;
  a.acc_ws = h->acc_ws;
  if (he == hipSuccess) he = launch_accept(a, h->stream);
  // the accepted rows' cache entries to consecutive slots after the pending token's
  if (he == hipSuccess)
    he = launch_tree_commit(c.kv_dtype == SPEC_DT_F32, h->kv, h->kv_layer_elems, c.n_layers, c.n_kv_heads, c.head_dim,
                            h->page_table, L, h->result_dev, a.path, h->stream);
  if (he == hipSuccess)
    he = hipMemcpyAsync(h->result_host, h->result_dev, 4 * sizeof(int), hipMemcpyDeviceToHost, h->stream);
  if (he == hipSuccess)
    he = hipMemcpyAsync(h->tree_host + 3 * kMaxRows, a.path, kMaxRows * sizeof(int), hipMemcpyDeviceToHost, h->stream);
  if (he == hipSuccess && logits_dev)
    he = hipMemcpy2DAsync(logits_dev, (size_t)c.vocab * 4, h->logits, (size_t)h->ldl * 4, (size_t)c.vocab * 4, m,
                          hipMemcpyDeviceToDevice, h->stream);
  if (he == hipSuccess) he = hipStreamSynchronize(h->stream);
  if (he != hipSuccess) {
    h->broken = true;
    return fail(h, SPEC_EHIP, std::string("tree step: ") + hipGetErrorString(he));
  }
  if (h->result_host[3] != 0) {
    h->broken = true;
    return fail(h, SPEC_EHIP, "grid barrier wait timed out inside the pass");
  }
  out->n_accepted = h->result_host[0];
  out->next_token = h->result_host[1];
  out->kv_len = h->result_host[2];
  for (int i = 0; i < out->n_accepted; ++i) path[i] = h->tree_host[3 * kMaxRows + i];
  h->kv_len = out->kv_len;
  h->err.clear();
  return SPEC_OK;
}

int spec_verify_batch(spec_verify_t* h, int32_t n, const int32_t* seqs, const int32_t* tokens, const int32_t* ks,
                      int32_t mode, spec_step_result* out, float* logits_dev) {
  if (!h) return SPEC_EINVAL;
  if (h->broken) return fail(h, SPEC_ESTATE, "handle unusable after an earlier GPU error");
  const spec_config& c = h->cfg;
  if (!seqs || !tokens || !ks || !out) return fail(h, SPEC_EINVAL, "seqs, tokens, ks and out are required");
  if (n < 1 || n > h->n_seqs || n > kMaxRows) return fail(h, SPEC_EINVAL, "n must be in [1, n_seqs]");
  if (mode != SPEC_ACCEPT_GREEDY && mode != SPEC_ACCEPT_NONE)
    return fail(h, SPEC_EINVAL, "several sequences step with greedy acceptance or none");
  int m = 0;
  for (int i = 0; i < n; ++i) {
    if (seqs[i] < 0 || seqs[i] >= h->n_seqs) return fail(h, SPEC_EINVAL, "sequence id out of range");
    for (int j = 0; j < i; ++j)
      if (seqs[j] == seqs[i]) return fail(h, SPEC_EINVAL, "a sequence appears twice");
    if (ks[i] < 0) return fail(h, SPEC_EINVAL, "k must be >= 0");
    m += ks[i] + 1;
  }
  if (m > c.max_k + 1) return fail(h, SPEC_EINVAL, "the blocks' rows (sum of k + 1) exceed max_k + 1");
  for (int i = 0; i < m; ++i)
    if (tokens[i] < 0 || tokens[i] >= c.vocab) return fail(h, SPEC_EINVAL, "token id out of range");
  auto len = [&](int s) { return s == 0 ? h->kv_len : h->seq_len[s]; };
  for (int i = 0; i < n; ++i)
    if ((long long)len(seqs[i]) + ks[i] + 1 > c.max_ctx) return fail(h, SPEC_ECAPACITY, "a block exceeds max_ctx");
  // one slot space: the sequences' live pages side by side, in call order
  int* B = h->batch_host;
  int* vpt = B + kBatchPages;
  int* live = vpt + h->n_pages;
  int V = 0, r = 0, T = 0;
  for (int i = 0; i < n; ++i) {
    const int s = seqs[i], L = len(s), mi = ks[i] + 1, np = cdiv(L + mi, kPage);
    for (int pg = 0; pg < np; ++pg) {
      vpt[V / kPage + pg] = h->pt_host[(size_t)s * h->pps + pg];
      live[V / kPage + pg] = std::min(kPage, L + mi - pg * kPage);
    }
    B[kBatchSeq + 3 * i + 0] = r;
    B[kBatchSeq + 3 * i + 1] = ks[i];
    B[kBatchSeq + 3 * i + 2] = L;
    for (int j = 0; j < mi; ++j, ++r) {
      B[kBatchSlot + r] = V + L + j;
      B[kBatchRope + r] = L + j;
      B[kBatchLo + r] = V;
      B[kBatchHi + r] = V + L + j;
    }
    T = V + L + mi;
    V += np * kPage;
  }
  std::memcpy(h->tokens_host, tokens, sizeof(int32_t) * m);
  hipError_t he = hipMemcpyAsync(h->tokens_dev, h->tokens_host, sizeof(int32_t) * m, hipMemcpyHostToDevice, h->stream);
  if (he == hipSuccess)
    he = hipMemcpyAsync(h->batch_dev, B, sizeof(int) * (kBatchPages + 2 * (size_t)h->n_pages), hipMemcpyHostToDevice,
                        h->stream);
  PassP p = pass_params(h, m, 0, h->tokens_dev, c.top_k, T);
  p.page_table = h->batch_dev + kBatchPages;
  p.page_live = h->batch_dev + kBatchPages + h->n_pages;
  p.row_slot = h->batch_dev + kBatchSlot;
  p.row_rope = h->batch_dev + kBatchRope;
  p.row_lo = h->batch_dev + kBatchLo;
  p.row_hi = h->batch_dev + kBatchHi;
  const bool moe = c.n_experts > 0;
  if (h->profiling && moe) p.union_hist = h->union_dev_prof;
  if (he == hipSuccess && h->profiling) he = hipEventRecord(h->ev[0], h->stream);
  if (he == hipSuccess) he = launch_counted(h, p);
  if (he == hipSuccess && h->profiling) he = hipEventRecord(h->ev[1], h->stream);
  AcceptParams a{};
  a.k = m - 1; a.V = c.vocab; a.L = 0; a.n_stat = h->n_stat;
  a.mode = mode == SPEC_ACCEPT_GREEDY ? kAcceptBatchGreedy : kAcceptBatchNone;
  a.n_seq = n; a.seq_info = h->batch_dev + kBatchSeq;
  a.tokens = h->tokens_dev;
  a.st_max = h->st_max; a.st_sum = h->st_sum; a.st_idx = h->st_idx;
  a.logits = h->logits; a.ldl = h->ldl;
  a.result = h->batch_res;
  a.acc_ws = h->acc_ws;
  if (he == hipSuccess) he = launch_accept(a, h->stream);
  if (he == hipSuccess && h->profiling && moe)
    he = hipMemcpyAsync(h->union_host.data(), h->union_dev_prof, sizeof(int) * c.n_layers, hipMemcpyDeviceToHost,
                        h->stream);
  if (he == hipSuccess)
    he = hipMemcpyAsync(h->batch_res_host, h->batch_res, sizeof(int) * 4 * n, hipMemcpyDeviceToHost, h->stream);
  if (he == hipSuccess)
    he = hipMemcpyAsync(h->result_host, h->result_dev, 4 * sizeof(int), hipMemcpyDeviceToHost, h->stream);
  if (he == hipSuccess && logits_dev)
    he = hipMemcpy2DAsync(logits_dev, (size_t)c.vocab * 4, h->logits, (size_t)h->ldl * 4, (size_t)c.vocab * 4, m,
                          hipMemcpyDeviceToDevice, h->stream);
  if (he == hipSuccess) he = hipStreamSynchronize(h->stream);
  if (he != hipSuccess) {
    h->broken = true;
    return fail(h, SPEC_EHIP, std::string("batch step: ") + hipGetErrorString(he));
  }
  if (h->result_host[3] != 0) {
    h->broken = true;
    return fail(h, SPEC_EHIP, "grid barrier wait timed out inside the pass");
  }
  if (h->profiling) {   // the pass's events; per-phase stamps are not taken for several sequences
    float pass_ms = 0.f;
    (void)hipEventElapsedTime(&pass_ms, h->ev[0], h->ev[1]);
    long long experts_loaded = 0, sum_L = 0;
    if (moe)
      for (int l = 0; l < c.n_layers; ++l) experts_loaded += h->union_host[l];
    for (int i = 0; i < n; ++i) sum_L += B[kBatchSeq + 3 * i + 2];
    h->prof_launches[SPEC_K_PASS] += 1;
    h->prof_ms[SPEC_K_PASS] += pass_ms;
    h->prof_bytes[SPEC_K_PASS] += spec_pass_bytes(h, (int32_t)sum_L, m - 1, SPEC_ACCEPT_GREEDY, experts_loaded);
  }
  for (int i = 0; i < n; ++i) {
    out[i].n_accepted = h->batch_res_host[4 * i + 0];
    out[i].next_token = h->batch_res_host[4 * i + 1];
    out[i].kv_len = h->batch_res_host[4 * i + 2];
    if (seqs[i] == 0) h->kv_len = out[i].kv_len;
    else h->seq_len[seqs[i]] = out[i].kv_len;
  }
  h->err.clear();
  return SPEC_OK;
}

int32_t spec_seq_kv_len(const spec_verify_t* h, int32_t seq) {
  if (!h || seq < 0 || seq >= h->n_seqs) return -1;
  return seq == 0 ? h->kv_len : h->seq_len[seq];
}

int spec_seq_rollback(spec_verify_t* h, int32_t seq, int32_t new_kv_len) {
  if (!h) return SPEC_EINVAL;
  if (h->broken) return fail(h, SPEC_ESTATE, "handle unusable after an earlier GPU error");
  if (seq < 0 || seq >= h->n_seqs) return fail(h, SPEC_EINVAL, "sequence id out of range");
  int& len = seq == 0 ? h->kv_len : h->seq_len[seq];
  if (new_kv_len < 0 || new_kv_len > len) return fail(h, SPEC_EINVAL, "rollback length must be in [0, kv_len]");
  len = new_kv_len;
  h->err.clear();
  return SPEC_OK;
}

int spec_seq_import(spec_verify_t* h, int32_t seq, const void* prompt_k, const void* prompt_v, int32_t prompt_len) {
  if (!h) return SPEC_EINVAL;
  if (h->broken) return fail(h, SPEC_ESTATE, "handle unusable after an earlier GPU error");
  const spec_config& c = h->cfg;
  if (seq < 0 || seq >= h->n_seqs) return fail(h, SPEC_EINVAL, "sequence id out of range");
  if (prompt_len < 0 || prompt_len > c.max_ctx) return fail(h, SPEC_ECAPACITY, "prompt exceeds max_ctx");
  if (prompt_len > 0 && (!prompt_k || !prompt_v)) return fail(h, SPEC_EINVAL, "prompt_k and prompt_v are required");
  const size_t kv_elem = c.kv_dtype == SPEC_DT_F32 ? 4 : 2;
  const size_t lb = (size_t)c.n_kv_heads * prompt_len * c.head_dim * kv_elem;
  if (prompt_len > 0) {
    void* staging = nullptr;
    HIPCHK(hipMalloc(&staging, 2 * lb));
    hipError_t he = hipSuccess;
    for (int l = 0; l < c.n_layers && he == hipSuccess; ++l) {
      he = hipMemcpyAsync(staging, static_cast<const char*>(prompt_k) + l * lb, lb, hipMemcpyHostToDevice, h->stream);
      if (he == hipSuccess)
        he = hipMemcpyAsync(static_cast<char*>(staging) + lb, static_cast<const char*>(prompt_v) + l * lb, lb,
                            hipMemcpyHostToDevice, h->stream);
      if (he == hipSuccess)
        he = launch_kv_import(c.kv_dtype == SPEC_DT_F32, staging, prompt_len, c.n_kv_heads, c.head_dim,
                              h->layers[l].kv, h->page_table + (size_t)seq * h->pps, h->stream);
      if (he == hipSuccess) he = hipStreamSynchronize(h->stream);
    }
    (void)hipFree(staging);
    if (he != hipSuccess) {
      h->broken = true;
      return fail(h, SPEC_EHIP, std::string("import: ") + hipGetErrorString(he));
    }
  }
  (seq == 0 ? h->kv_len : h->seq_len[seq]) = prompt_len;
  h->err.clear();
  return SPEC_OK;
}

int spec_draft(spec_verify_t* h, int32_t pending, int32_t n, int32_t draft_top_k, int32_t* drafts,
               float* logits_dev, int32_t* route_dev) {
  if (!h) return SPEC_EINVAL;
  if (h->broken) return fail(h, SPEC_ESTATE, "handle unusable after an earlier GPU error");
  const spec_config& c = h->cfg;
  if (c.n_experts <= 0) return fail(h, SPEC_EINVAL, "drafting by expert sparsity needs a MoE model");
  if (draft_top_k < 1 || draft_top_k > c.top_k) return fail(h, SPEC_EINVAL, "draft_top_k must be in [1, top_k]");
  if (n < 1 || n > kMaxRows) return fail(h, SPEC_EINVAL, "n must be in [1, 16]");
  if (!drafts) return fail(h, SPEC_EINVAL, "drafts must not be NULL");
  if (pending < 0 || pending >= c.vocab) return fail(h, SPEC_EINVAL, "token id out of range");
  const int L0 = h->kv_len;
  if ((long long)L0 + n > c.max_ctx) return fail(h, SPEC_ECAPACITY, "draft exceeds max_ctx");
  h->tokens_host[0] = pending;
  hipError_t he = hipMemcpyAsync(h->tokens_dev, h->tokens_host, sizeof(int32_t), hipMemcpyHostToDevice, h->stream);
  // pass i reads its token from pass i-1's acceptance record (device-side
  // chaining: no host round trip between draft tokens)
  for (int i = 0; i < n && he == hipSuccess; ++i) {
    const int* tok = i == 0 ? h->tokens_dev : h->draft_res + 4 * (i - 1) + 1;
    PassP p = pass_params(h, 1, L0 + i, tok, draft_top_k);
    if (route_dev) p.route_hist = route_dev + (long long)i * c.n_layers * draft_top_k;
    he = launch_counted(h, p);
    AcceptParams a{};
    a.k = 0; a.V = c.vocab; a.L = L0 + i; a.mode = SPEC_ACCEPT_NONE; a.n_stat = h->n_stat;
    a.tokens = tok;
    a.st_max = h->st_max; a.st_sum = h->st_sum; a.st_idx = h->st_idx;
    a.logits = h->logits; a.ldl = h->ldl;
    a.result = h->draft_res + 4 * i;
    a.acc_ws = h->acc_ws;
    if (he == hipSuccess) he = launch_accept(a, h->stream);
    if (he == hipSuccess && logits_dev)
      he = hipMemcpyAsync(logits_dev + (long long)i * c.vocab, h->logits, (size_t)c.vocab * 4, hipMemcpyDeviceToDevice,
                          h->stream);
  }
  if (he == hipSuccess)
    he = hipMemcpyAsync(h->draft_host, h->draft_res, sizeof(int) * 4 * n, hipMemcpyDeviceToHost, h->stream);
  if (he == hipSuccess)
    he = hipMemcpyAsync(h->draft_host + kMaxRows * 4, h->result_dev, sizeof(int) * 4, hipMemcpyDeviceToHost,
                        h->stream);
  if (he == hipSuccess) he = hipStreamSynchronize(h->stream);
  if (he != hipSuccess) {
    h->broken = true;
    return fail(h, SPEC_EHIP, std::string("draft: ") + hipGetErrorString(he));
  }
  if (h->draft_host[kMaxRows * 4 + 3] != 0) {
    h->broken = true;
    return fail(h, SPEC_EHIP, "grid barrier wait timed out inside a draft pass");
  }
  for (int i = 0; i < n; ++i) drafts[i] = h->draft_host[4 * i + 1];
  // the committed length is unchanged: the draft's cache entries are dead
  h->err.clear();
  return SPEC_OK;
}

int spec_kv_commit_rollback(spec_verify_t* h, int32_t new_kv_len) {
  if (!h) return SPEC_EINVAL;
  if (h->broken) return fail(h, SPEC_ESTATE, "handle unusable after an earlier GPU error");
  if (new_kv_len < 0 || new_kv_len > h->kv_len)
    return fail(h, SPEC_EINVAL, "rollback length must be in [0, kv_len]");
  h->kv_len = new_kv_len;
  h->err.clear();
  return SPEC_OK;
}

int32_t spec_kv_len(const spec_verify_t* h) { return h ? h->kv_len : -1; }

int32_t spec_tree_expand(int32_t n, const int32_t* parents, const double* p, const int32_t* exp_offsets,
                         const int32_t* exp_ids, int32_t n_base, const int32_t* base_ids, double t_ar, double t_exp,
                         const double* c_draft, int32_t max_nodes, int32_t* order, int32_t* row_parents) {
#pragma clang fp contract(off)   // the utilities are compared exactly: plain products and sums
  if (n < 0 || n_base < 0 || max_nodes < 0) return -1;
  if (n > 0 && (!parents || !p || !exp_offsets || !c_draft)) return -1;
  if (n_base > 0 && !base_ids) return -1;
  if (max_nodes > 0 && !order) return -1;
  if (!(t_ar >= 0.0) || !(t_exp >= 0.0) || !std::isfinite(t_ar) || !std::isfinite(t_exp)) return -1;
  if (n > 0 && exp_offsets[0] != 0) return -1;
  std::vector<std::vector<int32_t>> ex(n);
  std::vector<double> conf(n);
  for (int i = 0; i < n; ++i) {
    if (parents[i] < -1 || parents[i] >= i) return -1;
    if (!(p[i] >= 0.0 && p[i] <= 1.0) || !(c_draft[i] >= 0.0) || !std::isfinite(c_draft[i])) return -1;
    if (exp_offsets[i + 1] < exp_offsets[i] || (exp_offsets[i + 1] > exp_offsets[i] && !exp_ids)) return -1;
    for (int j = exp_offsets[i]; j < exp_offsets[i + 1]; ++j) {
      if (exp_ids[j] < 0) return -1;
      ex[i].push_back(exp_ids[j]);
    }
    std::sort(ex[i].begin(), ex[i].end());
    ex[i].erase(std::unique(ex[i].begin(), ex[i].end()), ex[i].end());
    // prefix confidence: the product of the draft probabilities root..i
    conf[i] = parents[i] < 0 ? p[i] : conf[parents[i]] * p[i];
  }
  std::vector<int32_t> active;
  for (int j = 0; j < n_base; ++j) {
    if (base_ids[j] < 0) return -1;
    active.push_back(base_ids[j]);
  }
  std::sort(active.begin(), active.end());
  active.erase(std::unique(active.begin(), active.end()), active.end());
  std::vector<char> taken(n, 0);
  std::vector<int32_t> row(n, -1);
  int cnt = 0;
  while (cnt < max_nodes) {
    int best = -1;
    double best_u = -1.0;
    for (int i = 0; i < n; ++i) {
      if (taken[i] || (parents[i] >= 0 && !taken[parents[i]])) continue;
      int fresh = 0;   // experts verifying i would activate beyond the admitted set's
      for (int32_t e : ex[i]) fresh += !std::binary_search(active.begin(), active.end(), e);
      const double benefit = conf[i] * t_ar;
      const double cost = (double)fresh * t_exp + c_draft[i];
      const double u = benefit <= 0.0 ? 0.0 : (cost <= 0.0 ? INFINITY : benefit / cost);
      if (u > best_u) { best = i; best_u = u; }
    }
    if (best < 0 || best_u < 1.0) break;
    taken[best] = 1;
    row[best] = cnt + 1;
    if (row_parents) row_parents[cnt + 1] = parents[best] < 0 ? 0 : row[parents[best]];
    order[cnt++] = best;
    std::vector<int32_t> merged;
    std::set_union(active.begin(), active.end(), ex[best].begin(), ex[best].end(), std::back_inserter(merged));
    active.swap(merged);
  }
  if (row_parents) row_parents[0] = -1;
  return cnt;
}

int64_t spec_debug_fail_alloc(int64_t n) { return g_fail_alloc.exchange(n < 0 ? -1 : n); }

int32_t spec_adaptive_k(int32_t k, int32_t n_accepted, int32_t max_k) {
  if (max_k < 1 || k < 1 || k > max_k || n_accepted < 0 || n_accepted > k) return -1;
  if (n_accepted == k) return k + 2 < max_k ? k + 2 : max_k;   // the whole block passed: look further
  return k - 1 > 1 ? k - 1 : 1;                               // a draft failed: back off by one
}

int spec_kv_poison_dead(spec_verify_t* h) {
  if (!h) return SPEC_EINVAL;
  if (h->broken) return fail(h, SPEC_ESTATE, "handle unusable after an earlier GPU error");
  const spec_config& c = h->cfg;
  HIPCHK(launch_kv_poison(c.kv_dtype == SPEC_DT_F32, h->kv, h->kv_layer_elems, c.n_layers, c.n_kv_heads,
                          c.head_dim, h->page_table, h->kv_len, c.max_ctx, h->stream));
  HIPCHK(hipStreamSynchronize(h->stream));
  h->err.clear();
  return SPEC_OK;
}

const char* spec_last_error(const spec_verify_t* h) { return h ? h->err.c_str() : kNullMsg; }

void spec_verify_destroy(spec_verify_t* h) {
  if (!h) return;
  free_all(h);
  delete h;
}

int spec_profile_enable(spec_verify_t* h, int32_t on) {
  if (!h) return SPEC_EINVAL;
  if (on < 0 || on > 2) return fail(h, SPEC_EINVAL, "profiling mode must be 0, 1 or 2");
  h->prof_mode = on;
  h->profiling = on != 0;
  for (int i = 0; i < SPEC_K_NCLASSES; ++i) {
    h->prof_launches[i] = 0;
    h->prof_ms[i] = 0;
    h->prof_bytes[i] = 0;
    for (int j = 0; j < 8; ++j) h->prof_detail[i][j] = 0;
  }
  return SPEC_OK;
}

int spec_profile_raw(const spec_verify_t* h, uint64_t* out, int64_t n, int64_t* count) {
  if (!h) return SPEC_EINVAL;
  const int64_t total = (int64_t)h->n_prog * h->n_wg * 4;
  if (count) *count = total;
  if (!out) return SPEC_OK;
  if (n < total) return SPEC_ECAPACITY;
  for (int64_t i = 0; i < total; ++i) out[i] = h->wstamps_host[i];
  return SPEC_OK;
}

int spec_profile_detail(const spec_verify_t* h, double* out) {
  if (!h || !out) return SPEC_EINVAL;
  for (int i = 0; i < SPEC_K_NCLASSES; ++i)
    for (int j = 0; j < 8; ++j) out[i * 8 + j] = h->prof_detail[i][j];
  return SPEC_OK;
}

int spec_profile_read(const spec_verify_t* h, int64_t* launches, double* ms, double* bytes) {
  if (!h) return SPEC_EINVAL;
  for (int i = 0; i < SPEC_K_NCLASSES; ++i) {
    if (launches) launches[i] = h->prof_launches[i];
    if (ms) ms[i] = h->prof_ms[i];
    if (bytes) bytes[i] = h->prof_bytes[i];
  }
  return SPEC_OK;
}

double spec_pass_bytes(const spec_verify_t* h, int32_t L, int32_t k, int32_t mode, int64_t experts_loaded) {
  if (!h) return -1.0;
  const spec_config& c = h->cfg;
  const double kvb = c.kv_dtype == SPEC_DT_F32 ? 4.0 : 2.0;
  const double kappa = (double)c.n_layers * c.n_kv_heads * c.head_dim * 2 * kvb;   // KV bytes / position
  double w = h->lm_head.alg_bytes;
  for (const auto& Lw : h->layers) {
    w += Lw.qkv.alg_bytes + Lw.o.alg_bytes;
    if (c.n_experts > 0) {
      w += Lw.router.alg_bytes + (double)c.n_shared * (Lw.ex_gateup.alg_bytes + Lw.ex_down.alg_bytes);
    } else {
      w += Lw.gateup.alg_bytes + Lw.down.alg_bytes;
    }
  }
  if (c.n_experts > 0 && !h->layers.empty())
    w += (double)experts_loaded * (h->layers[0].ex_gateup.alg_bytes + h->layers[0].ex_down.alg_bytes);
  const double m = k + 1;
  double b = w + (double)L * kappa + m * kappa + m * c.vocab * 4.0;
  if (mode == SPEC_ACCEPT_STOCHASTIC) b += (double)k * c.vocab * 4.0;
  return b;
}

}  // extern "C"
