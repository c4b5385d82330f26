// Host runtime of the verification-step library: configuration checks,
// weight upload and re-tiling, the paged KV cache, the launch sequence of
// one verification pass, acceptance readback and KV commit / rollback.
#include "../../include/spec_verify.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <map>
#include <string>
#include <tuple>
#include <vector>

#include "sv_common.h"

using namespace sv;

namespace {

inline int rup(int a, int b) { return ((a + b - 1) / b) * b; }
inline int cdiv(int a, int b) { return (a + b - 1) / b; }

struct Mat {
  void* w = nullptr;
  void* w2 = nullptr;
  int K = 0, N = 0, nkc = 0, n_tiles = 0;
  long long w_stride = 0, w2_stride = 0;   // bytes per expert (stacked MoE matrices)
  double alg_bytes = 0;                    // logical weight bytes per expert
};

struct LayerW {
  Mat qkv, o, gateup, down, router, ex_gateup, ex_down;
  float* attn_norm = nullptr;
  float* ffn_norm = nullptr;
  float* router_bias = nullptr;
};

struct ProfRec {
  int cls;
  double bytes;
  hipEvent_t a, b;
};

}  // namespace

struct spec_verify {
  spec_config cfg{};
  hipStream_t stream = nullptr;
  int device = 0;
  int wfmt = W_BF16;
  std::vector<LayerW> layers;
  void* embed = nullptr;
  Mat lm_head;
  float* final_norm = nullptr;
  // KV cache
  void* kv = nullptr;
  long long kv_layer_elems = 0;
  int n_pages = 0;
  int* page_table = nullptr;
  float* rope_cs = nullptr;
  // activations / scratch
  int ldx = 0, ldqkv = 0, ldo_attn = 0, ldact = 0, ldl = 0, n_ss = 0, n_stat = 0;
  float *x = nullptr, *qkv = nullptr, *attn_o = nullptr, *act = nullptr, *ss = nullptr, *logits = nullptr;
  float *st_max = nullptr, *st_sum = nullptr;
  int* st_idx = nullptr;
  float *pm = nullptr, *ps = nullptr, *pacc = nullptr;
  float* ws = nullptr;
  unsigned* counters = nullptr;
  int* tokens_dev = nullptr;
  int* result_dev = nullptr;
  int* tokens_host = nullptr;   // pinned
  int* result_host = nullptr;   // pinned
  // MoE
  float* rlog = nullptr;
  int *ucount = nullptr, *ulist = nullptr, *sel = nullptr, *slot_of = nullptr;
  float* selw = nullptr;
  float *ex_act = nullptr, *ex_y = nullptr;
  int ld_exact = 0;
  long long ex_act_stride = 0, ex_y_stride = 0;
  std::vector<void*> allocs;
  // state
  int kv_len = 0;
  bool broken = false;
  std::string err;
  // profiling
  bool profiling = false;
  std::vector<ProfRec> prof_pending;
  std::vector<hipEvent_t> ev_pool;
  size_t ev_used = 0;
  int64_t prof_launches[SPEC_K_NCLASSES] = {};
  double prof_ms[SPEC_K_NCLASSES] = {};
  double prof_bytes[SPEC_K_NCLASSES] = {};
};

namespace {

const char* kNullMsg = "null handle";

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

int dalloc(spec_verify* h, void** p, size_t bytes) {
  if (bytes == 0) bytes = 16;
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

bool check_cfg(const spec_config* c, std::string& msg) {
  auto bad = [&](const char* m) {
    msg = m;
    return false;
  };
  if (!c) return bad("null config");
  if (c->n_layers < 1 || c->d_model < 1 || c->n_q_heads < 1 || c->n_kv_heads < 1 || c->vocab < 2)
    return bad("n_layers, d_model, heads must be >= 1 and vocab >= 2");
  if (c->n_q_heads % c->n_kv_heads != 0) return bad("n_q_heads must be a multiple of n_kv_heads");
  if (c->head_dim != 64 && c->head_dim != 128) return bad("head_dim must be 64 or 128");
  if (c->weight_dtype < SPEC_DT_F32 || c->weight_dtype > SPEC_DT_INT4G128) return bad("bad weight_dtype");
  if (c->kv_dtype != SPEC_DT_F32 && c->kv_dtype != SPEC_DT_BF16) return bad("kv_dtype must be F32 or BF16");
  if (c->max_k < 0 || c->max_k > 15) return bad("max_k must be in [0, 15]");
  if (c->max_ctx < 1 || c->max_ctx > (1 << 22)) return bad("max_ctx out of range");
  if (!(c->rope_theta > 0.f) || !(c->rms_eps >= 0.f)) return bad("rope_theta must be > 0 and rms_eps >= 0");
  if (c->gemm_k_split < 0 || c->gemm_k_split % 128 != 0 || c->gemm_k_split > 2048)
    return bad("gemm_k_split must be a multiple of 128 in [0, 2048]");
  for (int i = 0; i < 7; ++i)
    if (c->reserved[i] != 0) return bad("reserved fields must be zero");
  const bool moe = c->n_experts > 0;
  if (moe) {
    if (c->n_experts > 256) return bad("n_experts must be <= 256");
    if (c->top_k < 1 || c->top_k > c->n_experts) return bad("top_k must be in [1, n_experts]");
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
  const int G = c->n_q_heads / c->n_kv_heads;
  const long long R = (long long)(c->max_k + 1) * G;
  const long long lds = 4LL * (R * c->head_dim + 2LL * kPage * (c->head_dim + 1) + R * kPage);
  if (lds > 160 * 1024) return bad("(max_k+1) * (n_q_heads/n_kv_heads) too large for the attention kernel");
  return true;
}

double elem_bytes(int dt) { return dt == SPEC_DT_F32 ? 4.0 : dt == SPEC_DT_BF16 ? 2.0 : 0.5; }

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
      h->err = "tensor kind=" + std::to_string(kind) + " layer=" + std::to_string(layer) + " expert=" +
               std::to_string(expert) + " part=" + std::to_string(part) + " has " +
               std::to_string(it->second->bytes) + " bytes, expected " + std::to_string(bytes);
      return nullptr;
    }
    return it->second;
  }

  int stage(const void* src, size_t bytes) {
    hipError_t e = hipMemcpyAsync(staging, src, bytes, hipMemcpyHostToDevice, h->stream);
    if (e != hipSuccess) return fail(h, SPEC_EHIP, std::string("staging copy: ") + hipGetErrorString(e));
    return SPEC_OK;
  }

  // allocate a (possibly stacked) fragment matrix
  int alloc_mat(Mat& M, int K, int N_tiles, int n_stack) {
    const int wf = h->wfmt;
    M.K = K;
    M.n_tiles = N_tiles;
    M.nkc = (wf == W_INT4) ? (K / 128) * 4 : cdiv(K, 32);
    if (wf == W_INT4) {
      M.w_stride = (long long)N_tiles * (K / 128) * 1024;
      M.w2_stride = (long long)N_tiles * (K / 128) * 32;
    } else {
      M.w_stride = (long long)N_tiles * M.nkc * 1024;
      M.w2_stride = (wf == W_F32) ? M.w_stride : 0;
    }
    int rc = dalloc(h, &M.w, (size_t)M.w_stride * n_stack);
    if (rc) return rc;
    if (M.w2_stride) {
      rc = dalloc(h, &M.w2, (size_t)M.w2_stride * n_stack);
      if (rc) return rc;
    }
    return SPEC_OK;
  }

  // upload one host matrix [K][N] into tiles tile_off + t*tile_stride of M (stack slot e)
  int put(Mat& M, int kind, int layer, int expert, int K, int N, int tile_off, int tile_stride, int e) {
    const int wf = h->wfmt;
    char* wdst = static_cast<char*>(M.w) + (long long)e * M.w_stride;
    char* w2dst = M.w2 ? static_cast<char*>(M.w2) + (long long)e * M.w2_stride : nullptr;
    hipError_t he;
    if (wf == W_INT4) {
      const spec_tensor* tq = get(kind, layer, expert, 0, (uint64_t)K / 2 * N);
      const spec_tensor* ts = get(kind, layer, expert, 1, (uint64_t)(K / 128) * N * 2);
      if (!tq || !ts) return SPEC_EINVAL;
      const size_t qb = (size_t)K / 2 * N;
      const size_t sb = (size_t)(K / 128) * N * 2;
      if (stage(tq->data, qb)) return SPEC_EHIP;
      const size_t soff = (qb + 255) / 256 * 256;
      he = hipMemcpyAsync(static_cast<char*>(staging) + soff, ts->data, sb, hipMemcpyHostToDevice, h->stream);
      if (he != hipSuccess) return fail(h, SPEC_EHIP, std::string("scale copy: ") + hipGetErrorString(he));
      he = launch_retile_int4(static_cast<const uint8_t*>(staging),
                              reinterpret_cast<const uint16_t*>(static_cast<char*>(staging) + soff), K, N, wdst,
                              w2dst, tile_off, tile_stride, M.n_tiles, h->stream);
    } else if (wf == W_F32) {
      const spec_tensor* t = get(kind, layer, expert, 0, (uint64_t)K * N * 4);
      if (!t) return SPEC_EINVAL;
      if (stage(t->data, (size_t)K * N * 4)) return SPEC_EHIP;
      he = launch_retile_f32(static_cast<const float*>(staging), K, N, wdst, w2dst, M.nkc, tile_off, tile_stride,
                             h->stream);
    } else {
      const spec_tensor* t = get(kind, layer, expert, 0, (uint64_t)K * N * 2);
      if (!t) return SPEC_EINVAL;
      if (stage(t->data, (size_t)K * N * 2)) return SPEC_EHIP;
      he = launch_retile_bf16(static_cast<const uint16_t*>(staging), K, N, wdst, M.nkc, tile_off, tile_stride,
                              h->stream);
    }
    if (he != hipSuccess) return fail(h, SPEC_EHIP, std::string("retile: ") + hipGetErrorString(he));
    he = hipStreamSynchronize(h->stream);
    if (he != hipSuccess) return fail(h, SPEC_EHIP, std::string("retile sync: ") + hipGetErrorString(he));
    M.alg_bytes += (double)K * N * elem_bytes(h->cfg.weight_dtype) +
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

// ------------------------------------------------------------------ launches

struct Launcher {
  spec_verify* h;
  int rc = SPEC_OK;

  template <typename F>
  void run(int cls, double bytes, F&& f) {
    if (rc) return;
    hipEvent_t a = nullptr, b = nullptr;
    if (h->profiling) {
      if (h->ev_used + 2 > h->ev_pool.size()) {
        for (int i = 0; i < 64; ++i) {
          hipEvent_t e;
          if (hipEventCreate(&e) != hipSuccess) {
            rc = fail(h, SPEC_EHIP, "hipEventCreate failed");
            return;
          }
          h->ev_pool.push_back(e);
        }
      }
      a = h->ev_pool[h->ev_used++];
      b = h->ev_pool[h->ev_used++];
      (void)hipEventRecord(a, h->stream);
    }
    hipError_t e = f();
    if (e != hipSuccess) {
      rc = fail(h, SPEC_EHIP, std::string("kernel launch (class ") + std::to_string(cls) + "): " +
                                  hipGetErrorString(e));
      return;
    }
    if (h->profiling) {
      (void)hipEventRecord(b, h->stream);
      h->prof_pending.push_back(ProfRec{cls, bytes, a, b});
    }
  }
};

GemmParams gemm_base(spec_verify* h, const Mat& M, int m, int N, const float* x, int ldx) {
  GemmParams p{};
  p.m = m;
  p.K = M.K;
  p.nkc = M.nkc;
  p.N = N;
  p.n_tiles = M.n_tiles;
  int kcs = (h->cfg.gemm_k_split > 0 ? h->cfg.gemm_k_split : 1024) / 32;
  kcs = std::min(kcs, M.nkc);
  if (h->wfmt == W_INT4) kcs = std::max(4, (kcs / 4) * 4);
  p.kcs = kcs;
  p.splits = cdiv(M.nkc, kcs);
  p.x = x;
  p.ldx = ldx;
  p.w = M.w;
  p.w2 = M.w2;
  p.w_stride = M.w_stride;
  p.w2_stride = M.w2_stride;
  p.ws = h->ws;
  p.counters = h->counters;
  p.eps = h->cfg.rms_eps;
  p.inv_dnorm = 1.0f / (float)h->cfg.d_model;
  return p;
}

size_t gemm_ws_floats(const Mat& M, int kcs_cfg, int wf, int n_slots) {
  int kcs = std::min(kcs_cfg / 32, M.nkc);
  if (wf == W_INT4) kcs = std::max(4, (kcs / 4) * 4);
  const int splits = cdiv(M.nkc, kcs);
  if (splits <= 1) return 0;
  return (size_t)n_slots * splits * 16 * M.n_tiles * 16;
}

int step_impl(spec_verify* h, const int32_t* tokens, int32_t k, int32_t mode, const float* q_dev,
              const float* u_dev, spec_step_result* out, float* logits_dev, float* trace_dev,
              int32_t* union_dev) {
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

  const int d = c.d_model, Hq = c.n_q_heads, Hkv = c.n_kv_heads, D = c.head_dim, V = c.vocab;
  const int G = Hq / Hkv;
  const bool moe = c.n_experts > 0;
  const double eb = elem_bytes(c.weight_dtype);
  const double kvb = c.kv_dtype == SPEC_DT_F32 ? 4.0 : 2.0;
  Launcher ln{h};

  std::memcpy(h->tokens_host, tokens, sizeof(int32_t) * m);
  hipError_t he = hipMemcpyAsync(h->tokens_dev, h->tokens_host, sizeof(int32_t) * m, hipMemcpyHostToDevice,
                                 h->stream);
  if (he != hipSuccess) {
    h->broken = true;
    return fail(h, SPEC_EHIP, std::string("token upload: ") + hipGetErrorString(he));
  }
  ln.run(SPEC_K_EMBED, (double)m * d * (eb == 4.0 ? 4 : 2) + (double)m * d * 4, [&] {
    return launch_embed(c.weight_dtype == SPEC_DT_F32, h->embed, h->tokens_dev, m, d, h->x, h->ss, h->stream);
  });
  const int n_chunks = cdiv(L + m, kPage);
  for (int l = 0; l < c.n_layers && !ln.rc; ++l) {
    LayerW& Lw = h->layers[l];
    char* kv_layer = static_cast<char*>(h->kv) + (long long)l * h->kv_layer_elems * (long long)kvb;
    {
      GemmParams p = gemm_base(h, Lw.qkv, m, (Hq + 2 * Hkv) * D, h->x, h->ldx);
      p.ss = h->ss;
      p.n_ss = h->n_ss;
      p.gain = Lw.attn_norm;
      p.out = h->qkv;
      p.ldo = h->ldqkv;
      ln.run(SPEC_K_QKV, Lw.qkv.alg_bytes + (double)m * d * 4 + (double)m * p.N * 4,
             [&] { return launch_gemm(h->wfmt, EPI_STORE, p, 1, h->stream); });
    }
    {
      AttnParams a{};
      a.m = m; a.L = L; a.G = G; a.Hq = Hq; a.Hkv = Hkv; a.D = D;
      a.n_chunks = n_chunks;
      a.qkv = h->qkv; a.ldqkv = h->ldqkv;
      a.rope_cs = h->rope_cs;
      a.kv = kv_layer;
      a.page_table = h->page_table;
      a.pm = h->pm; a.ps = h->ps; a.pacc = h->pacc;
      a.R = m * G;
      a.scale = 1.0f / std::sqrt((float)D);
      const double bytes = (double)L * Hkv * D * 2 * kvb + (double)m * Hkv * D * 2 * kvb +
                           (double)m * (Hq + 2 * Hkv) * D * 4;
      ln.run(SPEC_K_ATTN, bytes, [&] { return launch_attention(c.kv_dtype == SPEC_DT_F32, a, h->stream); });
      CombineParams cp{};
      cp.m = m; cp.G = G; cp.Hq = Hq; cp.D = D; cp.n_chunks = n_chunks; cp.R = m * G;
      cp.pm = h->pm; cp.ps = h->ps; cp.pacc = h->pacc;
      cp.o = h->attn_o; cp.ldo = h->ldo_attn;
      ln.run(SPEC_K_ATTN_COMBINE, (double)m * Hq * D * 4 * (1 + n_chunks),
             [&] { return launch_attn_combine(cp, h->stream); });
    }
    {
      GemmParams p = gemm_base(h, Lw.o, m, d, h->attn_o, h->ldo_attn);
      p.out = h->x;
      p.ldo = h->ldx;
      p.ss_out = h->ss;
      p.n_ss_out = h->n_ss;
      ln.run(SPEC_K_O, Lw.o.alg_bytes + (double)m * Hq * D * 4 + 2.0 * m * d * 4,
             [&] { return launch_gemm(h->wfmt, EPI_RESID, p, 1, h->stream); });
    }
    if (!moe) {
      GemmParams p = gemm_base(h, Lw.gateup, m, c.d_ff, h->x, h->ldx);
      p.ss = h->ss;
      p.n_ss = h->n_ss;
      p.gain = Lw.ffn_norm;
      p.out = h->act;
      p.ldo = h->ldact;
      ln.run(SPEC_K_GATEUP, Lw.gateup.alg_bytes + (double)m * d * 4 + (double)m * c.d_ff * 4,
             [&] { return launch_gemm(h->wfmt, EPI_SWIGLU, p, 1, h->stream); });
      GemmParams q = gemm_base(h, Lw.down, m, d, h->act, h->ldact);
      q.out = h->x;
      q.ldo = h->ldx;
      q.ss_out = h->ss;
      q.n_ss_out = h->n_ss;
      ln.run(SPEC_K_DOWN, Lw.down.alg_bytes + (double)m * c.d_ff * 4 + 2.0 * m * d * 4,
             [&] { return launch_gemm(h->wfmt, EPI_RESID, q, 1, h->stream); });
    } else {
      const int E = c.n_experts, S = c.n_shared, Fe = c.d_ff_expert;
      GemmParams p = gemm_base(h, Lw.router, m, E, h->x, h->ldx);
      p.ss = h->ss;
      p.n_ss = h->n_ss;
      p.gain = Lw.ffn_norm;
      p.out = h->rlog;
      p.ldo = rup(E, 32);
      ln.run(SPEC_K_ROUTER, Lw.router.alg_bytes + (double)m * d * 4,
             [&] { return launch_gemm(h->wfmt, EPI_STORE, p, 1, h->stream); });
      RouteParams rp{};
      rp.m = m; rp.E = E; rp.top_k = c.top_k;
      rp.rlogits = h->rlog; rp.ldr = rup(E, 32);
      rp.bias = Lw.router_bias;
      rp.union_count = h->ucount; rp.union_list = h->ulist; rp.sel = h->sel; rp.selw = h->selw;
      rp.slot_of = h->slot_of;
      rp.union_hist = union_dev ? union_dev + l : nullptr;
      ln.run(SPEC_K_ROUTE, (double)m * E * 4, [&] { return launch_route(rp, h->stream); });
      // expert gate/up (+SwiGLU) over the union, then down, per slot
      GemmParams g = gemm_base(h, Lw.ex_gateup, m, Fe, h->x, h->ldx);
      g.ss = h->ss;
      g.n_ss = h->n_ss;
      g.gain = Lw.ffn_norm;
      g.out = h->ex_act;
      g.ldo = h->ld_exact;
      g.out_stride = h->ex_act_stride;
      g.union_count = h->ucount; g.union_list = h->ulist; g.n_experts = E; g.n_shared = S;
      // bytes: accounted per pass from the union size (see spec_pass_bytes)
      ln.run(SPEC_K_EXPERT_GATEUP, 0.0, [&] { return launch_gemm(h->wfmt, EPI_SWIGLU, g, E + S, h->stream); });
      GemmParams dn = gemm_base(h, Lw.ex_down, m, d, h->ex_act, h->ld_exact);
      dn.x_stride = h->ex_act_stride;
      dn.out = h->ex_y;
      dn.ldo = h->ldx;
      dn.out_stride = h->ex_y_stride;
      dn.union_count = h->ucount; dn.union_list = h->ulist; dn.n_experts = E; dn.n_shared = S;
      ln.run(SPEC_K_EXPERT_DOWN, 0.0, [&] { return launch_gemm(h->wfmt, EPI_STORE, dn, E + S, h->stream); });
      MoeCombineParams mc{};
      mc.m = m; mc.d = d; mc.top_k = c.top_k; mc.n_shared = S; mc.n_ss = h->n_ss;
      mc.union_count = h->ucount; mc.sel = h->sel; mc.selw = h->selw; mc.slot_of = h->slot_of;
      mc.y = h->ex_y; mc.y_stride = h->ex_y_stride; mc.ldy = h->ldx;
      mc.x = h->x; mc.ldx = h->ldx; mc.ss_out = h->ss;
      ln.run(SPEC_K_MOE_COMBINE, (double)m * d * 4 * (2 + c.top_k + S),
             [&] { return launch_moe_combine(mc, h->stream); });
    }
    if (trace_dev && !ln.rc) {
      he = hipMemcpy2DAsync(trace_dev + (long long)l * m * d, (size_t)d * 4, h->x, (size_t)h->ldx * 4,
                            (size_t)d * 4, m, hipMemcpyDeviceToDevice, h->stream);
      if (he != hipSuccess) ln.rc = fail(h, SPEC_EHIP, std::string("trace copy: ") + hipGetErrorString(he));
    }
  }
  {
    GemmParams p = gemm_base(h, h->lm_head, m, V, h->x, h->ldx);
    p.ss = h->ss;
    p.n_ss = h->n_ss;
    p.gain = h->final_norm;
    p.out = h->logits;
    p.ldo = h->ldl;
    p.st_max = h->st_max; p.st_sum = h->st_sum; p.st_idx = h->st_idx; p.n_stat = h->n_stat;
    ln.run(SPEC_K_LMHEAD, h->lm_head.alg_bytes + (double)m * d * 4 + (double)m * V * 4,
           [&] { return launch_gemm(h->wfmt, EPI_LOGITS, p, 1, h->stream); });
  }
  {
    AcceptParams a{};
    a.k = k; a.V = V; a.L = L; a.mode = mode; a.n_stat = h->n_stat;
    a.tokens = h->tokens_dev;
    a.st_max = h->st_max; a.st_sum = h->st_sum; a.st_idx = h->st_idx;
    a.logits = h->logits; a.ldl = h->ldl;
    a.q = q_dev; a.u = u_dev;
    a.result = h->result_dev;
    const double bytes = (double)m * h->n_stat * 12 +
                         (mode == SPEC_ACCEPT_STOCHASTIC ? (double)V * 8 + (double)k * 8 : 0.0);
    ln.run(SPEC_K_ACCEPT, bytes, [&] { return launch_accept(a, h->stream); });
  }
  if (ln.rc) {
    h->broken = true;
    return ln.rc;
  }
  he = hipMemcpyAsync(h->result_host, h->result_dev, 3 * sizeof(int), hipMemcpyDeviceToHost, h->stream);
  if (he == hipSuccess && logits_dev)
    he = hipMemcpy2DAsync(logits_dev, (size_t)V * 4, h->logits, (size_t)h->ldl * 4, (size_t)V * 4, m,
                          hipMemcpyDeviceToDevice, h->stream);
  if (he == hipSuccess) he = hipStreamSynchronize(h->stream);
  if (he != hipSuccess) {
    h->broken = true;
    return fail(h, SPEC_EHIP, std::string("step completion: ") + hipGetErrorString(he));
  }
  if (h->profiling) {
    for (auto& r : h->prof_pending) {
      float ms = 0.f;
      if (hipEventElapsedTime(&ms, r.a, r.b) == hipSuccess) {
        h->prof_launches[r.cls] += 1;
        h->prof_ms[r.cls] += ms;
        h->prof_bytes[r.cls] += r.bytes;
      }
    }
    h->prof_pending.clear();
    h->ev_used = 0;
  }
  out->n_accepted = h->result_host[0];
  out->next_token = h->result_host[1];
  out->kv_len = h->result_host[2];
  h->kv_len = out->kv_len;
  h->err.clear();
  return SPEC_OK;
}

void free_all(spec_verify* h) {
  if (h->stream) (void)hipStreamSynchronize(h->stream);
  for (void* p : h->allocs) (void)hipFree(p);
  h->allocs.clear();
  if (h->tokens_host) (void)hipHostFree(h->tokens_host);
  if (h->result_host) (void)hipHostFree(h->result_host);
  for (auto e : h->ev_pool) (void)hipEventDestroy(e);
  h->ev_pool.clear();
}

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

int create_impl(spec_verify* h, const spec_tensor* tensors, int32_t n_tensors, const void* prompt_k,
                const void* prompt_v, int32_t prompt_len) {
  const spec_config& c = h->cfg;
  const int d = c.d_model, Hq = c.n_q_heads, Hkv = c.n_kv_heads, D = c.head_dim, V = c.vocab;
  const bool moe = c.n_experts > 0;
  h->wfmt = c.weight_dtype == SPEC_DT_F32 ? W_F32 : c.weight_dtype == SPEC_DT_BF16 ? W_BF16 : W_INT4;
  int rc;
  HIPCHK(hipGetDevice(&h->device));

  Uploader up{h};
  size_t max_bytes = 0;
  for (int i = 0; i < n_tensors; ++i) {
    const spec_tensor& t = tensors[i];
    TKey key(t.kind, t.layer, t.expert, t.part);
    if (up.idx.count(key)) return fail(h, SPEC_EINVAL, "duplicate tensor kind=" + std::to_string(t.kind));
    up.idx[key] = &t;
    max_bytes = std::max<size_t>(max_bytes, t.bytes);
  }
  // int4 matrices stage packed nibbles and scales together
  max_bytes = max_bytes * 2 + 256;
  const size_t kv_elem = c.kv_dtype == SPEC_DT_F32 ? 4 : 2;
  max_bytes = std::max(max_bytes, (size_t)2 * Hkv * std::max(prompt_len, 1) * D * kv_elem);
  if ((rc = dalloc(h, &up.staging, max_bytes))) return rc;
  up.staging_bytes = max_bytes;

  // embedding
  {
    const size_t eb = c.weight_dtype == SPEC_DT_F32 ? 4 : 2;
    const spec_tensor* t = up.get(SPEC_T_EMBED, -1, -1, 0, (uint64_t)V * d * eb);
    if (!t) return SPEC_EINVAL;
    if ((rc = dalloc(h, &h->embed, (size_t)V * d * eb))) return rc;
    HIPCHK(hipMemcpy(h->embed, t->data, (size_t)V * d * eb, hipMemcpyHostToDevice));
  }
  if ((rc = up.put_vec(&h->final_norm, SPEC_T_FINAL_NORM, -1, d))) return rc;
  h->layers.resize(c.n_layers);
  const int qkv_tiles = (Hq + 2 * Hkv) * D / 16;
  for (int l = 0; l < c.n_layers; ++l) {
    LayerW& Lw = h->layers[l];
    if ((rc = up.put_vec(&Lw.attn_norm, SPEC_T_ATTN_NORM, l, d))) return rc;
    if ((rc = up.put_vec(&Lw.ffn_norm, SPEC_T_FFN_NORM, l, d))) return rc;
    if ((rc = up.alloc_mat(Lw.qkv, d, qkv_tiles, 1))) return rc;
    if ((rc = up.put(Lw.qkv, SPEC_T_WQ, l, -1, d, Hq * D, 0, 1, 0))) return rc;
    if ((rc = up.put(Lw.qkv, SPEC_T_WK, l, -1, d, Hkv * D, Hq * D / 16, 1, 0))) return rc;
    if ((rc = up.put(Lw.qkv, SPEC_T_WV, l, -1, d, Hkv * D, (Hq + Hkv) * D / 16, 1, 0))) return rc;
    if ((rc = up.alloc_mat(Lw.o, Hq * D, cdiv(d, 16), 1))) return rc;
    if ((rc = up.put(Lw.o, SPEC_T_WO, l, -1, Hq * D, d, 0, 1, 0))) return rc;
    if (!moe) {
      const int F = c.d_ff;
      if ((rc = up.alloc_mat(Lw.gateup, d, 2 * cdiv(F, 16), 1))) return rc;
      if ((rc = up.put(Lw.gateup, SPEC_T_W_GATE, l, -1, d, F, 0, 2, 0))) return rc;
      if ((rc = up.put(Lw.gateup, SPEC_T_W_UP, l, -1, d, F, 1, 2, 0))) return rc;
      if ((rc = up.alloc_mat(Lw.down, F, cdiv(d, 16), 1))) return rc;
      if ((rc = up.put(Lw.down, SPEC_T_W_DOWN, l, -1, F, d, 0, 1, 0))) return rc;
    } else {
      const int E = c.n_experts, S = c.n_shared, F = c.d_ff_expert;
      if ((rc = up.alloc_mat(Lw.router, d, cdiv(E, 16), 1))) return rc;
      if ((rc = up.put(Lw.router, SPEC_T_ROUTER, l, -1, d, E, 0, 1, 0))) return rc;
      if ((rc = up.put_vec(&Lw.router_bias, SPEC_T_ROUTER_BIAS, l, E))) return rc;
      if ((rc = up.alloc_mat(Lw.ex_gateup, d, 2 * cdiv(F, 16), E + S))) return rc;
      if ((rc = up.alloc_mat(Lw.ex_down, F, cdiv(d, 16), E + S))) return rc;
      for (int e = 0; e < E + S; ++e) {
        if ((rc = up.put(Lw.ex_gateup, SPEC_T_W_GATE, l, e, d, F, 0, 2, e))) return rc;
        if ((rc = up.put(Lw.ex_gateup, SPEC_T_W_UP, l, e, d, F, 1, 2, e))) return rc;
        if ((rc = up.put(Lw.ex_down, SPEC_T_W_DOWN, l, e, F, d, 0, 1, e))) return rc;
      }
      // per-expert logical bytes (the stack accumulated E+S experts)
      Lw.ex_gateup.alg_bytes /= (E + S);
      Lw.ex_down.alg_bytes /= (E + S);
    }
  }
  if ((rc = up.alloc_mat(h->lm_head, d, cdiv(V, 16), 1))) return rc;
  if ((rc = up.put(h->lm_head, SPEC_T_LM_HEAD, -1, -1, d, V, 0, 1, 0))) return rc;

  // KV cache pages + identity page table
  h->n_pages = cdiv(c.max_ctx, kPage);
  h->kv_layer_elems = (long long)h->n_pages * Hkv * 2 * kPage * D;
  if ((rc = dalloc(h, &h->kv, (size_t)h->kv_layer_elems * c.n_layers * kv_elem))) return rc;
  HIPCHK(hipMemsetAsync(h->kv, 0, (size_t)h->kv_layer_elems * c.n_layers * kv_elem, h->stream));
  {
    std::vector<int> pt(h->n_pages);
    for (int i = 0; i < h->n_pages; ++i) pt[i] = i;
    if ((rc = dalloc_t(h, &h->page_table, h->n_pages))) return rc;
    HIPCHK(hipMemcpy(h->page_table, pt.data(), sizeof(int) * h->n_pages, hipMemcpyHostToDevice));
  }
  if (prompt_len > 0) {
    const size_t lb = (size_t)Hkv * prompt_len * D * kv_elem;
    for (int l = 0; l < c.n_layers; ++l) {
      HIPCHK(hipMemcpyAsync(up.staging, static_cast<const char*>(prompt_k) + l * lb, lb, hipMemcpyHostToDevice,
                            h->stream));
      HIPCHK(hipMemcpyAsync(static_cast<char*>(up.staging) + lb, static_cast<const char*>(prompt_v) + l * lb, lb,
                            hipMemcpyHostToDevice, h->stream));
      char* base = static_cast<char*>(h->kv) + (long long)l * h->kv_layer_elems * (long long)kv_elem;
      HIPCHK(launch_kv_import(c.kv_dtype == SPEC_DT_F32, up.staging, prompt_len, Hkv, D, base, h->page_table,
                              h->stream));
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
  // activations and scratch
  h->ldx = rup(d, 32);
  h->ldqkv = rup((Hq + 2 * Hkv) * D, 32);
  h->ldo_attn = rup(Hq * D, 32);
  h->ldact = rup(moe ? 32 : c.d_ff, 32);
  h->ldl = rup(V, 32);
  h->n_ss = cdiv(d, 64);
  h->n_stat = cdiv(cdiv(V, 16), 4);
  if ((rc = dalloc_t(h, &h->x, 16 * h->ldx))) return rc;
  if ((rc = dalloc_t(h, &h->qkv, 16 * h->ldqkv))) return rc;
  if ((rc = dalloc_t(h, &h->attn_o, 16 * h->ldo_attn))) return rc;
  if ((rc = dalloc_t(h, &h->act, 16 * h->ldact))) return rc;
  if ((rc = dalloc_t(h, &h->ss, 16 * h->n_ss))) return rc;
  if ((rc = dalloc_t(h, &h->logits, 16 * (size_t)h->ldl))) return rc;
  if ((rc = dalloc_t(h, &h->st_max, 16 * h->n_stat))) return rc;
  if ((rc = dalloc_t(h, &h->st_sum, 16 * h->n_stat))) return rc;
  if ((rc = dalloc_t(h, &h->st_idx, 16 * h->n_stat))) return rc;
  const int G = Hq / Hkv;
  const size_t Rmax = (size_t)(c.max_k + 1) * G;
  const size_t max_chunks = cdiv(c.max_ctx, kPage);
  if ((rc = dalloc_t(h, &h->pm, Hkv * max_chunks * Rmax))) return rc;
  if ((rc = dalloc_t(h, &h->ps, Hkv * max_chunks * Rmax))) return rc;
  if ((rc = dalloc_t(h, &h->pacc, Hkv * max_chunks * Rmax * D))) return rc;
  // split-K scratch and tickets
  const int ksplit = c.gemm_k_split > 0 ? c.gemm_k_split : 1024;
  size_t ws = 0, ctr = 0;
  auto acc_mat = [&](const Mat& M, int n_slots) {
    ws = std::max(ws, gemm_ws_floats(M, ksplit, h->wfmt, n_slots));
    ctr = std::max(ctr, (size_t)n_slots * cdiv(M.n_tiles, 4));
  };
  for (auto& Lw : h->layers) {
    acc_mat(Lw.qkv, 1);
    acc_mat(Lw.o, 1);
    if (!moe) {
      acc_mat(Lw.gateup, 1);
      acc_mat(Lw.down, 1);
    } else {
      acc_mat(Lw.router, 1);
      acc_mat(Lw.ex_gateup, c.n_experts + c.n_shared);
      acc_mat(Lw.ex_down, c.n_experts + c.n_shared);
    }
  }
  acc_mat(h->lm_head, 1);
  if ((rc = dalloc_t(h, &h->ws, std::max<size_t>(ws, 16)))) return rc;
  if ((rc = dalloc_t(h, &h->counters, std::max<size_t>(ctr, 16)))) return rc;
  HIPCHK(hipMemsetAsync(h->counters, 0, std::max<size_t>(ctr, 16) * sizeof(unsigned), h->stream));
  if ((rc = dalloc_t(h, &h->tokens_dev, 16))) return rc;
  if ((rc = dalloc_t(h, &h->result_dev, 4))) return rc;
  HIPCHK(hipHostMalloc(reinterpret_cast<void**>(&h->tokens_host), 16 * sizeof(int), hipHostMallocDefault));
  HIPCHK(hipHostMalloc(reinterpret_cast<void**>(&h->result_host), 4 * sizeof(int), hipHostMallocDefault));
  if (moe) {
    const int E = c.n_experts, S = c.n_shared, F = c.d_ff_expert;
    if ((rc = dalloc_t(h, &h->rlog, 16 * rup(E, 32)))) return rc;
    if ((rc = dalloc_t(h, &h->ucount, 4))) return rc;
    if ((rc = dalloc_t(h, &h->ulist, E + 4))) return rc;
    if ((rc = dalloc_t(h, &h->sel, 16 * c.top_k))) return rc;
    if ((rc = dalloc_t(h, &h->selw, 16 * c.top_k))) return rc;
    if ((rc = dalloc_t(h, &h->slot_of, E + 4))) return rc;
    h->ld_exact = rup(F, 32);
    h->ex_act_stride = 16LL * h->ld_exact;
    h->ex_y_stride = 16LL * h->ldx;
    if ((rc = dalloc_t(h, &h->ex_act, (size_t)(E + S) * h->ex_act_stride))) return rc;
    if ((rc = dalloc_t(h, &h->ex_y, (size_t)(E + S) * h->ex_y_stride))) return rc;
  }
  // the staging buffer is no longer needed
  HIPCHK(hipStreamSynchronize(h->stream));
  auto it = std::find(h->allocs.begin(), h->allocs.end(), up.staging);
  if (it != h->allocs.end()) {
    (void)hipFree(up.staging);
    h->allocs.erase(it);
  }
  return SPEC_OK;
}

}  // namespace

// ====================================================================== C ABI

extern "C" {

int spec_config_check(const spec_config* cfg, char* msg, int32_t msg_len) {
  std::string m;
  const bool ok = check_cfg(cfg, m);
  if (msg && msg_len > 0) {
    std::snprintf(msg, (size_t)msg_len, "%s", ok ? "" : m.c_str());
  }
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
  return step_impl(h, tokens, k, mode, q_dev, u_dev, out, logits_dev, nullptr, nullptr);
}

int spec_verify_step_debug(spec_verify_t* h, const int32_t* tokens, int32_t k, int32_t mode,
                           const float* q_dev, const float* u_dev, spec_step_result* out, float* logits_dev,
                           float* trace_dev, int32_t* union_dev) {
  return step_impl(h, tokens, k, mode, q_dev, u_dev, out, logits_dev, trace_dev, union_dev);
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

const char* spec_last_error(const spec_verify_t* h) { return h ? h->err.c_str() : kNullMsg; }

void spec_verify_destroy(spec_verify_t* h) {
  if (!h) return;
  free_all(h);
  delete h;
}

int spec_profile_enable(spec_verify_t* h, int32_t on) {
  if (!h) return SPEC_EINVAL;
  h->profiling = on != 0;
  for (int i = 0; i < SPEC_K_NCLASSES; ++i) {
    h->prof_launches[i] = 0;
    h->prof_ms[i] = 0;
    h->prof_bytes[i] = 0;
  }
  h->prof_pending.clear();
  h->ev_used = 0;
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
