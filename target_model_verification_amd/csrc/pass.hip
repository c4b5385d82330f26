// The verification pass as one persistent cooperative kernel (gfx950).
//
// One target forward pass over the block [pending, d_1..d_k] (m = k+1 rows)
// at cache positions L..L+m-1: embedding, then per layer QKV projection,
// causal attention over the paged KV cache (the block's rotated keys and
// values are rounded to the KV dtype and appended), O projection, FFN
// (dense SwiGLU, or MoE router + union of the block's experts + combine),
// and the LM head.  (Essay "LLM Inference: Speculative Decoding", "The
// loop" step 2: one target pass answers every block position; S2-MoE §3,
// Challenge 2: a verification block activates a union of experts.)
//
// Why one kernel.  The pass is bound by HBM bandwidth: every weight byte is
// used by at most 16 rows.  At 7B scale each layer streams ~400 MB in
// ~60 us at 8 TB/s, so per-kernel launch gaps and ramp-up/drain would cost a
// large share of the time.  Here one workgroup of 4 waves runs on every CU
// for the whole pass; phases are separated by grid barriers, and before
// waiting at a barrier each wave already issues the loads of its first
// weight batches of the next phase (weights never depend on activations),
// so HBM keeps streaming through the synchronization.
//
// Weight-streaming phases ("GEMM phases") compute Y[m][N] = A[m][K] W[K][N]
// on v_mfma_f32_16x16x32_bf16 tiles:
//  - W is pre-tiled into 1 KB B-operand fragments grouped in supergroups of
//    4 output units (one per wave); the workgroups split the flattened
//    (supergroup, K chunk) space into equal contiguous runs (stream-K), so
//    every CU streams the same number of bytes whatever the shape;
//  - A (the activations) is kept as pre-split bf16 hi + lo fragments; each
//    weight fragment feeds two MFMAs (hi, lo) so products keep ~16 bits of
//    activation precision with fp32 accumulation; A windows are staged in
//    LDS once per workgroup and phase;
//  - a unit whose K range was split between workgroups is finished by the
//    last workgroup to arrive (atomic ticket), which sums the partials in
//    ascending K order: results are deterministic and do not depend on m;
//  - RMSNorm is applied as a row scale after the product
//    ((x * s) . (g * W) = s * ((x * g) . W)); producers of A write x * g.
#include "sv_common.h"
#include "stream_plan.h"

namespace sv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const u4 gu4;
typedef __attribute__((address_space(1))) const uint16_t gu16;
typedef __attribute__((address_space(1))) void gvoid;
typedef __attribute__((address_space(3))) void lvoid;
constexpr int kCpolSc1 = 16;   // cache-policy bit of a direct-to-LDS load: agent-coherent (sc1)
// A generic pointer known to address global memory, as a global-space
// pointer: its accesses then compile to global (not flat) instructions,
// which never hold up the LDS counter.
template <class T>
__device__ __forceinline__ __attribute__((address_space(1))) T* glb(T* p) {
  return (__attribute__((address_space(1))) T*)p;
}

enum Epi : int { EPI_STORE = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_LOGITS = 3, EPI_QKV = 4 };

// ------------------------------------------------------------ small helpers
__device__ __forceinline__ uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ float bf2f(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ f32x4 mfma(const u4& a, const u4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// 8 offset nibbles of one dword (u = q + 8, pairs (2j, 2j+1) at bits 4j and
// 16 + 4j) -> 8 bf16 of value 128 + u = q + 136 (exact: bf16 holds every
// integer below 256).  The constant 136 is taken out after the products:
// sum_k a_k q_k = sum_k a_k (q_k + 136) - 136 sum_k a_k.
constexpr float kInt4Bias = 136.f;
__device__ __forceinline__ u4 nib8_to_bf16(uint32_t d) {
  uint32_t o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) o[j] = ((d >> (4 * j)) & 0x000F000Fu) | 0x43004300u;
  return u4{o[0], o[1], o[2], o[3]};
}

// Data one workgroup writes and another reads later in the same pass is
// stored through to the device-coherent level (agent-scope relaxed atomic
// stores, "sc1"): a signal then needs no L2 write-back, only each wave's
// wait on its own stores.  Buffers rewritten during a pass are read with
// agent-scope loads; buffers written once per pass may be read with plain
// (L2-cached) loads, since no cache can hold an older copy of them.
__device__ __forceinline__ void cst(float* p, float v) {
  __hip_atomic_store(glb(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void cst(int* p, int v) {
  __hip_atomic_store(glb(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void cst16(uint16_t* p, uint16_t v) {
  __hip_atomic_store(glb(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void cst4(float* p, f32x4 v) {   // p 16-byte aligned
  unsigned long long* q = reinterpret_cast<unsigned long long*>(p);
  const unsigned long long a = (unsigned long long)__float_as_uint(v[0]) | (unsigned long long)__float_as_uint(v[1]) << 32;
  const unsigned long long b = (unsigned long long)__float_as_uint(v[2]) | (unsigned long long)__float_as_uint(v[3]) << 32;
  __hip_atomic_store(glb(q), a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(glb(q + 1), b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float cld(const float* p) {
  return __hip_atomic_load(glb(const_cast<float*>(p)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int cld(const int* p) {
  return __hip_atomic_load(glb(const_cast<int*>(p)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ f32x4 cld4(const float* p) {   // p 16-byte aligned
  unsigned long long* q = reinterpret_cast<unsigned long long*>(const_cast<float*>(p));
  const unsigned long long a = __hip_atomic_load(glb(q), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const unsigned long long b = __hip_atomic_load(glb(q + 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return f32x4{__uint_as_float((uint32_t)a), __uint_as_float((uint32_t)(a >> 32)), __uint_as_float((uint32_t)b),
               __uint_as_float((uint32_t)(b >> 32))};
}

// Ready counters: a producer adds one per finished unit of output (after
// its stores are complete); a consumer waits until a counter reaches the
// pass's target (bounded, like the grid barrier: on a timeout it raises
// the error flag and goes on).
__device__ __forceinline__ void ready_add(unsigned long long* c, unsigned long long n = 1) {
  __hip_atomic_fetch_add(glb(c), n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void ready_wait(const unsigned long long* c, unsigned long long target, int* err) {
  unsigned spins = 0;
  while (__hip_atomic_load(glb(const_cast<unsigned long long*>(c)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
    __builtin_amdgcn_s_sleep(1);
    if (++spins == (1u << 24)) {
      __hip_atomic_store(glb(err), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
  }
}

// Element (row, col) of an A operand in hi/lo fragment layout: 32-k chunk
// col/32 holds 128 uint4 (hi[64], lo[64]); lane l of a fragment holds 8
// consecutive k of row l%16 starting at 8*(l/16).
__device__ __forceinline__ void afrag_put(uint4* a, int row, int col, float v) {
  const uint32_t h = f2bf(v);
  const uint32_t l = f2bf(v - bf2f(h));
  const int ch = col >> 5, kk = col & 31;
  const int ln = row + 16 * (kk >> 3), e = kk & 7;
  uint16_t* base = reinterpret_cast<uint16_t*>(a + (long long)ch * 128);
  cst16(base + ln * 8 + e, (uint16_t)h);
  cst16(base + (64 + ln) * 8 + e, (uint16_t)l);
}

// Eight consecutive elements (row, col .. col+7; col a multiple of 8) of an
// A operand: one 16-byte word of the hi fragment and one of the lo fragment,
// each stored through to the device-coherent level as two 64-bit stores.
__device__ __forceinline__ void afrag_put8(uint4* a, int row, int col, const float (&v)[8]) {
  uint32_t hw[4], lw[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t h0 = f2bf(v[2 * e]), h1 = f2bf(v[2 * e + 1]);
    const uint32_t l0 = f2bf(v[2 * e] - bf2f(h0)), l1 = f2bf(v[2 * e + 1] - bf2f(h1));
    hw[e] = h0 | h1 << 16;
    lw[e] = l0 | l1 << 16;
  }
  const int ch = col >> 5, ln = row + 16 * ((col & 31) >> 3);
  unsigned long long* ph = reinterpret_cast<unsigned long long*>(a + (long long)ch * 128 + ln);
  unsigned long long* pl = reinterpret_cast<unsigned long long*>(a + (long long)ch * 128 + 64 + ln);
  __hip_atomic_store(glb(ph), (unsigned long long)hw[0] | (unsigned long long)hw[1] << 32, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(glb(ph + 1), (unsigned long long)hw[2] | (unsigned long long)hw[3] << 32, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(glb(pl), (unsigned long long)lw[0] | (unsigned long long)lw[1] << 32, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(glb(pl + 1), (unsigned long long)lw[2] | (unsigned long long)lw[3] << 32, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

// raw workgroup barrier: execution only; the compiler may not move memory
// operations across it
__device__ __forceinline__ void raw_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Per-workgroup stamp i (0 start, 1 after A staging, 2 after the weight
// stream, 3 end of work) of the current phase; ws is null when off.
__device__ __forceinline__ void wstamp(unsigned long long* ws, int i) {
  if (ws && threadIdx.x == 0) ws[i] = wall_clock64();
}

// ------------------------------------------------------------ grid barrier
// Hierarchical: workgroups arrive on one of 8 group counters (by
// blockIdx % 8, i.e. per XCD under round-robin dispatch), the last of a
// group arrives on the top counter, the last group publishes the
// generation on 8 flags, each workgroup polls its group's flag.  Counters
// are 64-bit and monotonic over the handle's lifetime; the host passes the
// generation reached before the launch.  Layout (u64, 128-byte lines):
// group g at 16*g, top at 128, flag g at 16*(9+g).
//
// No acquire (L2 invalidation) follows the wait.  Data produced in a pass
// and read by another workgroup is stored through to memory (agent-scope
// stores) and read either with agent-scope loads (the residual stream, norm
// partials, split-K partials, attention partials, MoE routing and expert
// outputs) or from addresses written once per pass (the per-site A
// operands, per-layer query fragments and cache rows), which no XCD's L2
// can hold from earlier in the pass since the L2s start every launch
// invalidated.
struct GridBar {
  unsigned long long* bar;
  unsigned long long gen;
  int* err;          // set to 1 if a wait ran out (the pass then skips all later waits)
  bool aborted;
};

// ~2^24 polls of 64 cycles: about half a second at 2.4 GHz, far beyond any
// legitimate wait
constexpr unsigned kSpinLimit = 1u << 24;

// Every wave's global writes must be complete before the workgroup's one
// signalling thread publishes them: the workgroup barrier does not wait for
// other waves' outstanding stores.  Each wave waits for its own memory
// operations (completed stores sit in the L2), then the signalling thread's
// agent-scope release makes the L2 contents visible device-wide.  (A
// per-wave agent release instead costs about three times as much per grid
// barrier: every wave then writes back the L2.)
__device__ __forceinline__ void release_all_waves() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

template <class PF>
__device__ __forceinline__ void grid_sync(GridBar& gb, PF&& prefetch) {
  release_all_waves();
  __syncthreads();
  ++gb.gen;
  if (threadIdx.x == 0) {
    const unsigned g = blockIdx.x & 7u;
    const unsigned long long ng = (gridDim.x - g + 7u) / 8u;
    const unsigned long long ngr = gridDim.x < 8 ? gridDim.x : 8;
    // (no release fence: the phase's shared data was stored through, and
    // every wave waited for its stores before the workgroup barrier)
    const unsigned long long old =
        __hip_atomic_fetch_add(glb(gb.bar + 16 * g), 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old == gb.gen * ng - 1) {
      const unsigned long long o2 =
          __hip_atomic_fetch_add(glb(gb.bar + 128), 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (o2 == gb.gen * ngr - 1) {
        for (int x = 0; x < 8; ++x)
          __hip_atomic_store(glb(gb.bar + 16 * (9 + x)), gb.gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  // weight loads of the next phase go out after the arrival, so they stream
  // during the wait (wave 0 drains its own at its first poll)
  prefetch();
  if (threadIdx.x == 0 && !gb.aborted) {
    const unsigned g = blockIdx.x & 7u;
    unsigned spins = 0;
    while (__hip_atomic_load(glb(gb.bar + 16 * (9 + g)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < gb.gen) {
      __builtin_amdgcn_s_sleep(1);
      if (++spins == kSpinLimit) {
        gb.aborted = true;
        __hip_atomic_store(glb(gb.err), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
  }
  raw_barrier();
}

// ------------------------------------------------------------ control area
// (the LDS plan is in the shared header)
struct Ctl {
  float rs[16];                 // RMSNorm row scales of the current phase
  int pend_n;                   // split units this workgroup flushed in the phase
  int pend[kMaxPending];        // split unit blocks flushed: slot << 20 | sg
  int uc;                       // MoE: union size
  int ulist[256];               // MoE: union (expert ids, ascending)
  int misc[8];
};
static_assert(sizeof(Ctl) <= kCtlBytes, "control area overflows its LDS slot");

__device__ __forceinline__ Ctl* ctl(unsigned char* smem, size_t lds) {
  return reinterpret_cast<Ctl*>(smem + lds - kCtlBytes);
}

// ------------------------------------------------------------ GEMM phase
template <int WF, int TPU>
struct Fmt {
  static constexpr int FPC = TPU * (WF == W_F32 ? 2 : 1);   // ring slots per chunk
  static constexpr int U = batch_chunks(WF, TPU);           // chunks per batch
  static constexpr int ACH = a_chunks(WF);                  // 32-k A chunks per weight chunk
};

// One batch of weight fragments per wave (int4 scales travel with their
// fragments, so the compute loop never waits on another global load).
// A wave computes on a batch, then issues the next one; the four waves of a
// CU keep 4 x 32 KB in flight while they wait.
struct Ring {
  u4 r[kRing];
  uint32_t s[kRing];   // int4: fp16 scale bits of each fragment's column
};

struct SlotMap {
  const int* ulist;   // MoE union list in LDS (null: dense phase, one slot)
  int uc, n_experts, n_slots;
};

// Load cursor: walks the range batch by batch (batches never cross a
// segment, i.e. one (slot, win, sg) run of chunks).
struct LCur {
  Cur q;
  bool done;
};

// Loads the next batch (up to U chunks of the current segment) into the ring;
// slots past the batch are zero (never read).  An idle wave (unit past the
// matrix) loads nothing: its ring is zero and its compute is skipped, so the
// ring is provably rewritten by every batch and dead between phases.
template <int WF, int TPU>
__device__ __forceinline__ void next_batch(const Mat& M, const Lin& L, LCur& l, int u1, Ring& ring) {
  using F = Fmt<WF, TPU>;
  if (l.done) return;
  const Cur& q = l.q;
  const int n = min(F::U, seg_left(q, u1));
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool live = q.sg * kWaves + wave < M.n_units;
  const long long fi0 = (((long long)q.sg * M.nkc + (long long)q.win * M.win + q.c) * kWaves + wave) * TPU;
  const char* wb = static_cast<const char*>(M.w) + (long long)q.e * M.w_stride + fi0 * 1024 + lane * 16;
  const char* wb2 = static_cast<const char*>(M.w2) + (long long)q.e * M.w2_stride;
  constexpr int RPC = TPU * (WF == W_F32 ? 2 : 1);   // ring slots per chunk
#pragma unroll
  for (int i = 0; i < F::U; ++i) {
    if (live && i < n) {   // (wave-uniform)
#pragma unroll
      for (int t = 0; t < TPU; ++t) {
        const long long fo = ((long long)i * kWaves * TPU + t) * 1024;
        if constexpr (WF == W_F32) {
          ring.r[(i * TPU + t) * 2 + 0] = __builtin_nontemporal_load((gu4*)(wb + fo));
          ring.r[(i * TPU + t) * 2 + 1] = __builtin_nontemporal_load((gu4*)(wb2 + fi0 * 1024 + lane * 16 + fo));
        } else {
          ring.r[i * TPU + t] = __builtin_nontemporal_load((gu4*)(wb + fo));
          if constexpr (WF == W_INT4) {
            // raw fp16 bits: converting here would wait on the load (and,
            // with in-order load counting, on every load before it)
            const gu16* sp = (gu16*)(wb2 + (fi0 + (long long)i * kWaves * TPU + t) * 32 + (lane & 15) * 2);
            ring.s[i * TPU + t] = *sp;
          }
        }
      }
    } else {
#pragma unroll
      for (int t = 0; t < RPC; ++t) ring.r[i * RPC + t] = u4{0u, 0u, 0u, 0u};
      if constexpr (WF == W_INT4) {
#pragma unroll
        for (int t = 0; t < TPU; ++t) ring.s[i * TPU + t] = 0u;
      }
    }
  }
  batch_advance(L, l.q, n, u1, l.done);
}

// What a GEMM phase reads and writes besides the weights.
struct GemmIO {
  const uint4* a;            // A operand (hi/lo fragments)
  long long a_slot;          // uint4 per slot (0: shared by all slots)
  float* out; int ldo; long long out_slot;   // STORE / LOGITS outputs
  int scale;                 // STORE: multiply by the RMSNorm row scale
  const float* gain;         // RESID: gain of the next norm
  uint4* a_out; long long a_out_slot;        // RESID / SWIGLU: next A operand
  float* trace;              // RESID: residual copy for this layer (nullable)
  void* kv;                  // QKV: the layer's cache pages
  unsigned long long* ready;  // this layer's ready counters
  int dep, notify;            // DepKind of the inputs / outputs
  const float* ss_in;         // sum-of-squares partials of the input's norm
  float* ss_out;              // RESID: partials of the next norm
  float* ws; unsigned* tickets;   // the phase's split-K workspace bank
};

// Query element (block row j, query head h, dim d), already rotated and
// scaled, into the attention's MFMA A fragments: per KV head g = h / G,
// row r = j * G + h % G of row tile r / 16, 32-dim chunk d / 32, hi and lo
// bf16 parts; lane (r % 16) + 16 * ((d % 32) / 8) holds 8 consecutive dims.
__device__ __forceinline__ void qfrag_put(const PassP& P, uint4* qf, int h, int j, int d, float v) {
  const int g = h / P.G, r = j * P.G + (h - g * P.G);
  const int KDC = P.D >> 5;
  const long long f = (((long long)g * P.qf_rt + (r >> 4)) * KDC + (d >> 5)) * 2;   // hi fragment
  const int ln = (r & 15) + 16 * ((d & 31) >> 3), e = d & 7;
  uint16_t* q = reinterpret_cast<uint16_t*>(qf);
  const uint32_t hb = f2bf(v);
  cst16(q + (f * 64 + ln) * 8 + e, (uint16_t)hb);
  cst16(q + ((f + 1) * 64 + ln) * 8 + e, (uint16_t)f2bf(v - bf2f(hb)));
}

// one cache element, rounded to the cache dtype
template <bool KVF32>
__device__ __forceinline__ void kv_put(void* kv, long long i, float v) {
  if constexpr (KVF32) cst(static_cast<float*>(kv) + i, v);
  else cst16(static_cast<uint16_t*>(kv) + i, (uint16_t)f2bf(v));
}

// Rotary factors and cache pages of one QKV unit's rows (they depend only
// on the unit, so a reducer loads them before it waits for the partials).
struct QkvPre {
  float cs[4], sn[4];
  long long pg[4];
};
template <bool GEN>
__device__ __forceinline__ void qkv_pre(const PassP& P, int unit, QkvPre& q) {
  const int lane = threadIdx.x & 63;
  const int col = unit * kTileN + (lane & 15), rg = lane >> 4;
  const int D = P.D, H = D >> 1;
  const int qc = P.Hq * D, kc = P.Hkv * D;
  const bool rot_col = col < qc + kc;
  const int c2 = col < qc ? col : col - qc;
  const int ii = (c2 % D) >> 1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = min(4 * rg + i, P.m - 1);
    const int t = GEN && P.row_slot ? P.row_slot[row] : P.L + row;   // cache slot
    const int tp = GEN && P.row_rope ? P.row_rope[row] : t;          // rotary position
    q.pg[i] = (long long)P.page_table[t / kPage] * P.Hkv;
    q.cs[i] = rot_col ? P.rope_cs[((long long)tp * H + ii) * 2 + 0] : 0.f;
    q.sn[i] = rot_col ? P.rope_cs[((long long)tp * H + ii) * 2 + 1] : 0.f;
  }
}

// Epilogue of one finished unit (one wave, acc[t] = tile t of the unit).
// QKV takes the unit's rotary factors and pages (qkv_pre).
template <int WF, int EPI, int TPU, bool GEN>
__device__ __forceinline__ void epilogue(const PassP& P, const Mat& M, const GemmIO& io, const float* rs, int slot,
                                         int unit, f32x4 (&acc)[TPU], const QkvPre* qp = nullptr) {
  // the lane index is made opaque here, so the compiler cannot hoist the
  // per-row addresses below out of a stream loop (they would stay live, and
  // spill, across the whole loop)
  int lane = threadIdx.x & 63;
  asm volatile("" : "+v"(lane));
  const int cl = lane & 15, rg = lane >> 4;
  if constexpr (EPI == EPI_STORE) {
    const int col = unit * kTileN + cl;
    float* out = io.out + (long long)slot * io.out_slot;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * rg + i;
      if (row < P.m && col < M.N) cst(out + (long long)row * io.ldo + col, io.scale ? rs[row] * acc[0][i] : acc[0][i]);
    }
  } else if constexpr (EPI == EPI_RESID) {
    const int col = unit * kTileN + cl;
    // every load first (the stores below could alias later loads)
    float xv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * rg + i;
      xv[i] = (row < P.m && col < M.N) ? cld(P.x + (long long)row * P.ldx + col) : 0.f;
    }
    const float gn = col < M.N ? *glb(io.gain + col) : 0.f;
    float sq[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * rg + i;
      float v = 0.f;
      if (row < P.m && col < M.N) {
        v = xv[i] + acc[0][i];
        cst(P.x + (long long)row * P.ldx + col, v);
        if (io.trace) io.trace[(long long)row * P.d + col] = v;
      }
      sq[i] = v * v;
      if (col < M.N) afrag_put(io.a_out, row, col, v * gn);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) sq[i] += __shfl_xor(sq[i], o, 64);
    }
    if (cl == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 4 * rg + i;
        if (row < P.m) cst(io.ss_out + row * P.n_ss + unit, sq[i]);
      }
    }
  } else if constexpr (EPI == EPI_QKV) {
    // RMSNorm row scale, then the rotary embedding of query and key columns
    // (pairs side by side: the partner is the neighbouring lane); queries,
    // scaled by 1/sqrt(D), go to the attention's fragments, keys and values
    // (rounded to the cache dtype) to the cache at positions L .. L+m-1
    const int col = unit * kTileN + cl;
    const int D = P.D, H = D >> 1;
    const int qc = P.Hq * D, kc = P.Hkv * D;
    const bool rot_col = col < qc + kc;
    const int c2 = col < qc ? col : (rot_col ? col - qc : col - qc - kc);
    const int head = c2 / D, p = c2 - head * D, ii = p >> 1, odd = p & 1;
    const float* cs = qp->cs;
    const float* sn = qp->sn;
    const long long* pg = qp->pg;
    float v[4], pv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * rg + i;
      v[i] = rs[row] * acc[0][i];
      pv[i] = __shfl_xor(v[i], 1, 64);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * rg + i;
      if (row < P.m && col < M.N) {
        const int t = GEN && P.row_slot ? P.row_slot[row] : P.L + row;
        if (rot_col) {
          const float a = odd ? pv[i] : v[i], b = odd ? v[i] : pv[i];   // x[ii], x[ii + H]
          const float rot = odd ? (b * cs[i] + a * sn[i]) : (a * cs[i] - b * sn[i]);
          const int dd = ii + odd * H;
          if (col < qc) qfrag_put(P, io.a_out, head, row, dd, rot * P.attn_scale);
          else kv_put<WF == W_F32>(io.kv, ((pg[i] + head) * 2 + 0) * kPage * D + (long long)(t % kPage) * D + dd, rot);
        } else {
          kv_put<WF == W_F32>(io.kv, ((pg[i] + head) * 2 + 1) * kPage * D + (long long)p * kPage + (t % kPage), v[i]);
        }
      }
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    const int col = unit * kTileN + cl;   // activation column
    uint4* a_out = io.a_out + (long long)slot * io.a_out_slot;
    if (col < M.N) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 4 * rg + i;
        float a = 0.f;
        if (row < P.m) {
          const float g = rs[row] * acc[0][i];
          const float u = rs[row] * acc[TPU - 1][i];
          a = g / (1.0f + expf(-g)) * u;
        }
        afrag_put(a_out, row, col, a);
      }
    }
  } else {  // EPI_LOGITS
    const int col = unit * kTileN + cl;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * rg + i;
      const bool ok = row < P.m && col < M.N;
      const float v = rs[row] * acc[0][i];
      if (ok) *glb(io.out + (long long)row * io.ldo + col) = v;
      float mx = ok ? v : -INFINITY;
      int ix = ok ? col : 0x7fffffff;
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        const float om = __shfl_xor(mx, o, 64);
        const int oi = __shfl_xor(ix, o, 64);
        if (om > mx || (om == mx && oi < ix)) { mx = om; ix = oi; }
      }
      float e = (ok && mx != -INFINITY) ? expf(v - mx) : 0.f;
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) e += __shfl_xor(e, o, 64);
      if (cl == 0 && row < P.m) {
        P.st_max[row * P.n_stat + unit] = mx;
        P.st_sum[row * P.n_stat + unit] = e;
        P.st_idx[row * P.n_stat + unit] = ix;
      }
    }
  }
}

// Row scales 1/sqrt(mean(x^2) + eps) from the sum-of-squares partials, in
// a fixed order (identical in every workgroup).
__device__ __forceinline__ void row_scales(const PassP& P, const float* ss, float* rs) {
  const int t = threadIdx.x;
  const int row = t >> 4, j = t & 15;   // 16 rows x 16 lanes
  constexpr int B = 16;                 // loads in flight per lane
  const float* src = ss + row * P.n_ss;
  float s = 0.f;
  if (row < P.m) {
    for (int i0 = j; i0 < P.n_ss; i0 += 16 * B) {
      float v[B];
#pragma unroll
      for (int q = 0; q < B; ++q) {
        const int i = i0 + 16 * q;
        v[q] = i < P.n_ss ? cld(src + i) : 0.f;
      }
#pragma unroll
      for (int q = 0; q < B; ++q) s += v[q];
    }
  }
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) s += __shfl_xor(s, o, 64);
  if (j == 0) rs[row] = row < P.m ? 1.0f / sqrtf(s * P.inv_d + P.eps) : 0.f;
}

// Stages the A window of block (slot, win) into LDS window slot `ws`.
// Stages the A window of block (slot, win) into LDS with direct
// global-to-LDS loads (lane l of a wave writes its 16 bytes at base + 16 l):
// every load is in flight at once and no registers are used.  The caller
// waits (s_waitcnt) and synchronises before reading the window.  The
// window holds a multiple of 128 words, so each wave's 64-word block lies
// wholly inside it.
template <int WF>
__device__ __forceinline__ void stage_window(const Lin& L, const GemmIO& io, int slot, int win, unsigned char* smem,
                                             int m) {
  constexpr int ACH = (WF == W_INT4) ? 4 : 1;
  const int n16 = L.wlen(win) * ACH * 128;    // 16-byte words to copy
  const uint4* src = io.a + (long long)slot * io.a_slot + (long long)win * L.W * ACH * 128;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // lane l of every 64-word block carries row l % 16: rows past the block's
  // m are not loaded (what LDS holds there only reaches output rows that
  // nothing reads)
  if ((lane & 15) < m)
    for (int i0 = wave * 64; i0 < n16; i0 += kThreads)
      __builtin_amdgcn_global_load_lds((gvoid*)(src + i0 + lane), (lvoid*)(smem + (size_t)i0 * 16), 16, 0, 0);
}

// int4: per 128-k chunk of the staged window and per row, the sum of the A
// operand (hi + lo) over the chunk's k, for the offset correction
// (kInt4Bias); [chunk][16 rows] floats after the window.  Called by the whole
// workgroup after the window's loads are complete and visible.
__device__ __forceinline__ void int4_rowsums(const unsigned char* smem, int nch, float* S) {
  const int t = threadIdx.x;
  const int ai = t >> 4, row = t & 15;   // 256 threads: 16 chunks x 16 rows
  if (ai < nch) {
    const uint4* aw = reinterpret_cast<const uint4*>(smem) + (long long)ai * 4 * 128;
    float sum = 0.f;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
      for (int kg = 0; kg < 4; ++kg) {
        const uint4 h = aw[q4 * 128 + row + 16 * kg], l = aw[q4 * 128 + 64 + row + 16 * kg];
        const uint32_t hw[4] = {h.x, h.y, h.z, h.w}, lw[4] = {l.x, l.y, l.z, l.w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          sum += (bf2f(hw[e] & 0xFFFFu) + bf2f(lw[e] & 0xFFFFu)) + (bf2f(hw[e] >> 16) + bf2f(lw[e] >> 16));
      }
    S[ai * 16 + row] = sum;
  }
  __syncthreads();
}

// Dependency bookkeeping of the dataflow edges (one 64-column block of a
// phase's output = one supergroup).
// KV head of the QKV output block starting at column c0.
__device__ __forceinline__ int qkv_block_head(const PassP& P, int c0) {
  const int qc = P.Hq * P.D, kc = P.Hkv * P.D;
  if (c0 < qc) return (c0 / P.D) / P.G;
  return c0 < qc + kc ? (c0 - qc) / P.D : (c0 - qc - kc) / P.D;
}
// QKV blocks feeding one KV head's attention: its G query heads, key, value.
__device__ __forceinline__ unsigned long long heads_expect(const PassP& P) {
  return (unsigned long long)(P.G + 2) * (P.D / 64);
}
// O-input window w: the query heads whose columns meet it.
__device__ __forceinline__ unsigned long long owin_expect(const PassP& P, int w) {
  const int c0 = w * P.o_wcols, c1 = min(c0 + P.o_wcols, P.Hq * P.D);
  return (unsigned long long)((c1 - 1) / P.D - c0 / P.D + 1);
}
// announces a finished output block (stores complete) of a producing phase
__device__ __forceinline__ void notify_block(const PassP& P, const GemmIO& io, int sg) {
  if (io.notify == kDepHeads) ready_add(io.ready + qkv_block_head(P, sg * 64));
}
// waits (workgroup-wide) until the input window win of a consuming phase is ready
__device__ __forceinline__ void wait_window(const PassP& P, const GemmIO& io, int win) {
  if (io.dep == kDepOWin) {
    if (threadIdx.x == 0) ready_wait(io.ready + kRdyOWin + win, P.epoch * owin_expect(P, win), P.err);
    __syncthreads();
  }
}

// One weight-streaming phase over `sm.n_slots` slots (experts) of M.
// FIXED: the fixed-order split-K of the expert phases (seg_info_fixed):
// every piece (one batch) is summed from zero and added to the block's
// running chain in K order, so the result does not depend on how the
// routed union's size cuts the work.
template <int WF, int EPI, int TPU, bool GEN, bool FIXED = false>
__device__ __forceinline__ void gemm_phase(const PassP& P, const Mat M, const GemmIO io, const SlotMap sm,
                                        bool slot_major, Ring& ring, unsigned char* smem, unsigned long long* wst,
                                        bool staged = false) {
  using F = Fmt<WF, TPU>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = gridDim.x, g = blockIdx.x;
  Ctl* C = ctl(smem, (size_t)P.lds_bytes);
  const Lin L = make_lin(M, sm.n_slots, slot_major, sm.ulist, sm.uc, sm.n_experts);
  const int u0 = run_begin(L, g, G), u1 = run_begin(L, g + 1, G);

  if (threadIdx.x == 0) C->pend_n = 0;
  // the A window of the range's first block (a range that crosses into
  // another (key, window) restages: a few workgroups per phase), with the
  // row scales' loads in flight at the same time
  // (staged: window 0 of a shared A and its row scales are already in LDS)
  int sk = -1, sw = -1;
  if (u0 < u1) {
    const Cur a = cur_at(L, u0);
    sk = slot_major ? a.slot : 0;
    sw = a.win;
    if (!(staged && sk == 0 && sw == 0)) {
      wait_window(P, io, sw);
      stage_window<WF>(L, io, sk, sw, smem, P.m);
    }
  }
  if ((EPI == EPI_SWIGLU || EPI == EPI_LOGITS || EPI == EPI_QKV || (EPI == EPI_STORE && io.scale)) && !staged)
    row_scales(P, io.ss_in, C->rs);
  __builtin_amdgcn_s_waitcnt(0);   // the window's direct loads
  __syncthreads();
  float* const S4 = reinterpret_cast<float*>(smem + kAWindowBytes);   // int4 row sums
  if constexpr (WF == W_INT4) {
    if (u0 < u1) int4_rowsums(smem, L.wlen(sw), S4);
  }
  wstamp(wst, 1);
  if (u0 >= u1) {
    wstamp(wst, 2);
    return;
  }

  // the caller issued the first batch (gemm_prefetch); advance the load
  // cursor past it
  LCur lc;
  lc.q = cur_at(L, u0);
  lc.done = false;
  batch_advance(L, lc.q, min(F::U, seg_left(lc.q, u1)), u1, lc.done);

  Cur cc = cur_at(L, u0);
  f32x4 acc[TPU];

  // one batch of n chunks starting at window chunk c0.  Ring slots past n
  // hold zeros (next_batch) and read a valid, finite A chunk, so they add
  // exact zeros.  bf16 / fp32: the A fragments of the next group of GR
  // chunks are read from LDS while the current group's MFMAs run (the
  // scheduling barriers keep exactly one group in flight: bounded registers,
  // hidden LDS latency).
  auto compute = [&](int c0, int n, bool live) {
    if (!live) return;
    const uint4* aw = reinterpret_cast<const uint4*>(smem) + (long long)c0 * F::ACH * 128;
    if constexpr (WF == W_INT4) {
      // The A fragments (and row sums) of chunk i + 1 are read from LDS
      // while chunk i's MFMAs run, and chunk i's scaled, offset-corrected
      // sum is added once chunk i + 1's MFMAs are issued (its result is
      // ready by then); acc still takes the chunks in order.
      u4 ch[4], cl[4], nh[4], nl[4];
      f32x4 crs, nrs, prs = f32x4{0.f, 0.f, 0.f, 0.f};
      f32x4 pg[TPU];
      uint32_t psc[TPU];
      auto read_chunk = [&](int i, u4 (&h)[4], u4 (&l)[4], f32x4& rs) {
        const int ai = i < n ? i : 0;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          h[q4] = __builtin_bit_cast(u4, aw[(ai * 4 + q4) * 128 + lane]);
          l[q4] = __builtin_bit_cast(u4, aw[(ai * 4 + q4) * 128 + 64 + lane]);
        }
        // this lane's four rows: 4 (lane / 16) .. +3
        rs = *reinterpret_cast<const f32x4*>(S4 + (c0 + ai) * 16 + 4 * (lane >> 4));
      };
      auto fold = [&]() {
#pragma unroll
        for (int t = 0; t < TPU; ++t) {
          const float sc = (float)__builtin_bit_cast(_Float16, (uint16_t)psc[t]);
          acc[t] += sc * (pg[t] - kInt4Bias * prs);
        }
      };
      read_chunk(0, ch, cl, crs);
#pragma unroll
      for (int i = 0; i < F::U; ++i) {
        if (i + 1 < F::U) read_chunk(i + 1, nh, nl, nrs);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_sched_barrier(0);
        f32x4 gacc[TPU];
#pragma unroll
        for (int t = 0; t < TPU; ++t) gacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
#pragma unroll
          for (int t = 0; t < TPU; ++t) {
            const u4 wv = nib8_to_bf16(ring.r[i * TPU + t][q4]);
            gacc[t] = mfma(ch[q4], wv, gacc[t]);
            gacc[t] = mfma(cl[q4], wv, gacc[t]);
          }
        }
        if (i > 0) fold();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < TPU; ++t) {
          pg[t] = gacc[t];
          psc[t] = ring.s[i * TPU + t];
        }
        prs = crs;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          ch[q4] = nh[q4];
          cl[q4] = nl[q4];
        }
        crs = nrs;
      }
      fold();
    } else {
      constexpr int GR = 4;   // chunks per group
      static_assert(F::U % GR == 0, "batch not a whole number of groups");
      u4 ch[GR], cl[GR], nh[GR], nl[GR];
      auto read_group = [&](int g0, u4 (&h)[GR], u4 (&l)[GR]) {
#pragma unroll
        for (int j = 0; j < GR; ++j) {
          const int ai = g0 + j < n ? g0 + j : 0;
          h[j] = __builtin_bit_cast(u4, aw[ai * 128 + lane]);
          l[j] = __builtin_bit_cast(u4, aw[ai * 128 + 64 + lane]);
        }
      };
      read_group(0, ch, cl);
#pragma unroll
      for (int g0 = 0; g0 < F::U; g0 += GR) {
        if (g0 + GR < F::U) read_group(g0 + GR, nh, nl);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < GR; ++j) {
          const int i = g0 + j;
#pragma unroll
          for (int t = 0; t < TPU; ++t) {
            if constexpr (WF == W_F32) {
              const u4 wh = ring.r[(i * TPU + t) * 2 + 0], wl = ring.r[(i * TPU + t) * 2 + 1];
              acc[t] = mfma(ch[j], wh, acc[t]);
              acc[t] = mfma(cl[j], wh, acc[t]);
              acc[t] = mfma(ch[j], wl, acc[t]);
              acc[t] = mfma(cl[j], wl, acc[t]);
            } else {
              const u4 wv = ring.r[i * TPU + t];
              acc[t] = mfma(ch[j], wv, acc[t]);
              acc[t] = mfma(cl[j], wv, acc[t]);
            }
          }
        }
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < GR; ++j) {
          ch[j] = nh[j];
          cl[j] = nl[j];
        }
      }
    }
  };


  for (;;) {
    // ---- one segment: (slot, win, sg), chunks [cc.c, cc.c + nch)
    const int nch = seg_left(cc, u1);
    const bool live = cc.sg * kWaves + wave < M.n_units;
    int idx, nseg;
    if constexpr (!FIXED) {
#pragma unroll
      for (int t = 0; t < TPU; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int c0 = 0; c0 < nch; c0 += F::U) {
        const int n = min(F::U, nch - c0);
        compute(cc.c + c0, n, live);
        next_batch<WF, TPU>(M, L, lc, u1, ring);
      }
      cc.u += nch;
      cc.c += nch;
      // ---- flush the segment: epilogue if it covers the whole unit, else a
      // partial for the last arriver
      seg_info(L, cc.slot, cc.sg, cc.win, g, G, idx, nseg);
      if (live) {
        if (nseg == 1) {
          QkvPre qp;
          if constexpr (EPI == EPI_QKV) qkv_pre<GEN>(P, cc.sg * kWaves + wave, qp);
          epilogue<WF, EPI, TPU, GEN>(P, M, io, C->rs, cc.slot, cc.sg * kWaves + wave, acc, &qp);
        } else {
          float* p = io.ws + ((((long long)cc.slot * M.n_sg + cc.sg) * M.max_seg + idx) * kWaves + wave) * TPU * 256;
#pragma unroll
          for (int t = 0; t < TPU; ++t) cst4(p + t * 256 + lane * 4, acc[t]);
        }
      }
      // split segments (and, for producing phases, blocks finished here) are
      // listed; bit 31 marks a finished block
      if ((nseg > 1 || io.notify) && threadIdx.x == 0) {
        const int k = C->pend_n;   // capacity guaranteed by the host (kMaxPending)
        C->pend[k] = (nseg > 1 ? 0 : (int)0x80000000u) | cc.slot << 20 | cc.sg;
        C->pend_n = k + 1;
      }
    } else {
      // fixed order: every batch (one piece) from zero; a segment holding the
      // block's first piece adds them to its running chain (kept per lane in
      // LDS, not live in registers across the batch's MFMAs) and hands the
      // chain over as partial 0; a later segment hands over each piece
      seg_info_fixed(L, cc.slot, cc.sg, cc.win, g, G, idx, nseg);
      auto part = [&](int i) {   // this wave's slot of partial i of the block
        return io.ws + ((((long long)cc.slot * M.n_sg + cc.sg) * M.max_seg + i) * kWaves + wave) * TPU * 256;
      };
      f32x4* const chain = reinterpret_cast<f32x4*>(smem + kChainBase) + wave * TPU * 64 + lane;
#pragma unroll
      for (int t = 0; t < TPU; ++t) chain[t * 64] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int c0 = 0; c0 < nch; c0 += F::U) {
        const int n = min(F::U, nch - c0);
#pragma unroll
        for (int t = 0; t < TPU; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        compute(cc.c + c0, n, live);
        next_batch<WF, TPU>(M, L, lc, u1, ring);
        if (idx == 0) {
#pragma unroll
          for (int t = 0; t < TPU; ++t) chain[t * 64] = chain[t * 64] + acc[t];
        } else if (live) {
          float* p = part(idx + c0 / F::U);
#pragma unroll
          for (int t = 0; t < TPU; ++t) cst4(p + t * 256 + lane * 4, acc[t]);
        }
      }
      cc.u += nch;
      cc.c += nch;
      if (live && idx == 0) {
#pragma unroll
        for (int t = 0; t < TPU; ++t) acc[t] = chain[t * 64];
        if (nseg == 1) {
          QkvPre qp;
          epilogue<WF, EPI, TPU, GEN>(P, M, io, C->rs, cc.slot, cc.sg * kWaves + wave, acc, &qp);
        } else {
          float* p = part(0);
#pragma unroll
          for (int t = 0; t < TPU; ++t) cst4(p + t * 256 + lane * 4, acc[t]);
        }
      }
      // one list entry per partial handed over (bit 31: a block finished here)
      if ((nseg > 1 || io.notify) && threadIdx.x == 0) {
        const int nparts = nseg > 1 && idx > 0 ? (nch + F::U - 1) / F::U : 1;
        int k = C->pend_n;   // capacity guaranteed by the host (kMaxPending)
        for (int i = 0; i < nparts; ++i) C->pend[k++] = (nseg > 1 ? 0 : (int)0x80000000u) | cc.slot << 20 | cc.sg;
        C->pend_n = k;
      }
    }
    if (cc.u >= u1) break;
    seg_advance(L, cc);
    const int key = slot_major ? cc.slot : 0;
    if (key != sk || cc.win != sw) {
      __syncthreads();   // every wave is done with the staged window
      sk = key;
      sw = cc.win;
      wait_window(P, io, sw);
      stage_window<WF>(L, io, sk, sw, smem, P.m);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if constexpr (WF == W_INT4) int4_rowsums(smem, L.wlen(sw), S4);
    }
  }

  wstamp(wst, 2);
  // ---- split blocks.  The partials of a block are summed in K order and
  // the epilogue applied (by whichever workgroup reduces it: the result is
  // the same bit for bit).
  release_all_waves();
  __syncthreads();
  const int np = C->pend_n;
  constexpr int RB = TPU == 1 ? 16 : 8;   // partial loads in flight per lane (a block's usual count)
  auto pre = [&](int sg, QkvPre& qp) {   // QKV: rotary factors and cache pages of the block's rows
    if constexpr (EPI == EPI_QKV) {
      if (sg * kWaves + wave < M.n_units) qkv_pre<GEN>(P, sg * kWaves + wave, qp);
    }
  };
  auto reduce = [&](int s, int sg, int n, const QkvPre& qp) {
    const int unit = sg * kWaves + wave;
    if (unit < M.n_units) {
      f32x4 sum[TPU];
#pragma unroll
      for (int t = 0; t < TPU; ++t) sum[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      const float* p = io.ws + ((((long long)s * M.n_sg + sg) * M.max_seg) * kWaves + wave) * TPU * 256 + lane * 4;
      for (int j0 = 0; j0 < n; j0 += RB) {
        f32x4 v[RB][TPU];
#pragma unroll
        for (int q = 0; q < RB; ++q) {
#pragma unroll
          for (int t = 0; t < TPU; ++t)
            v[q][t] = j0 + q < n ? cld4(p + (long long)(j0 + q) * kWaves * TPU * 256 + t * 256)
                                 : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int q = 0; q < RB; ++q) {
          if (j0 + q < n) {
#pragma unroll
            for (int t = 0; t < TPU; ++t) sum[t] += v[q][t];
          }
        }
      }
      epilogue<WF, EPI, TPU, GEN>(P, M, io, C->rs, s, unit, sum, &qp);
    }
    if (io.notify) {
      release_all_waves();
      __syncthreads();
      if (threadIdx.x == 0) notify_block(P, io, sg);
    }
  };
  // every workgroup announces its segments (no waiting), then reduces the
  // blocks assigned to it (an even share of all blocks) once every segment
  // of the block is in
  for (int k = threadIdx.x; k < np; k += kThreads) {
    const int e = C->pend[k];
    const int s = (e >> 20) & 0x7ff, sg = e & 0xfffff;
    if (e < 0) notify_block(P, io, sg);
    else __hip_atomic_fetch_add(glb(io.tickets + (long long)s * M.n_sg + sg), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  const int nb = L.n_slots * M.n_sg;
  const int b0 = range_begin(nb, g, G), b1 = range_begin(nb, g + 1, G);
  for (int b = b0; b < b1; ++b) {
    const int s = b / M.n_sg, sg = b - s * M.n_sg;
    int idx, n;
    if constexpr (FIXED) seg_info_fixed(L, s, sg, 0, g, G, idx, n);
    else seg_info(L, s, sg, 0, g, G, idx, n);
    if (n == 1) continue;   // finished inside the stream
    QkvPre qp;
    pre(sg, qp);            // (its loads in flight while polling)
    if (threadIdx.x == 0) {
      unsigned* t = io.tickets + b;
      unsigned spins = 0;
      while (__hip_atomic_load(glb(t), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < (unsigned)n) {
        __builtin_amdgcn_s_sleep(1);
        if (++spins == kSpinLimit) {
          __hip_atomic_store(glb(P.err), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
      }
      __hip_atomic_store(glb(t), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();   // the partials are read with agent-scope loads
    reduce(s, sg, n, qp);
  }
}

// Issues the first two weight batches of a GEMM phase (before the grid
// barrier that precedes it, so they stream during the wait).  An empty
// range loads nothing and the phase returns before using the ring.
template <int WF, int TPU>
__device__ __forceinline__ void gemm_prefetch(const Mat M, const SlotMap sm, bool slot_major, Ring& ring) {
  const int G = gridDim.x, g = blockIdx.x;
  const Lin L = make_lin(M, sm.n_slots, slot_major, sm.ulist, sm.uc, sm.n_experts);
  const int u0 = run_begin(L, g, G), u1 = run_begin(L, g + 1, G);
  if (u0 >= u1) {
#pragma unroll
    for (int i = 0; i < kRing; ++i) {   // nothing to stream: a defined, unused ring
      ring.r[i] = u4{0u, 0u, 0u, 0u};
      ring.s[i] = 0u;
    }
    return;
  }
  LCur lc;
  lc.q = cur_at(L, u0);
  lc.done = false;
  next_batch<WF, TPU>(M, L, lc, u1, ring);
}

// ------------------------------------------------------------ embedding
// x[j] = E[t_j]; A operand x * gain0; sum-of-squares partials per 16 columns.
__device__ __forceinline__ void embed_phase(const PassP& P, bool emb_f32, uint4* a_out, float* ss_out) {
  const int n_tiles = (P.d + 15) / 16;
  const int t = threadIdx.x;
  const int row = t >> 4, cl = t & 15;
  for (int tile = blockIdx.x; tile < n_tiles; tile += gridDim.x) {
    if (t >= 256) continue;
    const int col = tile * 16 + cl;
    float v = 0.f;
    if (row < P.m && col < P.d) {
      const long long tok = P.tokens[row];
      v = emb_f32 ? static_cast<const float*>(P.embed)[tok * P.d + col]
                  : bf2f(static_cast<const uint16_t*>(P.embed)[tok * P.d + col]);
      cst(P.x + (long long)row * P.ldx + col, v);
    }
    if (col < P.d) afrag_put(a_out, row, col, v * P.gain0[col]);
    float sq = v * v;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) sq += __shfl_xor(sq, o, 64);
    if (cl == 0 && row < P.m) cst(ss_out + row * P.n_ss + tile, sq);
  }
}

// ------------------------------------------------------------ attention
// Work item (kv head g, group of GP pages of positions); block rows
// r = j*G + hh (block row j, query head g*G + hh) see positions t <= L + j.
// The group is walked in kPage sub-chunks with a running (max, sum, output)
// per row: S = Q K^T and O += P V on MFMA (Q and P split into bf16 hi + lo;
// bf16 keys and values are exact operands, fp32 ones are split too).  An
// item holding block positions first rotates the new keys, rounds keys and
// values to the cache dtype and writes them; it then attends to the rounded
// values like every other position.  Each item leaves per-row (max, sum,
// unnormalised output); PH_ATTN_MERGE combines the groups in ascending
// order.  The group grid is fixed, and a masked position or group adds
// exact zeros, so a row's result does not depend on the block size or on
// positions after it.
template <bool KVF32>
__device__ __forceinline__ void kv_st(void* base, long long i, float v) {
  if constexpr (KVF32) static_cast<float*>(base)[i] = v;
  else static_cast<uint16_t*>(base)[i] = (uint16_t)f2bf(v);
}
// 8 fp32 -> bf16 hi and lo parts (hi + lo carries ~16 significant bits)
__device__ __forceinline__ void split8(const float (&v)[8], u4& hi, u4& lo) {
  uint32_t h[8], l[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    h[e] = f2bf(v[e]);
    l[e] = f2bf(v[e] - bf2f(h[e]));
  }
  hi = u4{h[0] | h[1] << 16, h[2] | h[3] << 16, h[4] | h[5] << 16, h[6] | h[7] << 16};
  lo = u4{l[0] | l[1] << 16, l[2] | l[3] << 16, l[4] | l[5] << 16, l[6] | l[7] << 16};
}



// One output element (row r, dim d) of KV head g: the groups' partials
// combined in ascending group order.
__device__ __forceinline__ float attn_merge_one(const PassP& P, int g, int r, int d) {
  const int D = P.D, R = P.m * P.G, NG = P.n_groups;
  const long long base = (long long)g * NG * R + r;   // (g, grp, r) at base + grp * R
  constexpr int B = 8;                                // groups in flight
  float M = -INFINITY;
  for (int c0 = 0; c0 < NG; c0 += B) {
    float v[B];
#pragma unroll
    for (int q = 0; q < B; ++q) v[q] = c0 + q < NG ? cld(P.pm + base + (long long)(c0 + q) * R) : -INFINITY;
#pragma unroll
    for (int q = 0; q < B; ++q) M = fmaxf(M, v[q]);
  }
  float S = 0.f, A = 0.f;
  for (int c0 = 0; c0 < NG; c0 += B) {
    float vm[B], vs[B], va[B];
#pragma unroll
    for (int q = 0; q < B; ++q) {
      const bool ok = c0 + q < NG;
      const long long pi = base + (long long)(c0 + q) * R;
      vm[q] = ok ? cld(P.pm + pi) : -INFINITY;
      vs[q] = ok ? cld(P.ps + pi) : 0.f;
      va[q] = ok ? cld(P.pacc + pi * D + d) : 0.f;
    }
#pragma unroll
    for (int q = 0; q < B; ++q) {
      if (c0 + q < NG) {
        const float f = vm[q] == -INFINITY ? 0.f : expf(vm[q] - M);
        S += f * vs[q];
        A += f * va[q];
      }
    }
  }
  return A / S;
}

__device__ __forceinline__ void attn_merge_store(const PassP& P, uint4* a_o, int g, int r, int d) {
  const int j = r / P.G, h = g * P.G + r % P.G;
  afrag_put(a_o, j, h * P.D + d, attn_merge_one(P, g, r, d));
}

// The whole merge of KV head g by one workgroup (its last attention item).
// The head's accumulator partials (one contiguous block) go to LDS by
// direct agent-scope (sc1) global-to-LDS loads while the row maxima and
// sums are read with agent-scope loads, so the merge waits on memory once;
// then the per-row group factors, then each output from LDS.  Same
// arithmetic as attn_merge_one.  The host enables this path only when the
// head's partials fit in the LDS working set (kInlineMergeElems floats).
__device__ __forceinline__ void attn_merge_head(const PassP& P, uint4* a_o, int g, unsigned char* smem) {
  const int D = P.D, R = P.m * P.G, NG = P.n_groups;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float* pa = reinterpret_cast<float*>(smem);   // [NG][R][D]: accumulator partials
  float* fv = pa + (long long)NG * R * D;       // [NG][R]: pm, then the factors
  float* sv = fv + NG * R;                      // [NG][R]: ps
  float* Sr = sv + NG * R;                      // [R]
  const long long gb = (long long)g * NG * R;
  const int nbytes = NG * R * D * 4;
  const char* src = reinterpret_cast<const char*>(P.pacc + gb * D);
  for (int off = wave * 1024; off < nbytes; off += kWaves * 1024) {
    if (off + lane * 16 < nbytes)
      __builtin_amdgcn_global_load_lds((gvoid*)(src + off + lane * 16), (lvoid*)(smem + off), 16, 0, kCpolSc1);
  }
  for (int i = tid; i < NG * R; i += kThreads) {
    fv[i] = cld(P.pm + gb + i);
    sv[i] = cld(P.ps + gb + i);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int r = tid; r < R; r += kThreads) {
    float M = -INFINITY;
    for (int c = 0; c < NG; ++c) M = fmaxf(M, fv[c * R + r]);
    float S = 0.f;
    for (int c = 0; c < NG; ++c) {
      const float m = fv[c * R + r];
      const float f = m == -INFINITY ? 0.f : expf(m - M);
      S += f * sv[c * R + r];
      fv[c * R + r] = f;
    }
    Sr[r] = S;
  }
  __syncthreads();
  // eight consecutive dims of one row per thread (one 16-byte word of each
  // A fragment)
  for (int e = tid; e < R * (D / 8); e += kThreads) {
    const int r = e / (D / 8), d0 = (e - r * (D / 8)) * 8;
    float A[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int c = 0; c < NG; ++c) {
      const float f = fv[c * R + r];
      const float* src = pa + (c * R + r) * D + d0;
#pragma unroll
      for (int q = 0; q < 8; ++q) A[q] += f * src[q];
    }
    const float inv = Sr[r];
#pragma unroll
    for (int q = 0; q < 8; ++q) A[q] = A[q] / inv;
    const int j = r / P.G, h = g * P.G + r % P.G;
    afrag_put8(a_o, j, h * D + d0, A);
  }
}

// MFMA operand of 8 cache elements from their raw 16-byte word(s): bf16 is
// the word itself (lo part zero), fp32 is split into hi and lo.
template <bool KVF32>
__device__ __forceinline__ void kv_op(const u4* w, u4& hi, u4& lo) {
  if constexpr (KVF32) {
    float v[8] = {__uint_as_float(w[0][0]), __uint_as_float(w[0][1]), __uint_as_float(w[0][2]),
                  __uint_as_float(w[0][3]), __uint_as_float(w[1][0]), __uint_as_float(w[1][1]),
                  __uint_as_float(w[1][2]), __uint_as_float(w[1][3])};
    split8(v, hi, lo);
  } else {
    hi = w[0];
    lo = u4{0u, 0u, 0u, 0u};
  }
}

// Zeroes cache elements at positions p0 .. p0+7 that lie at or past nvalid.
template <bool KVF32>
__device__ __forceinline__ void kv_mask(u4* w, int p0, int nvalid) {
  if constexpr (KVF32) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (p0 + e >= nvalid) w[e >> 2][e & 3] = 0u;
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (p0 + 2 * c >= nvalid) w[0][c] &= 0xFFFF0000u;
      if (p0 + 2 * c + 1 >= nvalid) w[0][c] &= 0x0000FFFFu;
    }
  }
}

// Softmax of a group is taken in two passes with one maximum per row over
// the whole group: p = exp(s - max), l = sum over sub-chunks (in order) of
// the sub-chunk's sum (16 threads per row, 4 positions each, then a tree),
// O = sum over sub-chunks and 32-position chunks (in order) of P V.  With
// bf16 values and one row tile the whole group is scored at once; otherwise
// scores are recomputed per sub-chunk in the second pass -- the same
// operations in the same order, so both give identical bits.
template <bool KVF32, int MAXRT, bool GEN, int GP>
__device__ __forceinline__ void attention_phase(const PassP& P, void* kv, const uint4* qf, uint4* a_o,
                                                unsigned long long* ready, int dep, unsigned char* smem,
                                                unsigned long long* wst) {
  constexpr int W = KVF32 ? 2 : 1;                    // 16-byte words per 8 cache elements
  constexpr bool ONE = !KVF32 && MAXRT == 1;          // the whole group at once
  constexpr int NPF = ONE ? GP : 1;                   // sub-chunks whose operands are loaded together
  const int D = P.D, KDC = D / 32;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  Ctl* C = ctl(smem, (size_t)P.lds_bytes);
  const int R = P.m * P.G;
  const int NRT = (R + 15) >> 4;   // row tiles per KV head: one per work item
  const int RT = MAXRT;            // row tiles of this item
  const int T = P.T;
  constexpr int PSW = (ONE ? GP * kPage : kPage) + 4;  // floats per score row
  u4* Qf = reinterpret_cast<u4*>(smem);                              // [RT][KDC][2][64] (two-pass path)
  float* Ps = reinterpret_cast<float*>(smem + (size_t)RT * KDC * 2 * 1024);   // [RT*16][PSW]
  float* mrun = Ps + RT * 16 * PSW;
  float* lrun = mrun + RT * 16;
  const int n_items = P.Hkv * P.n_groups * NRT;
  const int DTW = D / 16 / kWaves;           // value tiles (16 d) per wave: 1 or 2
  const int key = 16 * wave + (lane & 15);   // this lane's key within a sub-chunk (scores)
  const int kq = 8 * (lane >> 4);            // first of this lane's 8 k in a 32-k chunk
  const int srow = tid >> 4, sq = (tid & 15) * 4;   // softmax: row, first of 4 positions
  // Items of one (KV head, group) read the same keys and values: they are
  // numbered 8 apart, so they run on one XCD (workgroups are dealt to the
  // eight XCDs in turn) and share its L2; the last, partial set of eight
  // (head, group) pairs is numbered densely.
  const int n_pairs = P.Hkv * P.n_groups;
  const int n_full = (n_pairs / 8) * 8 * NRT;
  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    int pair, rt0;
    if (item < n_full) {
      const int wi = item % (8 * NRT);
      rt0 = wi / 8;
      pair = item / (8 * NRT) * 8 + wi % 8;
    } else {
      const int rem = n_pairs % 8, wi = item - n_full;
      rt0 = wi / rem;
      pair = n_pairs / 8 * 8 + wi % rem;
    }
    const int g = pair / P.n_groups, grp = pair % P.n_groups;
    const int rb = rt0 * 16;   // first block row of this item
    const int gt0 = grp * GP * kPage;
    const int nsc = min(GP, (T - gt0 + kPage - 1) / kPage);   // sub-chunks holding positions
    // waits until this KV head's query fragments and new cache rows are written
    auto wait_head = [&]() {
      if (dep == kDepHeads) {
        if (tid == 0) ready_wait(ready + g, P.epoch * heads_expect(P), P.err);
        __syncthreads();
      }
    };
    const gu4* qsrc = (const gu4*)(qf + ((long long)g * P.qf_rt + rt0) * KDC * 2 * 64);
    // ---- query fragments: registers (one row tile) or LDS
    u4 qh[4], ql[4];
    if constexpr (!ONE) wait_head();
    if constexpr (ONE) {
      // (loaded below, after the old positions' operands and the wait)
    } else {
      constexpr int QB = 8;
      for (int i0 = tid; i0 < RT * KDC * 2 * 64; i0 += kThreads * QB) {
        u4 v[QB];
#pragma unroll
        for (int q = 0; q < QB; ++q)
          if (i0 + q * kThreads < RT * KDC * 2 * 64) v[q] = qsrc[i0 + q * kThreads];
#pragma unroll
        for (int q = 0; q < QB; ++q)
          if (i0 + q * kThreads < RT * KDC * 2 * 64) Qf[i0 + q * kThreads] = v[q];
      }
    }
    for (int r = tid; r < RT * 16; r += kThreads) {
      mrun[r] = -INFINITY;
      lrun[r] = 0.f;
    }
    // operand words of one sub-chunk: keys 16*wave.. of this lane (scores)
    // and values of this wave's d tiles (output)
    // pages of the group's sub-chunks, looked up together
    int phys[GP];
#pragma unroll
    for (int sc = 0; sc < GP; ++sc) phys[sc] = P.page_table[min(gt0 / kPage + sc, (T - 1) / kPage)];
    auto load_ops = [&](int sc, u4 (&kr)[4 * W], u4 (&vr)[2][2 * W]) {
      const long long kb = (((long long)phys[sc] * P.Hkv + g) * 2 + 0) * kPage * D;
      const long long vb = kb + (long long)kPage * D;
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        if (kc >= KDC) break;
        const gu4* src = (const gu4*)(static_cast<const char*>(kv) + (kb + (long long)key * D + kc * 32 + kq) * (KVF32 ? 4 : 2));
#pragma unroll
        for (int w = 0; w < W; ++w) kr[kc * W + w] = src[w];
      }
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        if (q >= DTW) break;
        const int d = (wave * DTW + q) * 16 + (lane & 15);
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
          const gu4* src = (const gu4*)(static_cast<const char*>(kv) + (vb + (long long)d * kPage + kc * 32 + kq) * (KVF32 ? 4 : 2));
#pragma unroll
          for (int w = 0; w < W; ++w) vr[q][kc * W + w] = src[w];
        }
      }
    };
    // scores of this wave's 16 keys of sub-chunk sc for row tile rt, masked
    auto scores = [&](int sc, int rt, const u4 (&kr)[4 * W]) -> f32x4 {
      const int t0 = gt0 + sc * kPage;
      const int nkeys = GEN && P.page_live ? P.page_live[t0 / kPage] : min(kPage, T - t0);
      f32x4 s4 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        if (kc >= KDC) break;
        u4 w[W];
#pragma unroll
        for (int x = 0; x < W; ++x) w[x] = kr[kc * W + x];
        if (key >= nkeys) {
#pragma unroll
          for (int x = 0; x < W; ++x) w[x] = u4{0u, 0u, 0u, 0u};
        }
        u4 kh, kl;
        kv_op<KVF32>(w, kh, kl);
        u4 a_h, a_l;
        if constexpr (ONE) {
          a_h = qh[kc];
          a_l = ql[kc];
        } else {
          a_h = Qf[((rt * KDC + kc) * 2 + 0) * 64 + lane];
          a_l = Qf[((rt * KDC + kc) * 2 + 1) * 64 + lane];
        }
        s4 = mfma(a_h, kh, s4);
        s4 = mfma(a_l, kh, s4);
        if constexpr (KVF32) {
          s4 = mfma(a_h, kl, s4);
          s4 = mfma(a_l, kl, s4);
        }
      }
      const int tk = t0 + key;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = rb + rt * 16 + 4 * (lane >> 4) + i;
        // causal: block row j sees positions up to L + j; a token tree: the
        // committed cache and the rows of its ancestor mask; several
        // sequences: the row's own slot interval
        bool seen = tk <= P.L + r / P.G;
        if (GEN && P.tree_anc && tk >= P.L && tk - P.L < kMaxRows && r < R)
          seen = ((P.tree_anc[r / P.G] >> (tk - P.L)) & 1u) != 0u;
        if (GEN && P.row_hi && r < R) seen = tk >= P.row_lo[r / P.G] && tk <= P.row_hi[r / P.G];
        const bool vis = r < R && key < nkeys && seen;
        s4[i] = vis ? s4[i] : -INFINITY;
      }
      return s4;
    };
    // O += P V for sub-chunk sc (P in Ps at column offset pc)
    f32x4 acc[MAXRT][2];
#pragma unroll
    for (int rt = 0; rt < MAXRT; ++rt)
#pragma unroll
      for (int q = 0; q < 2; ++q) acc[rt][q] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto pv = [&](int sc, int pc, u4 (&vr)[2][2 * W]) {
      const int nkeys = GEN && P.page_live ? P.page_live[gt0 / kPage + sc] : min(kPage, T - (gt0 + sc * kPage));
      u4 vh[2][2], vl[2][2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        if (q >= DTW) break;
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
          u4 w[W];
#pragma unroll
          for (int x = 0; x < W; ++x) w[x] = vr[q][kc * W + x];
          kv_mask<KVF32>(w, kc * 32 + kq, nkeys);
          kv_op<KVF32>(w, vh[q][kc], vl[q][kc]);
        }
      }
#pragma unroll
      for (int rt = 0; rt < MAXRT; ++rt) {
        if (rt >= RT) break;
        u4 ph[2], pl[2];
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
          const float* pr = Ps + (rt * 16 + (lane & 15)) * PSW + pc + kc * 32 + kq;
          float v[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = pr[e];
          split8(v, ph[kc], pl[kc]);
        }
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          if (q >= DTW) break;
          f32x4 a4 = acc[rt][q];
#pragma unroll
          for (int kc = 0; kc < 2; ++kc) {
            a4 = mfma(ph[kc], vh[q][kc], a4);
            a4 = mfma(pl[kc], vh[q][kc], a4);
            if constexpr (KVF32) {
              a4 = mfma(ph[kc], vl[q][kc], a4);
              a4 = mfma(pl[kc], vl[q][kc], a4);
            }
          }
          acc[rt][q] = a4;
        }
      }
    };
    // p = exp(s - max) over positions pc .. pc+63 of score row r (this
    // thread's 4); returns the sub-chunk sum over the row's 16 threads
    auto expsum = [&](int r, int pc) -> float {
      const float mr = mrun[r];
      float l = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float sv = Ps[r * PSW + pc + sq + e];
        const float p = (mr == -INFINITY || sv == -INFINITY) ? 0.f : expf(sv - mr);
        Ps[r * PSW + pc + sq + e] = p;
        l += p;
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) l += __shfl_xor(l, o, 64);
      return l;
    };

    if constexpr (ONE) {
      // sub-chunks wholly before L hold no new rows: their operands go out
      // before the wait on this head's QKV blocks
      const int n_old = min(nsc, max(0, (P.L - gt0) / kPage));
      u4 kr[NPF][4 * W], vr[NPF][2][2 * W];
#pragma unroll
      for (int sc = 0; sc < NPF; ++sc)
        if (sc < n_old) load_ops(sc, kr[sc], vr[sc]);
      wait_head();
#pragma unroll
      for (int kc = 0; kc < 4; ++kc)
        if (kc < KDC) {
          qh[kc] = qsrc[(kc * 2 + 0) * 64 + lane];
          ql[kc] = qsrc[(kc * 2 + 1) * 64 + lane];
        }
#pragma unroll
      for (int sc = 0; sc < NPF; ++sc)
        if (sc >= n_old && sc < nsc) load_ops(sc, kr[sc], vr[sc]);
      __syncthreads();   // mrun / lrun initialised
      wstamp(wst, 1);
#pragma unroll
      for (int sc = 0; sc < NPF; ++sc) {
        if (sc >= nsc) break;
        const f32x4 s4 = scores(sc, 0, kr[sc]);
#pragma unroll
        for (int i = 0; i < 4; ++i) Ps[(4 * (lane >> 4) + i) * PSW + sc * kPage + key] = s4[i];
      }
      __syncthreads();
      {
        // row maximum over the group, then the sums
        float mx = -INFINITY;
        for (int sc = 0; sc < nsc; ++sc)
#pragma unroll
          for (int e = 0; e < 4; ++e) mx = fmaxf(mx, Ps[srow * PSW + sc * kPage + sq + e]);
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
        if ((tid & 15) == 0) mrun[srow] = mx;
        // per-sub-chunk sums (the four trees interleaved), added in order
        float ls[GP];
#pragma unroll
        for (int sc = 0; sc < GP; ++sc) {
          ls[sc] = 0.f;
          if (sc < nsc) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              float* pp = Ps + srow * PSW + sc * kPage + sq + e;
              const float sv = *pp;
              const float p = (mx == -INFINITY || sv == -INFINITY) ? 0.f : expf(sv - mx);
              *pp = p;
              ls[sc] += p;
            }
          }
        }
#pragma unroll
        for (int o = 1; o < 16; o <<= 1)
#pragma unroll
          for (int sc = 0; sc < GP; ++sc) ls[sc] += __shfl_xor(ls[sc], o, 64);
        float l = 0.f;
        for (int sc = 0; sc < nsc; ++sc) l += ls[sc];
        if ((tid & 15) == 0) lrun[srow] = l;
      }
      __syncthreads();
#pragma unroll
      for (int sc = 0; sc < NPF; ++sc) {
        if (sc >= nsc) break;
        pv(sc, sc * kPage, vr[sc]);
      }
    } else {
      __syncthreads();   // query fragments and mrun / lrun in LDS
      wstamp(wst, 1);
      // pass 1: row maxima
      for (int sc = 0; sc < nsc; ++sc) {
        u4 kr[4 * W], vr[2][2 * W];
        load_ops(sc, kr, vr);
#pragma unroll
        for (int rt = 0; rt < MAXRT; ++rt) {
          if (rt >= RT) break;
          const f32x4 s4 = scores(sc, rt, kr);
#pragma unroll
          for (int i = 0; i < 4; ++i) Ps[(rt * 16 + 4 * (lane >> 4) + i) * PSW + key] = s4[i];
        }
        __syncthreads();
        for (int r = srow; r < RT * 16; r += kThreads / 16) {
          float mx = -INFINITY;
#pragma unroll
          for (int e = 0; e < 4; ++e) mx = fmaxf(mx, Ps[r * PSW + sq + e]);
#pragma unroll
          for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
          if ((tid & 15) == 0) mrun[r] = fmaxf(mrun[r], mx);
        }
        __syncthreads();
      }
      // pass 2: the same scores again, probabilities, sums and P V
      for (int sc = 0; sc < nsc; ++sc) {
        u4 kr[4 * W], vr[2][2 * W];
        load_ops(sc, kr, vr);
#pragma unroll
        for (int rt = 0; rt < MAXRT; ++rt) {
          if (rt >= RT) break;
          const f32x4 s4 = scores(sc, rt, kr);
#pragma unroll
          for (int i = 0; i < 4; ++i) Ps[(rt * 16 + 4 * (lane >> 4) + i) * PSW + key] = s4[i];
        }
        __syncthreads();
        for (int r = srow; r < RT * 16; r += kThreads / 16) {
          const float l = expsum(r, 0);
          if ((tid & 15) == 0) lrun[r] += l;
        }
        __syncthreads();
        pv(sc, 0, vr);
        __syncthreads();
      }
    }
    wstamp(wst, 2);
    // ---- per-row partials of this group
    const long long ib = ((long long)g * P.n_groups + grp) * R;
#pragma unroll
    for (int rt = 0; rt < MAXRT; ++rt) {
      if (rt >= RT) break;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        if (q >= DTW) break;
        const int d = (wave * DTW + q) * 16 + (lane & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = rb + rt * 16 + 4 * (lane >> 4) + i;
          if (r < R) cst(P.pacc + (ib + r) * D + d, acc[rt][q][i]);
        }
      }
    }
    __syncthreads();   // lrun complete
    for (int lr = tid; lr < RT * 16; lr += kThreads) {
      if (rb + lr < R) {
        cst(P.pm + ib + rb + lr, mrun[lr]);
        cst(P.ps + ib + rb + lr, lrun[lr]);
      }
    }
    if (P.attn_inline) {
      // the last item (group, row tile) of head g to finish merges the head
      release_all_waves();
      __syncthreads();
      if (tid == 0) {
        const unsigned old = __hip_atomic_fetch_add(glb(P.attn_tickets + g), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const bool last = old == (unsigned)(P.n_groups * NRT - 1);
        if (last) __hip_atomic_store(glb(P.attn_tickets + g), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        C->misc[0] = last ? 1 : 0;   // the partials are then read with agent-scope loads
      }
      __syncthreads();
      if (C->misc[0]) {
        attn_merge_head(P, a_o, g, smem);
        // the O projection's windows that hold these query heads
        release_all_waves();
        __syncthreads();
        if (tid == 0)
          for (int h = g * P.G; h < (g + 1) * P.G; ++h)
            for (int w = h * D / P.o_wcols; w <= ((h + 1) * D - 1) / P.o_wcols; ++w) ready_add(ready + kRdyOWin + w);
      }
    }
    __syncthreads();
  }
}

// The merge as a phase of its own (heads with many groups or rows): one
// output element per thread over the whole grid.
// The O projection then follows a grid barrier, so nothing in this pass
// waits on the O-window ready counters; they still advance by one pass's
// count (a later pass that merges inline waits for the pass number times
// that count).
__device__ __forceinline__ void attn_merge_phase(const PassP& P, uint4* a_o, unsigned long long* ready) {
  const int D = P.D, R = P.m * P.G;
  const long long total = (long long)P.Hkv * R * D;
  for (long long e = (long long)blockIdx.x * kThreads + threadIdx.x; e < total; e += (long long)gridDim.x * kThreads) {
    const int d = (int)(e % D);
    const long long gr = e / D;
    attn_merge_store(P, a_o, (int)(gr / R), (int)(gr % R), d);
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    const int n_win = (P.Hq * D + P.o_wcols - 1) / P.o_wcols;
    for (int w = 0; w < n_win; ++w) ready_add(ready + kRdyOWin + w, owin_expect(P, w));
  }
}

// ------------------------------------------------------------ MoE routing
// Every workgroup routes the block redundantly (same inputs, same order):
// pi = softmax(r + b) over the experts, each row keeps its top_k experts by
// probability (ties to the lower id), weights = those probabilities; the
// union of the rows' experts in ascending id order becomes the slot list.
// Workgroup 0 also writes the routing record for the combine phase.
// Router logits of the block computed by this workgroup alone (bf16 router
// weights, K in one A window): the normalised A operand is staged, each wave
// takes router units wave, wave + 4, ... (16 experts each) over every K
// chunk on MFMA, and the row-scaled logits go to zl[16][E] in LDS.  Every
// workgroup runs the same operations in the same order, so all hold the
// same logits.
template <int WF>
__device__ __forceinline__ void router_logits(const PassP& P, const Mat& Mr, const GemmIO& io, unsigned char* smem,
                                              float* zl) {
  Ctl* C = ctl(smem, (size_t)P.lds_bytes);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const Lin L = make_lin(Mr, 1, false);
  stage_window<WF>(L, io, 0, 0, smem, P.m);
  row_scales(P, io.ss_in, C->rs);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const uint4* aw = reinterpret_cast<const uint4*>(smem);
  constexpr int NB = 32;   // fragments in flight per lane
  constexpr int UPW = 4;   // units per wave at most (E <= 256: 16 units)
  f32x4 acc[UPW];
#pragma unroll
  for (int j = 0; j < UPW; ++j) {
    acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int unit = wave + kWaves * j;
    if (unit < Mr.n_units) {   // (wave-uniform)
      const int sg = unit / kWaves, w = unit % kWaves;
      const char* wb = static_cast<const char*>(Mr.w) + ((long long)sg * Mr.nkc * kWaves + w) * 1024 + lane * 16;
      f32x4 a4 = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int c0 = 0; c0 < Mr.nkc; c0 += NB) {
        u4 wf[NB];
#pragma unroll
        for (int i = 0; i < NB; ++i)
          wf[i] = c0 + i < Mr.nkc ? *(const gu4*)(wb + (long long)(c0 + i) * kWaves * 1024) : u4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          if (c0 + i < Mr.nkc) {
            const u4 ah = __builtin_bit_cast(u4, aw[(c0 + i) * 128 + lane]);
            const u4 al = __builtin_bit_cast(u4, aw[(c0 + i) * 128 + 64 + lane]);
            a4 = mfma(ah, wf[i], a4);
            a4 = mfma(al, wf[i], a4);
          }
        }
      }
      acc[j] = a4;
    }
  }
#pragma unroll
  for (int j = 0; j < UPW; ++j) {
    const int unit = wave + kWaves * j;
    const int col = unit * kTileN + (lane & 15);
    if (unit < Mr.n_units && col < P.E) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 4 * (lane >> 4) + i;
        zl[row * P.E + col] = C->rs[row] * acc[j][i];
      }
    }
  }
  __syncthreads();
}

// Reuse-aware gating (S2-MoE section 4.2; a lossy variant, off unless
// asked for): the block's gating logits l_b (router logits with bias) give
// each expert an importance g_e = sum_b w_b l_{b,e} (w_b the row's
// confidence, rows in order); the cap experts of largest importance (ties to
// the lower id) are preferred; every row b adds lambda_b = alpha (l_b(1) -
// l_b(top_k+1)) -- the gap between its first and (top_k+1)-th logit -- to
// the preferred experts' logits, and routing proceeds on the biased logits.
// z holds this wave's rows (row = wave + kWaves k), experts lane + 64 i.
template <int RPW, int EPL>
__device__ __forceinline__ void reuse_bias(const PassP& P, float* zs, float* gs, int* pref, float* lam,
                                           float (&z)[RPW][EPL]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = P.E;
#pragma unroll
  for (int k = 0; k < RPW; ++k) {
    const int row = wave + kWaves * k;
    if (row < P.m) {
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (lane + 64 * i < E) zs[row * E + lane + 64 * i] = z[k][i];
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += kThreads) {
    float g = 0.f;
    for (int b = 0; b < P.m; ++b) g += (P.reuse_w ? P.reuse_w[b] : 1.f) * zs[b * E + e];
    gs[e] = g;
  }
  // each row's first and (top_k+1)-th logit, by rank (lower id first on ties)
#pragma unroll
  for (int k = 0; k < RPW; ++k) {
    const int row = wave + kWaves * k;
    if (row < P.m) {
      const float* zr = zs + row * E;
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const int e = lane + 64 * i;
        if (e < E) {
          const float ze = z[k][i];
          int rank = 0;
          for (int j = 0; j < E; ++j) rank += (zr[j] > ze || (zr[j] == ze && j < e)) ? 1 : 0;
          if (rank == 0) lam[2 * row] = ze;
          if (rank == P.top_k) lam[2 * row + 1] = ze;
        }
      }
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += kThreads) {
    const float ge = gs[e];
    int rank = 0;
    for (int j = 0; j < E; ++j) rank += (gs[j] > ge || (gs[j] == ge && j < e)) ? 1 : 0;
    pref[e] = rank < P.reuse_cap ? 1 : 0;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < RPW; ++k) {
    const int row = wave + kWaves * k;
    if (row < P.m) {
      const float lb = P.reuse_alpha * (lam[2 * row] - lam[2 * row + 1]);
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (lane + 64 * i < E && pref[lane + 64 * i]) z[k][i] += lb;
    }
  }
  __syncthreads();   // zs / gs / pref / lam are dead (the probabilities reuse the space)
}

// bz: the router bias of this lane's experts (lane + 64 i), loaded by the
// caller before the router logits.
__device__ __forceinline__ void route_bias(const float* bias, int E, float (&bz)[4]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < 4; ++i) bz[i] = lane + 64 * i < E ? *glb(bias + lane + 64 * i) : 0.f;
}

__device__ __forceinline__ void route_block(const PassP& P, const float (&bz)[4], unsigned char* smem, int layer,
                                            const float* zl) {
  Ctl* C = ctl(smem, (size_t)P.lds_bytes);
  int* used = reinterpret_cast<int*>(smem + kRouteBase);   // [E]: used, then the expert's slot (-1: none)
  int* sel = used + 256;                              // [16][top_k]
  float* selw = reinterpret_cast<float*>(sel + 16 * 16);
  float* prs = reinterpret_cast<float*>(smem + kRouteZl);   // [16][E4] probabilities (after zl is read)
  float* rsum = selw + 16 * 16 + 256 + 256 + 32;      // [16] row sums (after the reuse-gating scratch)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E4 = (P.E + 3) & ~3;
  for (int e = tid; e < P.E; e += kThreads) used[e] = 0;
  constexpr int EPL = 4;                 // experts per lane (E <= 256)
  constexpr int RPW = kMaxRows / kWaves;  // rows per wave: row = wave + kWaves k
  // every row's router logits of this wave are loaded before any is used
  float z[RPW][EPL];
#pragma unroll
  for (int k = 0; k < RPW; ++k) {
    const int row = wave + kWaves * k;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane + 64 * i;
      z[k][i] = (row < P.m && e < P.E) ? (zl ? zl[row * P.E + e] : cld(P.rlog + row * P.ldr + e)) : 0.f;
    }
  }
  __syncthreads();   // every wave holds its logits (the area is rewritten below)
  // the gating logits (router logits with bias)
#pragma unroll
  for (int k = 0; k < RPW; ++k)
#pragma unroll
    for (int i = 0; i < EPL; ++i) z[k][i] = lane + 64 * i < P.E ? z[k][i] + bz[i] : -INFINITY;
  if (P.reuse_cap > 0) {
    float* zs = prs;                          // [16][E] (before the probabilities are written)
    float* gs = selw + 16 * 16;               // [E]
    int* pref = reinterpret_cast<int*>(gs + 256);   // [E]
    float* lam = gs + 512;                    // [16][2]
    reuse_bias<RPW, EPL>(P, zs, gs, pref, lam, z);
  }
  // softmax of every row, the rows' reductions side by side
  float mx[RPW], sum[RPW];
#pragma unroll
  for (int k = 0; k < RPW; ++k) {
    mx[k] = -INFINITY;
#pragma unroll
    for (int i = 0; i < EPL; ++i) mx[k] = fmaxf(mx[k], z[k][i]);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1)
#pragma unroll
    for (int k = 0; k < RPW; ++k) mx[k] = fmaxf(mx[k], __shfl_xor(mx[k], o, 64));
#pragma unroll
  for (int k = 0; k < RPW; ++k) {
    sum[k] = 0.f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      z[k][i] = (lane + 64 * i < P.E) ? expf(z[k][i] - mx[k]) : 0.f;   // now the probabilities (unnormalised)
      sum[k] += z[k][i];
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1)
#pragma unroll
    for (int k = 0; k < RPW; ++k) sum[k] += __shfl_xor(sum[k], o, 64);
  // top_k by rank: an expert's rank is the number of experts ahead of it in
  // the order (probability descending, lower id first on ties); the top_k
  // are the ranks below top_k, in rank order (a NaN counts as -inf, so the
  // ranks always form a permutation)
#pragma unroll
  for (int k = 0; k < RPW; ++k) {
    const int row = wave + kWaves * k;
    if (row < P.m) {
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const int e = lane + 64 * i;
        if (e < E4) prs[row * E4 + e] = e < P.E && z[k][i] == z[k][i] ? z[k][i] : -INFINITY;
      }
      if (lane == 0) rsum[row] = sum[k];
    }
  }
  __syncthreads();   // prs, the row sums and used[] complete
  // ranks of the (row, expert) pairs, spread over the workgroup's threads
  // (a row's probabilities read four at a time with several reads in
  // flight; the padding is -inf at ids past every expert, so it never
  // counts; bitwise, not short-circuit, tests: no branches)
  for (int pi = tid; pi < P.m * P.E; pi += kThreads) {
    const int row = pi / P.E, e = pi - row * P.E;
    const float* pr = prs + row * E4;
    const float pe = pr[e];
    int rank = 0;
#pragma unroll 8
    for (int j = 0; j < E4; j += 4) {
      const f32x4 q = *reinterpret_cast<const f32x4*>(pr + j);
#pragma unroll
      for (int t = 0; t < 4; ++t) rank += (int)(q[t] > pe) | ((int)(q[t] == pe) & (int)(j + t < e));
    }
    if (rank < P.top_k) {
      sel[row * P.top_k + rank] = e;
      selw[row * P.top_k + rank] = pe / rsum[row];
      used[e] = 1;
    }
  }
  __syncthreads();
  // the union in ascending expert id (wave 0: a ballot scan); used[e]
  // becomes the expert's slot, or -1
  if (wave == 0) {
    int cnt = 0;
    for (int e0 = 0; e0 < P.E; e0 += 64) {
      const int e = e0 + lane;
      const bool u = e < P.E && used[e] != 0;
      const unsigned long long bal = __ballot(u);
      const int pos = cnt + __popcll(bal & ((1ull << lane) - 1ull));
      if (u) C->ulist[pos] = e;
      if (e < P.E) used[e] = u ? pos : -1;
      cnt += __popcll(bal);
    }
    if (lane == 0) C->uc = cnt;
  }
  __syncthreads();
  if (blockIdx.x == 0) {
    int* rec = P.route;
    const int E = P.E, K = P.top_k;
    if (tid == 0) {
      cst(rec, C->uc);
      if (P.union_hist) P.union_hist[layer] = C->uc;
    }
    if (P.route_hist)
      for (int i = tid; i < P.m * K; i += kThreads) P.route_hist[(long long)layer * P.m * K + i] = sel[i];
    for (int e = tid; e < E; e += kThreads) {
      cst(rec + 1 + e, e < C->uc ? C->ulist[e] : -1);
      cst(rec + 1 + E + e, used[e]);
    }
    for (int i = tid; i < P.m * K; i += kThreads) {
      cst(rec + 1 + 2 * E + i, sel[i]);
      cst(reinterpret_cast<float*>(rec) + 1 + 2 * E + 16 * K + i, selw[i]);
    }
  }
  __syncthreads();
}

// x_j += sum_r w_{j,r} y[slot(sel_{j,r})]_j + sum_s y[shared slot s]_j, in
// rank order then shared; new sum-of-squares partials and next A operand.
__device__ __forceinline__ void moe_combine_phase(const PassP& P, const float* next_gain, float* trace, uint4* a_out,
                                                  float* ss_out) {
  const int n_tiles = (P.d + 15) / 16;
  const int t = threadIdx.x;
  const int row = t >> 4, cl = t & 15;
  const int* rec = P.route;
  const int E = P.E, K = P.top_k;
  const int uc = cld(rec);
  for (int tile = blockIdx.x; tile < n_tiles; tile += gridDim.x) {
    if (t >= 256) continue;
    const int col = tile * 16 + cl;
    float v = 0.f;
    if (row < P.m && col < P.d) {
      float y = 0.f;
      for (int r = 0; r < K; ++r) {
        const int e = cld(rec + 1 + 2 * E + row * K + r);
        const float w = cld(reinterpret_cast<const float*>(rec) + 1 + 2 * E + 16 * K + row * K + r);
        const int s = cld(rec + 1 + E + e);
        y += w * cld(P.ey + (long long)s * P.ey_slot + (long long)row * P.ldy + col);
      }
      for (int s = 0; s < P.n_shared; ++s) y += cld(P.ey + (long long)(uc + s) * P.ey_slot + (long long)row * P.ldy + col);
      v = cld(P.x + (long long)row * P.ldx + col) + y;
      cst(P.x + (long long)row * P.ldx + col, v);
      if (trace) trace[(long long)row * P.d + col] = v;
    }
    if (col < P.d) afrag_put(a_out, row, col, v * *glb(next_gain + col));
    float sq = v * v;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) sq += __shfl_xor(sq, o, 64);
    if (cl == 0 && row < P.m) cst(ss_out + row * P.n_ss + tile, sq);
  }
}

// ------------------------------------------------------------ the pass
// start of phase ph (after its barrier), taken by workgroup 0
__device__ __forceinline__ void stamp(const PassP& P, int ph) {
  if (P.stamps && blockIdx.x == 0 && threadIdx.x == 0) P.stamps[ph] = wall_clock64();
}


// The pass interprets a program of phases prepared by the host (one entry
// per phase, a grid barrier between consecutive phases).  Each phase kind
// is inlined once, and the weight ring lives in registers for the whole
// pass.  Dense and MoE models get separate instances, each holding only the
// phase kinds its programs use (the kernel's code size shows in its speed).
template <int WF, bool MOE, bool GEN>
__global__ __launch_bounds__(kThreads) void k_pass(PassP P) {
  extern __shared__ __align__(16) unsigned char smem[];
  Ctl* C = ctl(smem, (size_t)P.lds_bytes);
  GridBar gb{P.bar, P.bar_base, P.err, false};
  Ring ring;
  for (int ph = 0; ph < P.n_prog; ++ph) {
    // local copy: loop-invariant phase fields stay in registers (the phase's
    // own stores could otherwise alias the descriptor in memory)
    const Phase dd = P.prog[ph];
    const Phase* d = &dd;
    const int kind = d->kind;
    GemmIO io;
    io.a = d->a; io.a_slot = d->a_slot;
    io.out = d->out; io.ldo = d->ldo; io.out_slot = d->out_slot; io.scale = d->scale;
    io.gain = d->gain; io.a_out = d->a_out; io.a_out_slot = d->a_out_slot;
    io.trace = (d->trace && P.trace) ? P.trace + (long long)d->layer * P.m * P.d : nullptr;
    io.ready = P.ready + (long long)max(d->layer, 0) * kReadyStride;
    io.ss_in = d->ss_in; io.ss_out = d->ss_out;
    io.ws = P.ws_alt ? P.ws_alt + (long long)d->ws_bank * P.ws_bank_floats : d->ws;
    io.tickets = P.tickets_alt ? P.tickets_alt + (long long)d->ws_bank * P.tickets_bank : d->tickets;
    io.dep = d->dep;
    io.notify = d->notify;
    // the O projection waits on merged heads only when attention merges
    // inline; otherwise the merge phase and a barrier come first
    const bool dataflow = d->dep != kDepNone && !(d->dep == kDepOWin && !P.attn_inline);
    if (!dataflow) io.dep = kDepNone;
    const SlotMap dense{nullptr, 0, 0, 1};
    const SlotMap slots{C->ulist, C->uc, P.E, C->uc + P.n_shared};
    // Each phase but the first starts with a grid barrier, unless its inputs
    // come over ready counters (it then waits on those where it reads
    // them).  A weight-streaming phase issues its first weight batch during
    // that barrier (or right away); the ring is written right before every
    // phase that reads it, so it is dead (and its registers free) in the
    // other phases.
    unsigned long long* wst = P.wstamps ? P.wstamps + ((long long)ph * gridDim.x + blockIdx.x) * 4 : nullptr;
    auto sync = [&](auto&& prefetch) {
      if (ph > 0) wstamp(wst ? wst - (long long)gridDim.x * 4 : nullptr, 3);   // end of the previous phase's work
      if (ph > 0 && !dataflow) grid_sync(gb, prefetch);
      else prefetch();
      stamp(P, ph);
      wstamp(wst, 0);
    };
    switch (kind) {
      case PH_EMBED:
        sync([] {});
        embed_phase(P, WF == W_F32, d->a_out, d->ss_out);
        break;
      case PH_STORE: {
        if constexpr (!MOE) break;
        const SlotMap sm = d->slot_mode ? slots : dense;
        sync([&] { gemm_prefetch<WF, 1>(d->M, sm, d->slot_mode == 2, ring); });
        // (the MoE pass's stores: router and expert down, both in fixed order)
        gemm_phase<WF, EPI_STORE, 1, GEN, true>(P, d->M, io, sm, d->slot_mode == 2, ring, smem, wst);
        break;
      }
      case PH_QKV:
        sync([&] { gemm_prefetch<WF, 1>(d->M, dense, false, ring); });
        io.kv = d->kv;
        gemm_phase<WF, EPI_QKV, 1, GEN>(P, d->M, io, dense, false, ring, smem, wst);
        break;
      case PH_RESID:
        sync([&] { gemm_prefetch<WF, 1>(d->M, dense, false, ring); });
        gemm_phase<WF, EPI_RESID, 1, GEN>(P, d->M, io, dense, false, ring, smem, wst);
        break;
      case PH_ROUTE_SWIGLU:
        if constexpr (!MOE) break;
        sync([] {});
      {
        float* zl = nullptr;
        float bz[4];
        route_bias(d->bias, P.E, bz);
        bool staged = false;   // the router's A window is the routed experts' one
        if constexpr (WF == W_BF16) {
          if (d->Mr.w) {
            zl = reinterpret_cast<float*>(smem + kRouteZl);
            router_logits<WF>(P, d->Mr, io, smem, zl);
            staged = d->Mr.win == d->M.win;
          }
        }
        route_block(P, bz, smem, d->layer, zl);
        const SlotMap routed{C->ulist, C->uc, P.E, C->uc + P.n_shared};   // the union just built
        gemm_prefetch<WF, 2>(d->M, routed, false, ring);
        gemm_phase<WF, EPI_SWIGLU, 2, GEN, true>(P, d->M, io, routed, false, ring, smem, wst, staged);
        break;
      }
      case PH_SWIGLU:
        if constexpr (MOE) break;
        sync([&] { gemm_prefetch<WF, 2>(d->M, dense, false, ring); });
        gemm_phase<WF, EPI_SWIGLU, 2, GEN>(P, d->M, io, dense, false, ring, smem, wst);
        break;
      case PH_LOGITS:
        sync([&] { gemm_prefetch<WF, 1>(d->M, dense, false, ring); });
        gemm_phase<WF, EPI_LOGITS, 1, GEN>(P, d->M, io, dense, false, ring, smem, wst);
        break;
      case PH_ATTN:
        sync([] {});
        wstamp(wst, 1);
        wstamp(wst, 2);
        // (fp32 caches: groups of 3 pages only)
        if (WF != W_F32 && P.group_pages == 6)
          attention_phase<WF == W_F32, 1, GEN, 6>(P, d->kv, d->a, d->a_out, io.ready, io.dep, smem, wst);
        else if (WF != W_F32 && P.group_pages == 5)
          attention_phase<WF == W_F32, 1, GEN, 5>(P, d->kv, d->a, d->a_out, io.ready, io.dep, smem, wst);
        else
          attention_phase<WF == W_F32, 1, GEN, kGroupPages>(P, d->kv, d->a, d->a_out, io.ready, io.dep, smem, wst);
        break;
      case PH_ATTN_MERGE:
        if (P.attn_inline) {
          // merged by attention's last arrivers: no barrier, an empty phase
          stamp(P, ph);
          if (wst) {
            wstamp(wst - (long long)gridDim.x * 4, 3);   // end of the attention's work
            for (int i = 0; i < 3; ++i) wstamp(wst, i);  // (its end comes with the next phase)
          }
          break;
        }
        sync([] {});
        attn_merge_phase(P, d->a_out, io.ready);
        break;
      case PH_COMBINE:
        if constexpr (!MOE) break;
        sync([] {});
        moe_combine_phase(P, d->gain, io.trace, d->a_out, d->ss_out);
        break;
      default:
        sync([] {});
        break;
    }
  }
  if (P.wstamps) wstamp(P.wstamps + ((long long)(P.n_prog - 1) * gridDim.x + blockIdx.x) * 4, 3);
}


// The pass kernel for a weight format and model kind; gen: the instance
// that reads per-row placement (token trees, several sequences).
static const void* pick(int wfmt, bool moe, bool gen) {
#define SV_PICK(W)                                                                                    \
  return moe ? (gen ? reinterpret_cast<const void*>(&k_pass<W, true, true>)                         \
                    : reinterpret_cast<const void*>(&k_pass<W, true, false>))                       \
             : (gen ? reinterpret_cast<const void*>(&k_pass<W, false, true>)                        \
                    : reinterpret_cast<const void*>(&k_pass<W, false, false>))
  if (wfmt == W_F32) SV_PICK(W_F32);
  if (wfmt == W_BF16) SV_PICK(W_BF16);
  if (wfmt == W_INT4) SV_PICK(W_INT4);
#undef SV_PICK
  return nullptr;
}

hipError_t pass_occupancy(int wfmt, bool moe, size_t lds, int* blocks_per_cu) {
  const void* f = pick(wfmt, moe, false);
  const void* fg = pick(wfmt, moe, true);
  if (!f || !fg) return hipErrorInvalidValue;
  hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e == hipSuccess) e = hipFuncSetAttribute(fg, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  int a = 0, b = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&a, f, kThreads, lds);
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, fg, kThreads, lds);
  *blocks_per_cu = a < b ? a : b;
  return e;
}

hipError_t launch_pass(int wfmt, bool moe, const PassP& p, int n_wg, size_t lds, hipStream_t s) {
  const bool gen = p.row_slot || p.row_rope || p.row_lo || p.row_hi || p.page_live || p.tree_anc;
  const void* f = pick(wfmt, moe, gen);
  if (!f) return hipErrorInvalidValue;
  PassP q = p;
  void* args[] = {&q};
  return hipLaunchCooperativeKernel(f, dim3(n_wg), dim3(kThreads), args, (unsigned)lds, s);
}

}  // namespace sv
