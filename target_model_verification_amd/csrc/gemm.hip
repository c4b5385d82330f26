// Weight-streaming skinny GEMM for the verification block (m = k+1 <= 16
// rows): Y[m][N] (op)= X[m][K] . W[K][N], every weight read once per pass.
//
// The pass is bound by HBM bandwidth: each weight byte is used by at most
// 16 rows, far below the MFMA ridge.  The kernel is laid out for that:
//  - W is pre-tiled into 1 KB MFMA B-operand fragments (16 columns x 32 k,
//    lane-major), so every wave load is one fully coalesced 1 KB dwordx4
//    transaction and a tile's K extent is a contiguous stream;
//  - activations are split once per workgroup into bf16 hi + lo parts in
//    LDS (A-operand layout), and each fragment feeds two MFMAs (hi, lo), so
//    products carry ~16 bits of activation precision with fp32 accumulation
//    (fp32 weights are pre-split hi/lo too: four MFMAs);
//  - K is split across workgroups when the grid would otherwise be too small
//    to fill 256 CUs; partial tiles are reduced in a fixed order by the last
//    workgroup to arrive (atomic ticket), so results are deterministic and do
//    not depend on m (block rows are independent MFMA rows);
//  - prologue: RMSNorm row scale (from per-64-column sum-of-squares
//    partials written by the producer) and the norm gain; epilogues: plain
//    store, residual add (+ new sum-of-squares partials), SwiGLU over an
//    interleaved gate/up tile pair, and logits with per-64-column
//    (max, argmax, sum-exp) partials for acceptance.
#include "sv_common.h"

namespace sv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t f2bf_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ float bf_bits2f(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ f32x4 mfma(const u4& a, const u4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// 8 signed nibbles of one dword -> 8 bf16 (exact: |q| <= 8)
__device__ __forceinline__ u4 nib8_to_bf16(uint32_t d) {
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int lo = ((int)(d << (28 - 8 * i))) >> 28;
    int hi = ((int)(d << (24 - 8 * i))) >> 28;
    uint32_t bl = __float_as_uint((float)lo) >> 16;
    uint32_t bh = __float_as_uint((float)hi) & 0xFFFF0000u;
    o[i] = bl | bh;
  }
  return u4{o[0], o[1], o[2], o[3]};
}

template <int WF, int EPI>
__global__ __launch_bounds__(256) void k_gemm(GemmParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int TPW = (EPI == EPI_SWIGLU) ? 2 : 1;  // n-tiles per wave
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int ng = blockIdx.x, split = blockIdx.y, slot = blockIdx.z;

  int expert = 0;
  if (p.union_count) {
    const int uc = *p.union_count;
    if (slot >= uc + p.n_shared) return;              // uniform per workgroup
    expert = slot < uc ? p.union_list[slot] : p.n_experts + (slot - uc);
  }
  const int tile0 = (ng * kWavesPerWG + wave) * TPW;
  const bool live = tile0 < p.n_tiles;
  const int c0 = split * p.kcs;
  const int c1 = min(p.nkc, c0 + p.kcs);
  const int nck = c1 - c0;

  float* rscale = reinterpret_cast<float*>(smem);                 // [16]
  float* red = rscale + 16;                                        // [4][16] + [4][16][3]
  u4* afr = reinterpret_cast<u4*>(smem + 1024);              // [nck][2][64]

  // ---- weight stream setup (issued before staging to overlap latency)
  const char* wbase = static_cast<const char*>(p.w) + (long long)expert * p.w_stride;
  const char* w2base = static_cast<const char*>(p.w2) + (long long)expert * p.w2_stride;

  const float* xin = p.x + (long long)slot * p.x_stride;
  f32x4 acc[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- prologue: row scales
  if (threadIdx.x < 16) {
    float sc = 1.f;
    const int r = threadIdx.x;
    if (p.ss && r < p.m) {
      float s = 0.f;
      for (int i = 0; i < p.n_ss; ++i) s += p.ss[r * p.n_ss + i];
      sc = 1.0f / sqrtf(s * p.inv_dnorm + p.eps);
    }
    rscale[threadIdx.x] = sc;
  }
  __syncthreads();
  // ---- stage X[:, c0*32 : c1*32] as hi/lo bf16 A fragments.  Each slot is
  // (chunk c, lane l): 8 consecutive k of row l%16.  Loads of up to 8 slots
  // are issued together before any is used.
  const int nslots = nck * 64;
  for (int base = 0; base < nslots; base += 8 * 256) {
    float4 xa[8], xb[8], ga[8], gb[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int slotA = base + i * 256 + threadIdx.x;
      const int c = slotA >> 6, l = slotA & 63, row = l & 15;
      const int kb = (c0 + c) * kChunkK + (l >> 4) * 8;
      xa[i] = xb[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      ga[i] = gb[i] = make_float4(1.f, 1.f, 1.f, 1.f);
      if (slotA < nslots && row < p.m && kb + 8 <= p.K) {
        const float4* xp = reinterpret_cast<const float4*>(xin + row * p.ldx + kb);
        xa[i] = xp[0];
        xb[i] = xp[1];
        if (p.gain) {
          const float4* gp = reinterpret_cast<const float4*>(p.gain + kb);
          ga[i] = gp[0];
          gb[i] = gp[1];
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int slotA = base + i * 256 + threadIdx.x;
      if (slotA >= nslots) break;
      const int c = slotA >> 6, l = slotA & 63, row = l & 15;
      const int kb = (c0 + c) * kChunkK + (l >> 4) * 8;
      float v[8];
      if (row < p.m && kb + 8 <= p.K) {
        const float sc = rscale[row];
        v[0] = xa[i].x * sc * ga[i].x; v[1] = xa[i].y * sc * ga[i].y;
        v[2] = xa[i].z * sc * ga[i].z; v[3] = xa[i].w * sc * ga[i].w;
        v[4] = xb[i].x * sc * gb[i].x; v[5] = xb[i].y * sc * gb[i].y;
        v[6] = xb[i].z * sc * gb[i].z; v[7] = xb[i].w * sc * gb[i].w;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int kk = kb + e;
          float xv = 0.f;
          if (row < p.m && kk < p.K) {
            xv = xin[row * p.ldx + kk] * rscale[row];
            if (p.gain) xv *= p.gain[kk];
          }
          v[e] = xv;
        }
      }
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const uint32_t h0 = f2bf_bits(v[2 * e2]), h1 = f2bf_bits(v[2 * e2 + 1]);
        const uint32_t l0 = f2bf_bits(v[2 * e2] - bf_bits2f(h0));
        const uint32_t l1 = f2bf_bits(v[2 * e2 + 1] - bf_bits2f(h1));
        hi[e2] = h0 | (h1 << 16);
        lo[e2] = l0 | (l1 << 16);
      }
      afr[(c * 2 + 0) * 64 + l] = u4{hi[0], hi[1], hi[2], hi[3]};
      afr[(c * 2 + 1) * 64 + l] = u4{lo[0], lo[1], lo[2], lo[3]};
    }
  }
  __syncthreads();

  // ---- weight stream.  Loads are unconditional: indices past the end of
  // the slice are clamped to its last fragment (a cache hit) and their
  // contribution is zeroed, so the loop body has no branches and the
  // compiler keeps two batches of loads in flight.
  if (live) {
    const u4 zero4 = u4{0u, 0u, 0u, 0u};
    if constexpr (WF == W_BF16 || WF == W_F32) {
      constexpr int U = 8 / TPW;
      const u4* wp[TPW];
      const u4* wq[TPW];
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const long long fo = ((long long)(tile0 + t) * p.nkc + c0) * 64 + lane;
        wp[t] = reinterpret_cast<const u4*>(wbase) + fo;
        wq[t] = reinterpret_cast<const u4*>(w2base) + fo;
      }
      u4 b0[U][TPW], b1[U][TPW], q0[U][TPW], q1[U][TPW];
      auto load = [&](u4 (&b)[U][TPW], u4 (&q)[U][TPW], int cb) {
#pragma unroll
        for (int i = 0; i < U; ++i) {
          const long long ci = min(cb + i, nck - 1);
#pragma unroll
          for (int t = 0; t < TPW; ++t) {
            b[i][t] = __builtin_nontemporal_load(wp[t] + ci * 64);
            if constexpr (WF == W_F32) q[i][t] = __builtin_nontemporal_load(wq[t] + ci * 64);
          }
        }
      };
      auto compute = [&](u4 (&b)[U][TPW], u4 (&q)[U][TPW], int cb) {
#pragma unroll
        for (int i = 0; i < U; ++i) {
          const bool ok = cb + i < nck;
          const int ci = min(cb + i, nck - 1);
          const u4 ah = afr[(ci * 2 + 0) * 64 + lane];
          const u4 al = afr[(ci * 2 + 1) * 64 + lane];
#pragma unroll
          for (int t = 0; t < TPW; ++t) {
            const u4 wv = ok ? b[i][t] : zero4;
            acc[t] = mfma(ah, wv, acc[t]);
            acc[t] = mfma(al, wv, acc[t]);
            if constexpr (WF == W_F32) {
              const u4 wl = ok ? q[i][t] : zero4;
              acc[t] = mfma(ah, wl, acc[t]);
              acc[t] = mfma(al, wl, acc[t]);
            }
          }
        }
      };
      load(b0, q0, 0);
      for (int cb = 0; cb < nck; cb += 2 * U) {
        load(b1, q1, cb + U);
        compute(b0, q0, cb);
        load(b0, q0, cb + 2 * U);
        compute(b1, q1, cb + U);
      }
    } else {  // W_INT4: one 1 KB fragment = 16 columns x 128 k (4 chunks)
      constexpr int U = 4;
      const int ngk = p.nkc / 4;          // groups along K
      const int g0 = c0 / 4, ngr = nck / 4;
      const u4* wp[TPW];
      const __half* sp[TPW];
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        wp[t] = reinterpret_cast<const u4*>(wbase) + ((long long)(tile0 + t) * ngk + g0) * 64 + lane;
        sp[t] = reinterpret_cast<const __half*>(w2base) + ((long long)(tile0 + t) * ngk + g0) * 16 + (lane & 15);
      }
      u4 b0[U][TPW], b1[U][TPW];
      float s0[U][TPW], s1[U][TPW];
      auto load = [&](u4 (&b)[U][TPW], float (&s)[U][TPW], int gb) {
#pragma unroll
        for (int i = 0; i < U; ++i) {
          const long long gi = min(gb + i, ngr - 1);
#pragma unroll
          for (int t = 0; t < TPW; ++t) {
            b[i][t] = __builtin_nontemporal_load(wp[t] + gi * 64);
            s[i][t] = __half2float(sp[t][gi * 16]);
          }
        }
      };
      auto compute = [&](u4 (&b)[U][TPW], float (&s)[U][TPW], int gb) {
#pragma unroll
        for (int i = 0; i < U; ++i) {
          const bool ok = gb + i < ngr;
          const int gi = min(gb + i, ngr - 1);
#pragma unroll
          for (int t = 0; t < TPW; ++t) {
            f32x4 g = f32x4{0.f, 0.f, 0.f, 0.f};
            const uint32_t dw[4] = {b[i][t].x, b[i][t].y, b[i][t].z, b[i][t].w};
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) {
              const int c = gi * 4 + cc;
              const u4 wv = nib8_to_bf16(dw[cc]);
              g = mfma(afr[(c * 2 + 0) * 64 + lane], wv, g);
              g = mfma(afr[(c * 2 + 1) * 64 + lane], wv, g);
            }
            acc[t] += (ok ? s[i][t] : 0.f) * g;
          }
        }
      };
      load(b0, s0, 0);
      for (int gb = 0; gb < ngr; gb += 2 * U) {
        load(b1, s1, gb + U);
        compute(b0, s0, gb);
        load(b0, s0, gb + 2 * U);
        compute(b1, s1, gb + U);
      }
    }
  }

  // ---- split-K: partial tiles to scratch, last workgroup reduces in order
  const int npad = p.n_tiles * kTileN;
  if (p.splits > 1) {
    if (live) {
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const int col = (tile0 + t) * kTileN + (lane & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 4 * (lane >> 4) + i;
          if (row < p.m)
            p.ws[((long long)(slot * p.splits + split) * 16 + row) * npad + col] = acc[t][i];
        }
      }
    }
    __threadfence();
    __syncthreads();
    __shared__ int is_last;
    if (threadIdx.x == 0) {
      unsigned* ctr = p.counters + slot * gridDim.x + ng;
      const unsigned prev = atomicAdd(ctr, 1u);
      is_last = (prev == (unsigned)(p.splits - 1));
      if (is_last) atomicExch(ctr, 0u);
    }
    __syncthreads();
    if (!is_last) return;
    __threadfence();
    if (live) {
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const int col = (tile0 + t) * kTileN + (lane & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 4 * (lane >> 4) + i;
          float v = 0.f;
          if (row < p.m)
            for (int s = 0; s < p.splits; ++s)
              v += p.ws[((long long)(slot * p.splits + s) * 16 + row) * npad + col];
          acc[t][i] = v;
        }
      }
    }
  }

  // ---- epilogues
  float* out = p.out + (long long)slot * p.out_stride;
  if constexpr (EPI == EPI_STORE) {
    if (live) {
      const int col = tile0 * kTileN + (lane & 15);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 4 * (lane >> 4) + i;
        if (row < p.m && col < p.N) out[row * p.ldo + col] = acc[0][i];
      }
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    if (live) {
      const int col = (tile0 / 2) * kTileN + (lane & 15);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 4 * (lane >> 4) + i;
        if (row < p.m && col < p.N) {
          const float g = acc[0][i], u = acc[1][i];
          out[row * p.ldo + col] = g / (1.0f + expf(-g)) * u;
        }
      }
    }
  } else if constexpr (EPI == EPI_RESID) {
    const int col = tile0 * kTileN + (lane & 15);
    float sq[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * (lane >> 4) + i;
      float v = 0.f;
      if (live && row < p.m && col < p.N) {
        v = out[row * p.ldo + col] + acc[0][i];
        out[row * p.ldo + col] = v;
      }
      sq[i] = v * v;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) sq[i] += __shfl_xor(sq[i], o, 64);
    }
    if ((lane & 15) == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave * 16 + 4 * (lane >> 4) + i] = sq[i];
    }
    __syncthreads();
    if (threadIdx.x < p.m) {
      const int r = threadIdx.x;
      p.ss_out[r * p.n_ss_out + ng] = ((red[r] + red[16 + r]) + red[32 + r]) + red[48 + r];
    }
  } else {  // EPI_LOGITS
    const int col = tile0 * kTileN + (lane & 15);
    float mx[4], se[4];
    int ix[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * (lane >> 4) + i;
      const bool ok = live && row < p.m && col < p.N;
      if (ok) out[row * p.ldo + col] = acc[0][i];
      mx[i] = ok ? acc[0][i] : -INFINITY;
      ix[i] = ok ? col : 0x7fffffff;
    }
    // (max, lowest index of max) over the 16 columns of the tile
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        const float om = __shfl_xor(mx[i], o, 64);
        const int oi = __shfl_xor(ix[i], o, 64);
        if (om > mx[i] || (om == mx[i] && oi < ix[i])) { mx[i] = om; ix[i] = oi; }
      }
      const int row = 4 * (lane >> 4) + i;
      const float v = (live && row < p.m && col < p.N) ? acc[0][i] : -INFINITY;
      float e = (mx[i] == -INFINITY) ? 0.f : expf(v - mx[i]);
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) e += __shfl_xor(e, o, 64);
      se[i] = e;
    }
    float* rm = red;            // [4][16]
    float* rsum = red + 64;     // [4][16]
    int* ri = reinterpret_cast<int*>(red + 128);  // [4][16]
    if ((lane & 15) == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * (lane >> 4) + i;
        rm[wave * 16 + r] = mx[i];
        rsum[wave * 16 + r] = se[i];
        ri[wave * 16 + r] = ix[i];
      }
    }
    __syncthreads();
    if (threadIdx.x < p.m) {
      const int r = threadIdx.x;
      float M = rm[r];
      int I = ri[r];
      for (int w = 1; w < 4; ++w)
        if (rm[w * 16 + r] > M) { M = rm[w * 16 + r]; I = ri[w * 16 + r]; }
      float S = 0.f;
      for (int w = 0; w < 4; ++w)
        if (rm[w * 16 + r] != -INFINITY) S += rsum[w * 16 + r] * expf(rm[w * 16 + r] - M);
      p.st_max[r * p.n_stat + ng] = M;
      p.st_sum[r * p.n_stat + ng] = S;
      p.st_idx[r * p.n_stat + ng] = I;
    }
  }
}

template <int WF, int EPI>
static hipError_t launch_t(const GemmParams& p, int n_slots, hipStream_t s) {
  constexpr int TPW = (EPI == EPI_SWIGLU) ? 2 : 1;
  const int tiles_per_wg = kWavesPerWG * TPW;
  dim3 grid((p.n_tiles + tiles_per_wg - 1) / tiles_per_wg, p.splits, n_slots);
  const size_t lds = 1024 + (size_t)p.kcs * 2 * 64 * 16;
  static size_t attr_lds = 64 * 1024;
  if (lds > attr_lds) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm<WF, EPI>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_lds = lds;
  }
  hipLaunchKernelGGL((k_gemm<WF, EPI>), grid, dim3(256), lds, s, p);
  return hipGetLastError();
}

hipError_t launch_gemm(int wfmt, int epi, const GemmParams& p, int n_slots, hipStream_t s) {
#define SV_CASE(WF, EP) \
  if (wfmt == WF && epi == EP) return launch_t<WF, EP>(p, n_slots, s);
  SV_CASE(W_BF16, EPI_STORE) SV_CASE(W_BF16, EPI_RESID) SV_CASE(W_BF16, EPI_SWIGLU) SV_CASE(W_BF16, EPI_LOGITS)
  SV_CASE(W_INT4, EPI_STORE) SV_CASE(W_INT4, EPI_RESID) SV_CASE(W_INT4, EPI_SWIGLU) SV_CASE(W_INT4, EPI_LOGITS)
  SV_CASE(W_F32, EPI_STORE) SV_CASE(W_F32, EPI_RESID) SV_CASE(W_F32, EPI_SWIGLU) SV_CASE(W_F32, EPI_LOGITS)
#undef SV_CASE
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------- re-tiling
// Row-major host layout [K][N] -> fragments.  Source n-tile t lands at
// destination n-tile tile_off + t*tile_stride (fuses Q|K|V side by side and
// interleaves gate/up tiles).  K and N tails are zero-filled.
__global__ void k_retile_bf16(const uint16_t* __restrict__ src, int K, int N, uint4* __restrict__ dst,
                              int nkc, int tile_off, int tile_stride) {
  const long long total = (long long)((N + 15) / 16) * nkc * 64;
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < total;
       i += (long long)gridDim.x * blockDim.x) {
    const int l = (int)(i & 63);
    const long long fc = i >> 6;
    const int c = (int)(fc % nkc);
    const int t = (int)(fc / nkc);
    const int n = t * 16 + (l & 15);
    const int kb = c * 32 + (l >> 4) * 8;
    uint32_t w[4];
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      uint32_t a = 0, b = 0;
      if (n < N && kb + 2 * e2 < K) a = src[(long long)(kb + 2 * e2) * N + n];
      if (n < N && kb + 2 * e2 + 1 < K) b = src[(long long)(kb + 2 * e2 + 1) * N + n];
      w[e2] = a | (b << 16);
    }
    const long long dt = (long long)tile_off + (long long)t * tile_stride;
    dst[(dt * nkc + c) * 64 + l] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

__global__ void k_retile_f32(const float* __restrict__ src, int K, int N, uint4* __restrict__ dhi,
                             uint4* __restrict__ dlo, int nkc, int tile_off, int tile_stride) {
  const long long total = (long long)((N + 15) / 16) * nkc * 64;
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < total;
       i += (long long)gridDim.x * blockDim.x) {
    const int l = (int)(i & 63);
    const long long fc = i >> 6;
    const int c = (int)(fc % nkc);
    const int t = (int)(fc / nkc);
    const int n = t * 16 + (l & 15);
    const int kb = c * 32 + (l >> 4) * 8;
    uint32_t hw[4], lw[4];
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      uint32_t hb[2], lb[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int kk = kb + 2 * e2 + h;
        const float v = (n < N && kk < K) ? src[(long long)kk * N + n] : 0.f;
        hb[h] = f2bf_bits(v);
        lb[h] = f2bf_bits(v - bf_bits2f(hb[h]));
      }
      hw[e2] = hb[0] | (hb[1] << 16);
      lw[e2] = lb[0] | (lb[1] << 16);
    }
    const long long dt = (long long)tile_off + (long long)t * tile_stride;
    dhi[(dt * nkc + c) * 64 + l] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
    dlo[(dt * nkc + c) * 64 + l] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
  }
}

// int4: source packed [K/2][N] (even k low nibble) + fp16 scales [K/128][N].
// Fragment (tile, group): lane l holds 4 dwords; dword cc nibble e is
// k = g*128 + cc*32 + 8*(l/16) + e of column l%16.  Scales [tile][group][16].
__global__ void k_retile_int4(const uint8_t* __restrict__ sq, const uint16_t* __restrict__ ss, int K,
                              int N, uint4* __restrict__ dst, uint16_t* __restrict__ dsc, int tile_off,
                              int tile_stride) {
  const int ngk = K / 128;
  const long long total = (long long)((N + 15) / 16) * ngk * 64;
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < total;
       i += (long long)gridDim.x * blockDim.x) {
    const int l = (int)(i & 63);
    const long long fg = i >> 6;
    const int g = (int)(fg % ngk);
    const int t = (int)(fg / ngk);
    const int n = t * 16 + (l & 15);
    uint32_t dw[4];
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      uint32_t d = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int k = g * 128 + cc * 32 + (l >> 4) * 8 + e;
        uint32_t nib = 0;
        if (n < N) nib = (sq[(long long)(k >> 1) * N + n] >> ((k & 1) * 4)) & 0xFu;
        d |= nib << (4 * e);
      }
      dw[cc] = d;
    }
    const long long dt = (long long)tile_off + (long long)t * tile_stride;
    dst[(dt * ngk + g) * 64 + l] = make_uint4(dw[0], dw[1], dw[2], dw[3]);
    if (l < 16) dsc[(dt * ngk + g) * 16 + l] = (n < N) ? ss[(long long)g * N + n] : (uint16_t)0;
  }
}

static dim3 grid_for(long long total) {
  long long b = (total + 255) / 256;
  if (b > 65535) b = 65535;
  if (b < 1) b = 1;
  return dim3((unsigned)b);
}

hipError_t launch_retile_bf16(const uint16_t* src, int K, int N, void* dst, int nkc, int tile_off,
                              int tile_stride, hipStream_t s) {
  const long long total = (long long)((N + 15) / 16) * nkc * 64;
  hipLaunchKernelGGL(k_retile_bf16, grid_for(total), dim3(256), 0, s, src, K, N,
                     static_cast<uint4*>(dst), nkc, tile_off, tile_stride);
  return hipGetLastError();
}

hipError_t launch_retile_f32(const float* src, int K, int N, void* dhi, void* dlo, int nkc,
                             int tile_off, int tile_stride, hipStream_t s) {
  const long long total = (long long)((N + 15) / 16) * nkc * 64;
  hipLaunchKernelGGL(k_retile_f32, grid_for(total), dim3(256), 0, s, src, K, N,
                     static_cast<uint4*>(dhi), static_cast<uint4*>(dlo), nkc, tile_off, tile_stride);
  return hipGetLastError();
}

hipError_t launch_retile_int4(const uint8_t* sq, const uint16_t* ss, int K, int N, void* dst, void* dsc,
                              int tile_off, int tile_stride, int /*n_tiles_total*/, hipStream_t s) {
  const long long total = (long long)((N + 15) / 16) * (K / 128) * 64;
  hipLaunchKernelGGL(k_retile_int4, grid_for(total), dim3(256), 0, s, sq, ss, K, N,
                     static_cast<uint4*>(dst), static_cast<uint16_t*>(dsc), tile_off, tile_stride);
  return hipGetLastError();
}

}  // namespace sv
