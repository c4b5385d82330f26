// Causal verification attention over the paged KV cache (GQA), split-KV.
//
// Block rows j = 0..m-1 sit at positions L+j and see positions t <= L+j
// (the backwards-only rule; essay "LLM Inference: Speculative Decoding",
// "The four sentences are already inside one sentence").  One workgroup
// handles one 64-position chunk (= one KV page) of one KV head for all
// m*G query rows of that head group, so the KV bytes of a chunk are read
// once for all rows.  The workgroup that owns positions L.. L+m-1 first
// applies the rotary embedding to the block's new keys, rounds keys and
// values to the KV dtype, writes them into the cache pages and attends to
// the rounded values (the cache is the single source of keys/values).
// Each chunk emits (max, sum-exp, weighted values) per row; a combine
// kernel merges chunks in ascending order.  Reductions run in a fixed order
// that does not depend on m, and masked / absent keys contribute exact
// zeros, so row j is bitwise identical whatever the block size.
#include "sv_common.h"

namespace sv {

__device__ __forceinline__ uint32_t f2bf_bits_a(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

template <bool KVF32>
__device__ __forceinline__ float kv_load(const void* base, long long idx) {
  if constexpr (KVF32) return static_cast<const float*>(base)[idx];
  else return __uint_as_float(((uint32_t) static_cast<const uint16_t*>(base)[idx]) << 16);
}

// rounds to the KV dtype, stores, and returns the stored value
template <bool KVF32>
__device__ __forceinline__ float kv_store(void* base, long long idx, float v) {
  if constexpr (KVF32) {
    static_cast<float*>(base)[idx] = v;
    return v;
  } else {
    const uint32_t b = f2bf_bits_a(v);
    static_cast<uint16_t*>(base)[idx] = (uint16_t)b;
    return __uint_as_float(b << 16);
  }
}

__device__ __forceinline__ long long kv_index(const AttnParams& p, int t, int g, int sel, int d) {
  const int phys = p.page_table[t / kPage];
  return ((((long long)phys * p.Hkv + g) * 2 + sel) * kPage + (t % kPage)) * p.D + d;
}

template <bool KVF32, int D>
__global__ __launch_bounds__(256) void k_attn(AttnParams p) {
  extern __shared__ __align__(16) float sm[];
  constexpr int DP = D + 1;                  // padded row (bank-conflict free)
  const int c = blockIdx.x, g = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int R = p.R;
  const int t0 = c * kPage;
  const int T = p.L + p.m;
  const int nkeys = min(kPage, T - t0);
  float* Qs = sm;                            // [R][D]
  float* Ks = Qs + R * D;                    // [64][DP]
  float* Vs = Ks + kPage * DP;               // [64][DP]
  float* Ps = Vs + kPage * DP;               // [R][64]
  constexpr int H = D / 2;

  // queries: rotary at position L+j, scaled by 1/sqrt(D)
  for (int i = tid; i < R * D; i += 256) {
    const int r = i / D, d = i % D;
    const int j = r / p.G, hh = r % p.G;
    const int h = g * p.G + hh;
    const float* qrow = p.qkv + (long long)j * p.ldqkv + h * D;
    const int pos = p.L + j;
    const int ii = d < H ? d : d - H;
    const float cs = p.rope_cs[((long long)pos * H + ii) * 2 + 0];
    const float sn = p.rope_cs[((long long)pos * H + ii) * 2 + 1];
    const float a = qrow[ii], b = qrow[ii + H];
    const float v = d < H ? (a * cs - b * sn) : (b * cs + a * sn);
    Qs[r * D + d] = v * p.scale;
  }
  // keys / values of this chunk (new block rows: rotate, round, write to cache)
  for (int i = tid; i < kPage * D; i += 256) {
    const int kk = i / D, d = i % D;
    const int t = t0 + kk;
    float kv_k = 0.f, kv_v = 0.f;
    if (kk < nkeys) {
      if (t < p.L) {
        kv_k = kv_load<KVF32>(p.kv, kv_index(p, t, g, 0, d));
        kv_v = kv_load<KVF32>(p.kv, kv_index(p, t, g, 1, d));
      } else {
        const int j = t - p.L;
        const float* krow = p.qkv + (long long)j * p.ldqkv + (p.Hq + g) * D;
        const float* vrow = p.qkv + (long long)j * p.ldqkv + (p.Hq + p.Hkv + g) * D;
        const int ii = d < H ? d : d - H;
        const float cs = p.rope_cs[((long long)t * H + ii) * 2 + 0];
        const float sn = p.rope_cs[((long long)t * H + ii) * 2 + 1];
        const float a = krow[ii], b = krow[ii + H];
        const float kr = d < H ? (a * cs - b * sn) : (b * cs + a * sn);
        kv_k = kv_store<KVF32>(p.kv, kv_index(p, t, g, 0, d), kr);
        kv_v = kv_store<KVF32>(p.kv, kv_index(p, t, g, 1, d), vrow[d]);
      }
    }
    Ks[kk * DP + d] = kv_k;
    Vs[kk * DP + d] = kv_v;
  }
  __syncthreads();

  // scores: wave w handles rows r = w, w+4, ...; lane = key
  const int tk = t0 + lane;
  for (int r = wave; r < R; r += 4) {
    const int j = r / p.G;
    float s = 0.f;
#pragma unroll 8
    for (int d = 0; d < D; ++d) s += Qs[r * D + d] * Ks[lane * DP + d];
    const bool vis = (lane < nkeys) && (tk <= p.L + j);
    s = vis ? s : -INFINITY;
    float mx = s;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    const float e = (mx == -INFINITY || !vis) ? 0.f : expf(s - mx);
    float sum = e;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o, 64);
    Ps[r * kPage + lane] = e;
    if (lane == 0) {
      const long long pi = ((long long)g * p.n_chunks + c) * R + r;
      p.pm[pi] = mx;
      p.ps[pi] = sum;
    }
  }
  __syncthreads();

  // weighted values: thread -> (row group, d)
  constexpr int RG = 256 / D;
  const int d = tid % D, rg = tid / D;
  for (int r = rg; r < R; r += RG) {
    float a = 0.f;
#pragma unroll 8
    for (int kk = 0; kk < kPage; ++kk) a += Ps[r * kPage + kk] * Vs[kk * DP + d];
    p.pacc[(((long long)g * p.n_chunks + c) * R + r) * D + d] = a;
  }
}

__global__ void k_attn_combine(CombineParams p) {
  const int r = blockIdx.x, g = blockIdx.y, d = threadIdx.x;
  const int R = p.R;
  float M = -INFINITY;
  for (int c = 0; c < p.n_chunks; ++c) M = fmaxf(M, p.pm[((long long)g * p.n_chunks + c) * R + r]);
  float S = 0.f, A = 0.f;
  for (int c = 0; c < p.n_chunks; ++c) {
    const long long pi = ((long long)g * p.n_chunks + c) * R + r;
    const float mc = p.pm[pi];
    const float f = (mc == -INFINITY) ? 0.f : expf(mc - M);
    S += f * p.ps[pi];
    A += f * p.pacc[pi * p.D + d];
  }
  const int j = r / p.G, hh = r % p.G;
  const int h = g * p.G + hh;
  p.o[(long long)j * p.ldo + h * p.D + d] = A / S;
}

static size_t attn_lds(int R, int D) {
  return sizeof(float) * ((size_t)R * D + 2 * kPage * (D + 1) + (size_t)R * kPage);
}

template <bool KVF32, int D>
static hipError_t launch_attn_t(const AttnParams& p, hipStream_t s) {
  const size_t lds = attn_lds(p.R, D);
  static size_t attr_lds = 64 * 1024;
  if (lds > attr_lds) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_attn<KVF32, D>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_lds = lds;
  }
  hipLaunchKernelGGL((k_attn<KVF32, D>), dim3(p.n_chunks, p.Hkv), dim3(256), lds, s, p);
  return hipGetLastError();
}

hipError_t launch_attention(int kv_f32, const AttnParams& p, hipStream_t s) {
  if (attn_lds(p.R, p.D) > 160 * 1024) return hipErrorInvalidValue;
  if (kv_f32) {
    if (p.D == 64) return launch_attn_t<true, 64>(p, s);
    if (p.D == 128) return launch_attn_t<true, 128>(p, s);
  } else {
    if (p.D == 64) return launch_attn_t<false, 64>(p, s);
    if (p.D == 128) return launch_attn_t<false, 128>(p, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_attn_combine(const CombineParams& p, hipStream_t s) {
  hipLaunchKernelGGL(k_attn_combine, dim3(p.R, p.Hq / p.G), dim3(p.D), 0, s, p);
  return hipGetLastError();
}

// prompt cache import: src [Hkv][P][D] (K then V arrays already placed
// back to back: [2][Hkv][P][D]) -> pages
template <typename T>
__global__ void k_kv_import(const T* __restrict__ src, int P, int Hkv, int D, T* __restrict__ base,
                            const int* __restrict__ pt) {
  const long long total = 2LL * Hkv * P * D;
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < total;
       i += (long long)gridDim.x * blockDim.x) {
    const int d = (int)(i % D);
    const long long r = i / D;
    const int t = (int)(r % P);
    const long long r2 = r / P;
    const int g = (int)(r2 % Hkv);
    const int sel = (int)(r2 / Hkv);
    const int phys = pt[t / kPage];
    base[((((long long)phys * Hkv + g) * 2 + sel) * kPage + (t % kPage)) * D + d] = src[i];
  }
}

hipError_t launch_kv_import(int kv_f32, const void* src, int P, int Hkv, int D, void* base,
                            const int* pt, hipStream_t s) {
  const long long total = 2LL * Hkv * P * D;
  long long b = (total + 255) / 256;
  if (b > 65535) b = 65535;
  if (b < 1) b = 1;
  if (kv_f32)
    hipLaunchKernelGGL(k_kv_import<float>, dim3((unsigned)b), dim3(256), 0, s,
                       static_cast<const float*>(src), P, Hkv, D, static_cast<float*>(base), pt);
  else
    hipLaunchKernelGGL(k_kv_import<uint16_t>, dim3((unsigned)b), dim3(256), 0, s,
                       static_cast<const uint16_t*>(src), P, Hkv, D, static_cast<uint16_t*>(base), pt);
  return hipGetLastError();
}

}  // namespace sv
