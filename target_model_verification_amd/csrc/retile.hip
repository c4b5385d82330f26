// Weight re-tiling into the streaming layout, and the prompt-cache import.
#include "sv_common.h"

namespace sv {

__device__ __forceinline__ uint32_t f2bf_r(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Source: row-major [K][N] (bf16 bits or fp32), or int4 packed [K/2][N]
// (even k in the low nibble) with fp16 scales [K/128][N].  Source 16-column
// tile t lands at destination tile dt = tile_off + t * tile_stride, i.e. unit
// dt / tpu, half dt % tpu; fragment (unit, chunk c) is stored at
// ((sg * nkc + c) * kWaves + w) * tpu + half with sg = unit / kWaves,
// w = unit % kWaves.  bf16 / fp32 fragment lane l holds k = 32c + 8(l/16) + e
// (e = 0..7) of column 16t + l%16; int4 dword cc of lane l holds the
// nibbles of k = 128c + 32cc + 8(l/16) + e, stored offset (u = q + 8, in
// 0..15) with even e = 2j at bits 4j and odd e = 2j+1 at bits 16 + 4j, so
// (dword >> 4j) & 0x000F000F holds the pair (e = 2j, 2j+1) in the low bits
// of each 16-bit half.  K and N tails are zero (u = 8).  With
// pair_dim > 0 the columns of every pair_dim-wide head are taken
// interleaved: destination column 2i + h of a head is source column
// i + h * pair_dim / 2 (rotary pairs side by side).
template <int WF>
__global__ void k_retile(const void* __restrict__ src, const uint16_t* __restrict__ ssc, int K, int N,
                         uint4* __restrict__ dst, uint4* __restrict__ dst2, int nkc, int tpu, int tile_off,
                         int tile_stride, int pair_dim) {
  const int n_src_tiles = (N + 15) / 16;
  const long long total = (long long)n_src_tiles * nkc * 64;
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < total;
       i += (long long)gridDim.x * blockDim.x) {
    const int l = (int)(i & 63);
    const long long fc = i >> 6;
    const int c = (int)(fc % nkc);
    const int t = (int)(fc / nkc);
    const int n = t * 16 + (l & 15);
    int sn = n;   // source column
    if (pair_dim > 0) {
      const int hd = n / pair_dim, p = n - hd * pair_dim;
      sn = hd * pair_dim + (p >> 1) + (p & 1) * (pair_dim >> 1);
    }
    const int dt = tile_off + t * tile_stride;
    const int unit = dt / tpu, half = dt % tpu;
    const int sg = unit / kWaves, w = unit % kWaves;
    const long long fi = (((long long)sg * nkc + c) * kWaves + w) * tpu + half;
    if constexpr (WF == W_INT4) {
      const uint8_t* sq = static_cast<const uint8_t*>(src);
      uint32_t dw[4];
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        uint32_t d = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int k = c * 128 + cc * 32 + (l >> 4) * 8 + e;
          uint32_t nib = 0;   // two's complement q
          if (n < N && k < K) nib = (sq[(long long)(k >> 1) * N + sn] >> ((k & 1) * 4)) & 0xFu;
          d |= (nib ^ 0x8u) << (4 * (e >> 1) + 16 * (e & 1));
        }
        dw[cc] = d;
      }
      dst[fi * 64 + l] = make_uint4(dw[0], dw[1], dw[2], dw[3]);
      if (l < 16) reinterpret_cast<uint16_t*>(dst2)[fi * 16 + l] = (n < N) ? ssc[(long long)c * N + sn] : (uint16_t)0;
    } else {
      const int kb = c * 32 + (l >> 4) * 8;
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        uint32_t hb[2], lb[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int kk = kb + 2 * e2 + hh;
          const bool ok = n < N && kk < K;
          if constexpr (WF == W_F32) {
            const float v = ok ? static_cast<const float*>(src)[(long long)kk * N + sn] : 0.f;
            hb[hh] = f2bf_r(v);
            lb[hh] = f2bf_r(v - __uint_as_float(hb[hh] << 16));
          } else {
            hb[hh] = ok ? static_cast<const uint16_t*>(src)[(long long)kk * N + sn] : 0u;
            lb[hh] = 0;
          }
        }
        hw[e2] = hb[0] | (hb[1] << 16);
        lw[e2] = lb[0] | (lb[1] << 16);
      }
      dst[fi * 64 + l] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
      if constexpr (WF == W_F32) dst2[fi * 64 + l] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
    }
  }
}

static dim3 grid_for(long long total) {
  long long b = (total + 255) / 256;
  if (b > 65535) b = 65535;
  if (b < 1) b = 1;
  return dim3((unsigned)b);
}

hipError_t launch_retile(int wfmt, const void* src, const void* src_scales, int K, int N, void* dst, void* dst2,
                         int nkc, int tpu, int tile_off, int tile_stride, int pair_dim, hipStream_t s) {
  const long long total = (long long)((N + 15) / 16) * nkc * 64;
  const uint16_t* sc = static_cast<const uint16_t*>(src_scales);
  uint4* d1 = static_cast<uint4*>(dst);
  uint4* d2 = static_cast<uint4*>(dst2);
  if (wfmt == W_INT4)
    hipLaunchKernelGGL(k_retile<W_INT4>, grid_for(total), dim3(256), 0, s, src, sc, K, N, d1, d2, nkc, tpu, tile_off,
                       tile_stride, pair_dim);
  else if (wfmt == W_F32)
    hipLaunchKernelGGL(k_retile<W_F32>, grid_for(total), dim3(256), 0, s, src, sc, K, N, d1, d2, nkc, tpu, tile_off,
                       tile_stride, pair_dim);
  else
    hipLaunchKernelGGL(k_retile<W_BF16>, grid_for(total), dim3(256), 0, s, src, sc, K, N, d1, d2, nkc, tpu, tile_off,
                       tile_stride, pair_dim);
  return hipGetLastError();
}

// prompt cache import: src [2][Hkv][P][D] (K then V) -> pages through the
// page table; page block (page, head) holds K as [kPage][D] and V
// transposed as [D][kPage] (the MFMA operands of Q K^T and P V then read 8
// consecutive k per lane from one 16-byte word)
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
    // page block (phys, g): keys [pos][d], then values transposed [d][pos]
    const long long blk = (((long long)phys * Hkv + g) * 2 + sel) * kPage * D;
    base[blk + (sel == 0 ? (long long)(t % kPage) * D + d : (long long)d * kPage + (t % kPage))] = src[i];
  }
}

hipError_t launch_kv_import(int kv_f32, const void* src, int P, int Hkv, int D, void* base, const int* pt,
                            hipStream_t s) {
  const long long total = 2LL * Hkv * P * D;
  if (kv_f32)
    hipLaunchKernelGGL(k_kv_import<float>, grid_for(total), dim3(256), 0, s, static_cast<const float*>(src), P, Hkv,
                       D, static_cast<float*>(base), pt);
  else
    hipLaunchKernelGGL(k_kv_import<uint16_t>, grid_for(total), dim3(256), 0, s, static_cast<const uint16_t*>(src), P,
                       Hkv, D, static_cast<uint16_t*>(base), pt);
  return hipGetLastError();
}

// Every cache element at logical positions [from, to) of every layer and
// KV head set to NaN (debugging aid: dead entries must never be read).
template <typename T>
__global__ void k_kv_poison(T* __restrict__ base, long long layer_elems, int n_layers, int Hkv, int D,
                            const int* __restrict__ pt, int from, int to, T nan) {
  const long long per_layer = 2LL * Hkv * (long long)(to - from) * D;
  const long long total = per_layer * n_layers;
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < total;
       i += (long long)gridDim.x * blockDim.x) {
    const int l = (int)(i / per_layer);
    long long r = i - (long long)l * per_layer;
    const int d = (int)(r % D);
    r /= D;
    const int t = from + (int)(r % (to - from));
    r /= (to - from);
    const int g = (int)(r % Hkv);
    const int sel = (int)(r / Hkv);
    const long long blk = (((long long)pt[t / kPage] * Hkv + g) * 2 + sel) * kPage * D;
    base[(long long)l * layer_elems + blk + (sel == 0 ? (long long)(t % kPage) * D + d : (long long)d * kPage + (t % kPage))] =
        nan;
  }
}

// Cache entries of the accepted token-tree rows moved to consecutive slots:
// row path[j] (slot L + path[j]) -> slot L + 1 + j, keys and values of one
// (layer, KV head) per workgroup.  The path increases, so a destination can
// be the source of an earlier move only; every source element is read into
// registers before any write (at most 15 rows x 2 x 128 elements per 256
// threads).
template <typename T>
__global__ void k_tree_commit(T* __restrict__ base, long long layer_elems, int Hkv, int D,
                              const int* __restrict__ pt, int L, const int* __restrict__ result,
                              const int* __restrict__ path) {
  const int l = blockIdx.x / Hkv, g = blockIdx.x % Hkv;
  const int n = result[0];
  T* lb = base + (long long)l * layer_elems;
  constexpr int kMaxEl = 16 * 2 * 128 / 256;   // rows x (key + value) x head_dim per thread
  T v[kMaxEl];
  long long dst[kMaxEl];
  int cnt = 0;
  for (int e = threadIdx.x; e < n * 2 * D; e += blockDim.x) {
    const int j = e / (2 * D), r = e % (2 * D), sel = r / D, d = r % D;
    const int ts = L + path[j], td = L + 1 + j;
    const long long bs = (((long long)pt[ts / kPage] * Hkv + g) * 2 + sel) * kPage * D;
    const long long bd = (((long long)pt[td / kPage] * Hkv + g) * 2 + sel) * kPage * D;
    const long long os = sel == 0 ? (long long)(ts % kPage) * D + d : (long long)d * kPage + (ts % kPage);
    const long long od = sel == 0 ? (long long)(td % kPage) * D + d : (long long)d * kPage + (td % kPage);
    v[cnt] = lb[bs + os];
    dst[cnt] = bd + od;
    ++cnt;
  }
  __syncthreads();
  for (int i = 0; i < cnt; ++i) lb[dst[i]] = v[i];
}

hipError_t launch_tree_commit(int kv_f32, void* base, long long layer_elems, int n_layers, int Hkv, int D,
                              const int* pt, int L, const int* result, const int* path, hipStream_t s) {
  if (kv_f32)
    hipLaunchKernelGGL(k_tree_commit<float>, dim3(n_layers * Hkv), dim3(256), 0, s, static_cast<float*>(base),
                       layer_elems, Hkv, D, pt, L, result, path);
  else
    hipLaunchKernelGGL(k_tree_commit<uint16_t>, dim3(n_layers * Hkv), dim3(256), 0, s,
                       static_cast<uint16_t*>(base), layer_elems, Hkv, D, pt, L, result, path);
  return hipGetLastError();
}

hipError_t launch_kv_poison(int kv_f32, void* base, long long layer_elems, int n_layers, int Hkv, int D,
                            const int* pt, int from, int to, hipStream_t s) {
  if (to <= from) return hipSuccess;
  const long long total = 2LL * Hkv * (long long)(to - from) * D * n_layers;
  if (kv_f32)
    hipLaunchKernelGGL(k_kv_poison<float>, grid_for(total), dim3(256), 0, s, static_cast<float*>(base), layer_elems,
                       n_layers, Hkv, D, pt, from, to, __builtin_nanf(""));
  else
    hipLaunchKernelGGL(k_kv_poison<uint16_t>, grid_for(total), dim3(256), 0, s, static_cast<uint16_t*>(base),
                       layer_elems, n_layers, Hkv, D, pt, from, to, (uint16_t)0x7FC0u);
  return hipGetLastError();
}

}  // namespace sv
