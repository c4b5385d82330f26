// On-device acceptance of the verification step (one workgroup).
#include "sv_common.h"

namespace sv {

// ------------------------------------------------------------ acceptance
// Greedy (and NONE): a_j = argmax row j (lowest id on ties) from the LM-head
// partials; n_acc = longest prefix with d_i == a_{i-1}; next = a_{n_acc}.
// Stochastic: p_j = softmax(row j); accept d_i iff u_i * q_i(d_i) < p_{i-1}(d_i);
// at the first rejection draw from max(0, p - q) (p if that is all zero),
// else from p_k; draw = smallest x with C(x) > u_{k+1} * C(V-1), C the
// running sum in ascending id order.  result = {n_acc, next, kv_len}.
constexpr int kAccWaves = 16;            // 1024 threads
constexpr int kAccTiles = 4 * 1024;      // 64-id tiles: vocabularies up to 262144 ids
__global__ __launch_bounds__(1024) void k_accept(AcceptParams p) {
  __shared__ int amax[16];
  __shared__ float rowM[16], rowS[16];
  __shared__ float tsum[kAccTiles], tpre[kAccTiles], wsum[kAccWaves];
  __shared__ int s_row, s_resid, s_nacc, s_cand, s_last;
  __shared__ float s_thr, s_total;
  __shared__ float sP[16], sQ[16], sU[16];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int m = p.k + 1;
  constexpr int B = 16;   // loads in flight per lane
  if (w < m) {
    float M = -INFINITY;
    int I = 0x7fffffff;
    const float* smax = p.st_max + (long long)w * p.n_stat;
    const float* ssum = p.st_sum + (long long)w * p.n_stat;
    const int* sidx = p.st_idx + (long long)w * p.n_stat;
    for (int g0 = lane; g0 < p.n_stat; g0 += 64 * B) {
      float v[B];
      int ix[B];
#pragma unroll
      for (int q = 0; q < B; ++q) {
        const int g = g0 + 64 * q;
        v[q] = g < p.n_stat ? smax[g] : -INFINITY;
        ix[q] = g < p.n_stat ? sidx[g] : 0x7fffffff;
      }
#pragma unroll
      for (int q = 0; q < B; ++q)
        if (v[q] > M || (v[q] == M && ix[q] < I)) { M = v[q]; I = ix[q]; }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(M, o, 64);
      const int oi = __shfl_xor(I, o, 64);
      if (ov > M || (ov == M && oi < I)) { M = ov; I = oi; }
    }
    float S = 0.f;
    for (int g0 = lane; g0 < p.n_stat; g0 += 64 * B) {
      float v[B], e[B];
#pragma unroll
      for (int q = 0; q < B; ++q) {
        const int g = g0 + 64 * q;
        v[q] = g < p.n_stat ? smax[g] : -INFINITY;
        e[q] = g < p.n_stat ? ssum[g] : 0.f;
      }
#pragma unroll
      for (int q = 0; q < B; ++q)
        if (v[q] != -INFINITY) S += e[q] * expf(v[q] - M);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) S += __shfl_xor(S, o, 64);
    if (lane == 0) { amax[w] = I; rowM[w] = M; rowS[w] = S; }
  }
  __syncthreads();
  if (p.mode == kAcceptTree) {     // greedy walk down a token tree
    if (tid == 0) {
      int cur = 0, n = 0;
      for (;;) {
        const int a = amax[cur];
        int c = -1;
        for (int i = cur + 1; i < m; ++i)
          if (p.parents[i] == cur && p.tokens[i] == a) { c = i; break; }   // lowest-numbered matching child
        if (c < 0) break;
        p.path[n++] = c;
        cur = c;
      }
      p.result[0] = n;
      p.result[1] = amax[cur];
      p.result[2] = p.L + 1 + n;
    }
    return;
  }
  if (p.mode == kAcceptBatchGreedy || p.mode == kAcceptBatchNone) {   // several sequences' blocks
    if (tid < p.n_seq) {
      const int r0 = p.seq_info[3 * tid + 0], k = p.seq_info[3 * tid + 1], L = p.seq_info[3 * tid + 2];
      int n = 0;
      if (p.mode == kAcceptBatchGreedy) {
        while (n < k && p.tokens[r0 + n + 1] == amax[r0 + n]) ++n;
      } else {
        n = k;
      }
      p.result[4 * tid + 0] = n;
      p.result[4 * tid + 1] = amax[r0 + n];
      p.result[4 * tid + 2] = L + 1 + n;
      p.result[4 * tid + 3] = 0;
    }
    return;
  }
  if (p.mode != 1) {               // greedy / none
    if (tid == 0) {
      int n = 0;
      if (p.mode == 0) {
        while (n < p.k && p.tokens[n + 1] == amax[n]) ++n;
      } else {
        n = p.k;
      }
      p.result[0] = n;
      p.result[1] = amax[n];
      p.result[2] = p.L + 1 + n;
    }
    return;
  }
  // stochastic: the k tests' operands side by side, then the tests in order
  if (tid >= 1 && tid <= p.k) {
    const int i = tid, d = p.tokens[i];
    sP[i] = expf(p.logits[(long long)(i - 1) * p.ldl + d] - rowM[i - 1]) / rowS[i - 1];
    sQ[i] = p.q[(long long)(i - 1) * p.V + d];
    sU[i] = p.u[i - 1];
  }
  __syncthreads();
  if (tid == 0) {
    int n = p.k, resid = 0;
    for (int i = 1; i <= p.k; ++i) {
      const float P = sP[i], Q = sQ[i];
      if (sU[i] * Q < P) continue;
      n = i - 1;
      resid = 1;
      break;
    }
    s_nacc = n;
    s_row = n;          // rejection at i: row i-1 = n; all accepted: row k = n
    s_resid = resid;
    s_cand = 0x7fffffff;
    s_last = -1;
  }
  __syncthreads();
  const int row = s_row;
  const float M = rowM[row], S = rowS[row];
  const float* lrow = p.logits + (long long)row * p.ldl;
  // q has k rows; it is read only for a residual draw (row < k)
  const float* qrow = s_resid ? p.q + (long long)row * p.V : lrow;
  // weight of id x from its logit l and draft probability qx
  auto wfun = [&](float l, float qx, int resid) -> float {
    const float px = expf(l - M) / S;
    return resid ? fmaxf(0.f, px - qx) : px;
  };
  auto weight = [&](int x, int resid) -> float { return wfun(lrow[x], resid ? qrow[x] : 0.f, resid); };
  // Inverse CDF over tiles of 64 consecutive ids: tile sums (one wave per
  // tile, loads coalesced), an exclusive scan of the tile sums in id order,
  // the first tile whose running sum passes the threshold, then a scan
  // inside that tile.
  const int nt = (p.V + 63) / 64;                 // <= kAccTiles (checked at launch)
  const int per = (nt + kAccWaves - 1) / kAccWaves;
  for (int pass = 0; pass < 2; ++pass) {
    const int resid = s_resid;
    const int tend = min(nt, (w + 1) * per);
    for (int t0 = w * per; t0 < tend; t0 += B) {
      float lv[B], qv[B];
#pragma unroll
      for (int q = 0; q < B; ++q) {
        const int x = (t0 + q) * 64 + lane;
        const bool ok = t0 + q < tend && x < p.V;
        lv[q] = ok ? lrow[x] : 0.f;
        qv[q] = ok && resid ? qrow[x] : 0.f;
      }
#pragma unroll
      for (int q = 0; q < B; ++q) {
        const int x = (t0 + q) * 64 + lane;
        float v = (t0 + q < tend && x < p.V) ? wfun(lv[q], qv[q], resid) : 0.f;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
        if (lane == 0 && t0 + q < tend) tsum[t0 + q] = v;
      }
    }
    __syncthreads();
    // thread j: tiles 4j .. 4j+3 in order, then a block scan of the totals
    float loc[4], tot = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 4 * tid + e;
      loc[e] = t < nt ? tsum[t] : 0.f;
      tot += loc[e];
    }
    float inc = tot;   // inclusive scan within the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float y = __shfl_up(inc, o, 64);
      if (lane >= o) inc += y;
    }
    if (lane == 63) wsum[w] = inc;
    __syncthreads();
    if (tid == 0) {
      float run = 0.f;
      for (int i = 0; i < kAccWaves; ++i) {
        const float v = wsum[i];
        wsum[i] = run;
        run += v;
      }
      s_total = run;
    }
    __syncthreads();
    float pre = wsum[w] + inc - tot;   // exclusive prefix of tile 4*tid
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 4 * tid + e;
      if (t < nt) tpre[t] = pre;
      pre += loc[e];
    }
    if (tid == 0) {
      const float run = s_total;
      if (resid && !(run > 0.f)) {
        s_resid = 0;         // p == q everywhere: draw from p
        s_thr = -1.f;
      } else {
        s_thr = p.u[p.k] * run;
      }
    }
    __syncthreads();
    if (s_thr >= 0.f) break;
  }
  {
    const int resid = s_resid;
    const float thr = s_thr;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 4 * tid + e;
      if (t < nt && tsum[t] > 0.f) {
        atomicMax(&s_last, t);
        if (tpre[t] + tsum[t] > thr) atomicMin(&s_cand, t);
      }
    }
    __syncthreads();
    if (w == 0) {
      // the chosen tile (or, when rounding left the threshold unpassed, the
      // last tile holding any weight): first id whose running sum passes
      // the threshold, else the tile's last id with weight
      const int t = s_cand != 0x7fffffff ? s_cand : s_last;
      const int x = t * 64 + lane;
      const float v = (t >= 0 && x < p.V) ? weight(x, resid) : 0.f;
      float c = v;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const float y = __shfl_up(c, o, 64);
        if (lane >= o) c += y;
      }
      c += t >= 0 ? tpre[t] : 0.f;
      const unsigned long long hit = __ballot(v > 0.f && c > thr);
      const unsigned long long pos = __ballot(v > 0.f);
      if (lane == 0) {
        const int xs = hit ? t * 64 + __builtin_ctzll(hit) : (pos ? t * 64 + 63 - __builtin_clzll(pos) : 0);
        p.result[0] = s_nacc;
        p.result[1] = xs;
        p.result[2] = p.L + 1 + s_nacc;
      }
    }
  }
}

hipError_t launch_accept(const AcceptParams& p, hipStream_t s) {
  if (p.k + 1 > 16 || (p.V + 63) / 64 > kAccTiles) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_accept, dim3(1), dim3(1024), 0, s, p);
  return hipGetLastError();
}

}  // namespace sv
