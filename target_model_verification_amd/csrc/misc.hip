// On-device acceptance of the verification step: row statistics on a small
// grid, the rule in its last workgroup, the stochastic draw on a second grid.
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

// The step's result {n_acc, next, kv_len} and, when the caller gave a
// host-visible mirror (pinned host memory), the same three words plus the
// pass's error flag (result[3], written by the pass kernel) stored there with
// system-scope stores, so the host reads them without a device-to-host copy.
__device__ __forceinline__ void put_result(const AcceptParams& p, int n, int next, int len) {
  p.result[0] = n;
  p.result[1] = next;
  p.result[2] = len;
  if (p.result_mirror) {
    const int w[4] = {n, next, len, p.result[3]};
#pragma unroll
    for (int i = 0; i < 4; ++i) __hip_atomic_store(p.result_mirror + i, w[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  }
}

// Cross-workgroup hand-off inside one launch without L2 fences (an agent
// fence in every wave would write back and invalidate its XCD's L2 each
// time): partial results are stored write-through (agent-scope relaxed
// atomic stores), each wave waits for its own stores, the workgroup
// synchronises, one thread takes a ticket, and the last workgroup reads the
// partials with agent-scope loads, which bypass the L2.
__device__ __forceinline__ void wt_store(float* p, float v) {
  __hip_atomic_store((__attribute__((address_space(1))) float*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float agent_load(const float* p) {
  return __hip_atomic_load((__attribute__((address_space(1))) float*)const_cast<float*>(p), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}
// every wave's stores complete, then one ticket per workgroup; true in the
// last workgroup to arrive (which resets the ticket for the next launch)
__device__ __forceinline__ bool last_to_arrive(unsigned* ticket, int* s_flag) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  if (threadIdx.x == 0) {
    auto* t = (__attribute__((address_space(1))) unsigned*)ticket;
    const unsigned old = __hip_atomic_fetch_add(t, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *s_flag = old == gridDim.x - 1;
    if (*s_flag) __hip_atomic_store(t, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  return *s_flag != 0;
}
// Row statistics (max logit, its lowest id, softmax sum) from the LM head's
// per-16-column partials: the grid holds one workgroup per (row, chunk of
// kStatChunk partials); each reduces its chunk, and the last workgroup to
// finish combines the chunks of every row and applies the rule.
constexpr int kStatChunk = 4 * 1024;     // 4 partials per thread
__global__ __launch_bounds__(1024) void k_accept(AcceptParams p) {
  __shared__ int amax[16];
  __shared__ float rowM[16], rowS[16];
  __shared__ float sP[16], sQ[16], sU[16];
  __shared__ int sTok[16], sPar[16];
  __shared__ float redM[kAccWaves], redS[kAccWaves];
  __shared__ int redI[kAccWaves];
  __shared__ int s_is_last;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int m = p.k + 1;
  const int nch = gridDim.x / m;                       // chunks per row
  float* part = p.acc_ws + kAccPart;                   // [m][nch][3]: M, I (bits), S
  // the rule's small operands, loaded alongside the statistics (the last
  // workgroup would otherwise fetch them one dependent load at a time)
  int my_tok = 0, my_par = -1;
  float my_u = 0.f;
  if (tid < m) {
    my_tok = p.tokens[tid];
    if (p.mode == kAcceptTree) my_par = p.parents[tid];
    if (p.mode == 1) my_u = p.u[tid];                  // u has k + 1 entries
  }
  {
    const int row = blockIdx.x / nch, ch = blockIdx.x - row * nch;
    const float* smax = p.st_max + (long long)row * p.n_stat;
    const float* ssum = p.st_sum + (long long)row * p.n_stat;
    const int* sidx = p.st_idx + (long long)row * p.n_stat;
    float v[4], e[4];
    int ix[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int g = ch * kStatChunk + q * 1024 + tid;
      const bool ok = g < p.n_stat;
      v[q] = ok ? smax[g] : -INFINITY;
      ix[q] = ok ? sidx[g] : 0x7fffffff;
      e[q] = ok ? ssum[g] : 0.f;
    }
    float M = -INFINITY;
    int I = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (v[q] > M || (v[q] == M && ix[q] < I)) { M = v[q]; I = ix[q]; }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(M, o, 64);
      const int oi = __shfl_xor(I, o, 64);
      if (ov > M || (ov == M && oi < I)) { M = ov; I = oi; }
    }
    if (lane == 0) { redM[w] = M; redI[w] = I; }
    __syncthreads();
    M = redM[0];
    I = redI[0];
    for (int i = 1; i < kAccWaves; ++i)
      if (redM[i] > M || (redM[i] == M && redI[i] < I)) { M = redM[i]; I = redI[i]; }
    float S = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (v[q] != -INFINITY) S += e[q] * expf(v[q] - M);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) S += __shfl_xor(S, o, 64);
    if (lane == 0) redS[w] = S;
    __syncthreads();
    if (tid == 0) {
      S = 0.f;
      for (int i = 0; i < kAccWaves; ++i) S += redS[i];
      float* pp = part + 3 * (row * nch + ch);
      wt_store(pp, M);
      wt_store(pp + 1, __int_as_float(I));
      wt_store(pp + 2, S);
    }
  }
  // publish the chunk; the last workgroup goes on
  if (!last_to_arrive(reinterpret_cast<unsigned*>(p.acc_ws) + kAccTicket, &s_is_last)) return;
  if (tid < m) { sTok[tid] = my_tok; sPar[tid] = my_par; sU[tid] = my_u; }
  if (w < m) {      // wave w combines row w's chunks: M = max, S = sum of S_c e^(M_c - M)
    float M = -INFINITY, Mc = -INFINITY, Sc = 0.f;
    int I = 0x7fffffff;
    if (lane < nch) {
      const float* pp = part + 3 * (w * nch + lane);
      Mc = agent_load(pp);
      I = __float_as_int(agent_load(pp + 1));
      Sc = agent_load(pp + 2);
      M = Mc;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(M, o, 64);
      const int oi = __shfl_xor(I, o, 64);
      if (ov > M || (ov == M && oi < I)) { M = ov; I = oi; }
    }
    float S = Mc != -INFINITY ? Sc * expf(Mc - M) : 0.f;
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
          if (sPar[i] == cur && sTok[i] == a) { c = i; break; }   // lowest-numbered matching child
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
        while (n < k && sTok[r0 + n + 1] == amax[r0 + n]) ++n;
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
        while (n < p.k && sTok[n + 1] == amax[n]) ++n;
      } else {
        n = p.k;
      }
      put_result(p, n, amax[n], p.L + 1 + n);
    }
    return;
  }
  // stochastic: the k tests' operands side by side, then the tests in order;
  // the draw over the vocabulary follows in k_draw
  if (tid >= 1 && tid <= p.k) {
    const int i = tid, d = sTok[i];
    sP[i] = expf(p.logits[(long long)(i - 1) * p.ldl + d] - rowM[i - 1]) / rowS[i - 1];
    sQ[i] = p.q[(long long)(i - 1) * p.V + d];
  }
  __syncthreads();
  if (tid == 0) {
    int n = p.k, resid = 0;
    for (int i = 1; i <= p.k; ++i) {
      const float P = sP[i], Q = sQ[i];
      if (sU[i - 1] * Q < P) continue;
      n = i - 1;
      resid = 1;
      break;
    }
    // rejection at i: the draw uses row i-1 = n; all accepted: row k = n
    int* di = reinterpret_cast<int*>(p.acc_ws);
    di[kDrawRow] = n;
    di[kDrawResid] = resid;
    p.acc_ws[kDrawM] = rowM[n];
    p.acc_ws[kDrawS] = rowS[n];
  }
}

// The draw of the stochastic rule over the whole vocabulary: next = the
// smallest id x with C(x) > u_{k+1} * C(V-1), C the running sum of the
// weights in ascending id order, weight max(0, p - q) after a rejection (p
// when that is zero everywhere), p otherwise.  Tiles of 64 consecutive ids:
// every wave of the grid sums its tiles' weights (both the residual and the
// plain p weight, so the fallback needs no second sweep) and the last
// workgroup to finish scans the tile sums in id order, finds the first tile
// whose running sum passes the threshold and scans inside it.
__global__ __launch_bounds__(1024) void k_draw(AcceptParams p) {
  __shared__ float tsum[kAccTiles], tpre[kAccTiles], wsum[kAccWaves];
  __shared__ int s_cand, s_last, s_is_last;
  __shared__ float s_total;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int* di = reinterpret_cast<const int*>(p.acc_ws);
  const int row = di[kDrawRow];
  const int resid0 = di[kDrawResid];
  const float M = p.acc_ws[kDrawM], S = p.acc_ws[kDrawS];
  const float u_draw = p.u[p.k];
  const float* lrow = p.logits + (long long)row * p.ldl;
  const float* qrow = resid0 ? p.q + (long long)row * p.V : lrow;   // q has k rows: read only after a rejection
  float* sum_r = p.acc_ws + kDrawHead;
  float* sum_p = sum_r + kAccTiles;
  const int nt = (p.V + 63) / 64;                 // <= kAccTiles (checked at launch)
  for (int t = blockIdx.x * kAccWaves + w; t < nt; t += gridDim.x * kAccWaves) {
    const int x = t * 64 + lane;
    const bool ok = x < p.V;
    const float l = ok ? lrow[x] : 0.f;
    const float qx = ok && resid0 ? qrow[x] : 0.f;
    const float px = expf(l - M) / S;
    float vp = ok ? px : 0.f;
    float vr = ok ? (resid0 ? fmaxf(0.f, px - qx) : px) : 0.f;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      vp += __shfl_xor(vp, o, 64);
      vr += __shfl_xor(vr, o, 64);
    }
    if (lane == 0) {
      wt_store(sum_r + t, vr);
      wt_store(sum_p + t, vp);
    }
  }
  // publish the sums; the last workgroup draws
  if (!last_to_arrive(reinterpret_cast<unsigned*>(p.acc_ws) + kDrawTicket, &s_is_last)) return;
  if (tid == 0) {
    s_cand = 0x7fffffff;
    s_last = -1;
  }
  int resid = resid0;
  for (int pass = 0; pass < 2; ++pass) {
    const float* src = resid ? sum_r : sum_p;
    // thread j: tiles 4j .. 4j+3 in order, then a block scan of the totals
    float loc[4], tot = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 4 * tid + e;
      loc[e] = t < nt ? agent_load(src + t) : 0.f;
      if (t < nt) tsum[t] = loc[e];
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
    const float run = s_total;
    __syncthreads();
    if (resid && !(run > 0.f)) {      // p <= q everywhere: draw from p
      resid = 0;
      continue;
    }
    break;
  }
  const float thr = u_draw * s_total;
  {
    // first tile whose running sum passes the threshold, last tile with weight
    int cand = 0x7fffffff, lastw = -1;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 4 * tid + e;
      if (t < nt && tsum[t] > 0.f) {
        lastw = t;
        if (cand == 0x7fffffff && tpre[t] + tsum[t] > thr) cand = t;
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      cand = min(cand, __shfl_xor(cand, o, 64));
      lastw = max(lastw, __shfl_xor(lastw, o, 64));
    }
    if (lane == 0) {
      atomicMin(&s_cand, cand);
      atomicMax(&s_last, lastw);
    }
  }
  __syncthreads();
  if (w == 0) {
    // the chosen tile (or, when rounding left the threshold unpassed, the
    // last tile holding any weight): first id whose running sum passes the
    // threshold, else the tile's last id with weight
    const int t = s_cand != 0x7fffffff ? s_cand : s_last;
    const int x = t * 64 + lane;
    float v = 0.f;
    if (t >= 0 && x < p.V) {
      const float px = expf(lrow[x] - M) / S;
      v = resid ? fmaxf(0.f, px - qrow[x]) : px;
    }
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
      const int n = di[kDrawRow];
      const int xs = hit ? t * 64 + __builtin_ctzll(hit) : (pos ? t * 64 + 63 - __builtin_clzll(pos) : 0);
      put_result(p, n, xs, p.L + 1 + n);
    }
  }
}

hipError_t launch_accept(const AcceptParams& p, hipStream_t s) {
  if (p.k + 1 > 16 || (p.V + 63) / 64 > kAccTiles) return hipErrorInvalidValue;
  if (!p.acc_ws || p.n_stat > kAccMaxChunks * kStatChunk) return hipErrorInvalidValue;
  const int nch = (p.n_stat + kStatChunk - 1) / kStatChunk;
  hipLaunchKernelGGL(k_accept, dim3((p.k + 1) * nch), dim3(1024), 0, s, p);
  if (p.mode != 1) return hipGetLastError();
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nt = (p.V + 63) / 64;
  const int grid = std::min(256, (nt + kAccWaves - 1) / kAccWaves);
  hipLaunchKernelGGL(k_draw, dim3(grid), dim3(1024), 0, s, p);
  return hipGetLastError();
}

}  // namespace sv
