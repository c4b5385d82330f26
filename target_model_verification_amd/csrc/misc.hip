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
__global__ __launch_bounds__(1024) void k_accept(AcceptParams p) {
  __shared__ int amax[16];
  __shared__ float rowM[16], rowS[16];
  __shared__ float segsum[1024];
  __shared__ int s_row, s_resid, s_nacc, s_cand, s_last;
  __shared__ float s_thr;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int m = p.k + 1;
  if (w < m) {
    float M = -INFINITY;
    int I = 0x7fffffff;
    for (int g = lane; g < p.n_stat; g += 64) {
      const float v = p.st_max[w * p.n_stat + g];
      const int ix = p.st_idx[w * p.n_stat + g];
      if (v > M || (v == M && ix < I)) { M = v; I = ix; }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(M, o, 64);
      const int oi = __shfl_xor(I, o, 64);
      if (ov > M || (ov == M && oi < I)) { M = ov; I = oi; }
    }
    float S = 0.f;
    for (int g = lane; g < p.n_stat; g += 64) {
      const float v = p.st_max[w * p.n_stat + g];
      if (v != -INFINITY) S += p.st_sum[w * p.n_stat + g] * expf(v - M);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) S += __shfl_xor(S, o, 64);
    if (lane == 0) { amax[w] = I; rowM[w] = M; rowS[w] = S; }
  }
  __syncthreads();
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
  // stochastic: sequential tests
  if (tid == 0) {
    int n = p.k, resid = 0;
    for (int i = 1; i <= p.k; ++i) {
      const int d = p.tokens[i];
      const float P = expf(p.logits[(long long)(i - 1) * p.ldl + d] - rowM[i - 1]) / rowS[i - 1];
      const float Q = p.q[(long long)(i - 1) * p.V + d];
      if (p.u[i - 1] * Q < P) continue;
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
  const int seg = (p.V + 1023) / 1024;
  const int x0 = tid * seg, x1 = min(p.V, x0 + seg);
  for (int pass = 0; pass < 2; ++pass) {
    const int resid = s_resid;
    float loc = 0.f;
    for (int x = x0; x < x1; ++x) {
      const float px = expf(lrow[x] - M) / S;
      loc += resid ? fmaxf(0.f, px - qrow[x]) : px;
    }
    segsum[tid] = loc;
    __syncthreads();
    if (tid == 0) {
      float run = 0.f;
      for (int t = 0; t < 1024; ++t) {
        const float v = segsum[t];
        segsum[t] = run;
        run += v;
      }
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
    float c = segsum[tid];
    for (int x = x0; x < x1; ++x) {
      const float px = expf(lrow[x] - M) / S;
      const float wx = resid ? fmaxf(0.f, px - qrow[x]) : px;
      c += wx;
      if (wx > 0.f) atomicMax(&s_last, x);
      if (c > thr && wx > 0.f) { atomicMin(&s_cand, x); break; }
    }
  }
  __syncthreads();
  if (tid == 0) {
    const int x = (s_cand != 0x7fffffff) ? s_cand : s_last;
    p.result[0] = s_nacc;
    p.result[1] = x;
    p.result[2] = p.L + 1 + s_nacc;
  }
}

hipError_t launch_accept(const AcceptParams& p, hipStream_t s) {
  if (p.k + 1 > 16) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_accept, dim3(1), dim3(1024), 0, s, p);
  return hipGetLastError();
}

}  // namespace sv
