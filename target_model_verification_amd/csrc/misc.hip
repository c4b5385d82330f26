// Small kernels of the verification pass: embedding gather, MoE routing
// and union build, MoE combine, and on-device acceptance.
#include "sv_common.h"

namespace sv {

// ------------------------------------------------------------ embedding
// x[j][:] = E[tokens[j]][:], plus per-64-column sum-of-squares partials for
// the first RMSNorm (same grouping as the GEMM residual epilogue).
template <bool F32>
__global__ void k_embed(const void* __restrict__ table, const int* __restrict__ tok, int d,
                        float* __restrict__ x, int ldx, float* __restrict__ ss, int n_ss) {
  const int gcol = blockIdx.x, j = blockIdx.y, lane = threadIdx.x;
  const int col = gcol * 64 + lane;
  const long long row = tok[j];
  float v = 0.f;
  if (col < d) {
    if constexpr (F32) v = static_cast<const float*>(table)[row * d + col];
    else v = __uint_as_float(((uint32_t) static_cast<const uint16_t*>(table)[row * d + col]) << 16);
    x[j * ldx + col] = v;
  }
  float s = v * v;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o, 64);
  if (lane == 0) ss[j * n_ss + gcol] = s;
}

hipError_t launch_embed(int emb_f32, const void* table, const int* tokens, int m, int d, float* x,
                        float* ss_out, hipStream_t s) {
  const int ng = (d + 63) / 64;
  const int ldx = ((d + 31) / 32) * 32;
  if (emb_f32)
    hipLaunchKernelGGL(k_embed<true>, dim3(ng, m), dim3(64), 0, s, table, tokens, d, x, ldx, ss_out, ng);
  else
    hipLaunchKernelGGL(k_embed<false>, dim3(ng, m), dim3(64), 0, s, table, tokens, d, x, ldx, ss_out, ng);
  return hipGetLastError();
}

// ------------------------------------------------------------ MoE routing
// One wave per block row: pi = softmax(r + b) over the experts; top_k by
// probability, ties to the lower expert id.  Then the union of the rows'
// selections, listed in ascending expert id; slot_of maps expert -> slot.
__global__ __launch_bounds__(1024) void k_route(RouteParams p) {
  __shared__ int used[256];
  const int tid = threadIdx.x, lane = tid & 63, row = tid >> 6;
  for (int e = tid; e < p.E; e += blockDim.x) used[e] = 0;
  __syncthreads();
  if (row < p.m) {
    constexpr int EPL = 4;                 // experts per lane (E <= 256)
    float z[EPL];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane + 64 * i;
      z[i] = e < p.E ? p.rlogits[row * p.ldr + e] + p.bias[e] : -INFINITY;
      mx = fmaxf(mx, z[i]);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    float pr[EPL], sum = 0.f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      pr[i] = (lane + 64 * i < p.E) ? expf(z[i] - mx) : 0.f;
      sum += pr[i];
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o, 64);
    bool taken[EPL] = {false, false, false, false};
    for (int r = 0; r < p.top_k; ++r) {
      float bv = -INFINITY;
      int bi = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const int e = lane + 64 * i;
        if (e < p.E && !taken[i] && (pr[i] > bv || (pr[i] == bv && e < bi))) { bv = pr[i]; bi = e; }
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        const float ov = __shfl_xor(bv, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
      }
      if (bi >= p.E) bi = 0;               // only reachable with non-finite router logits
      if ((bi & 63) == lane) taken[bi >> 6] = true;
      if (lane == 0) {
        p.sel[row * p.top_k + r] = bi;
        p.selw[row * p.top_k + r] = bv / sum;
        used[bi] = 1;
      }
    }
  }
  __syncthreads();
  if (tid == 0) {
    int cnt = 0;
    for (int e = 0; e < p.E; ++e) {
      if (used[e]) {
        p.slot_of[e] = cnt;
        p.union_list[cnt++] = e;
      } else {
        p.slot_of[e] = -1;
      }
    }
    *p.union_count = cnt;
    if (p.union_hist) *p.union_hist = cnt;
  }
}

hipError_t launch_route(const RouteParams& p, hipStream_t s) {
  if (p.E > 256 || p.m > 16) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_route, dim3(1), dim3(1024), 0, s, p);
  return hipGetLastError();
}

// x_j += sum_r w_{j,r} y[slot(sel_{j,r})]_j + sum_s y[shared slot s]_j,
// in rank order then shared; new sum-of-squares partials per 64 columns.
__global__ void k_moe_combine(MoeCombineParams p) {
  const int gcol = blockIdx.x, j = blockIdx.y, lane = threadIdx.x;
  const int col = gcol * 64 + lane;
  float v = 0.f;
  if (col < p.d) {
    const int uc = *p.union_count;
    float y = 0.f;
    for (int r = 0; r < p.top_k; ++r) {
      const int slot = p.slot_of[p.sel[j * p.top_k + r]];
      y += p.selw[j * p.top_k + r] * p.y[(long long)slot * p.y_stride + j * p.ldy + col];
    }
    for (int s = 0; s < p.n_shared; ++s) y += p.y[(long long)(uc + s) * p.y_stride + j * p.ldy + col];
    v = p.x[j * p.ldx + col] + y;
    p.x[j * p.ldx + col] = v;
  }
  float sq = v * v;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) sq += __shfl_xor(sq, o, 64);
  if (lane == 0) p.ss_out[j * p.n_ss + gcol] = sq;
}

hipError_t launch_moe_combine(const MoeCombineParams& p, hipStream_t s) {
  hipLaunchKernelGGL(k_moe_combine, dim3((p.d + 63) / 64, p.m), dim3(64), 0, s, p);
  return hipGetLastError();
}

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
