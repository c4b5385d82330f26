// Fixed device scratch for the verification step of callers that cannot
// allocate device memory while stepping (code under HIP graph capture,
// tight serving loops, harnesses that forbid allocation).
//
// The split-K partial tiles and their arrival tickets of the pass kernel
// normally live in the handle's own workspace.  spec_verify_step_noalloc
// points the kernel at this file-scope array instead.  Host code never uses
// the array's name as an address: its device address is looked up once per
// device (hipGetSymbolAddress, with that device current) and kept.
#include <mutex>

#include "sv_common.h"

namespace sv {

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};
}  // namespace

hipError_t scratch_setup(int device, void** out) {
  *out = nullptr;
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[device]) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != device) return hipErrorInvalidDevice;   // the caller makes `device` current
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_ptr[device] = p;
  }
  *out = g_ptr[device];
  return hipSuccess;
}

// Zeroes n 32-bit words (a kernel, not a memset: it may be captured in a
// graph and replayed).
__global__ void k_zero_u32(unsigned* __restrict__ p, long long n) {
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n; i += (long long)gridDim.x * blockDim.x)
    p[i] = 0u;
}

hipError_t launch_zero_u32(unsigned* p, long long n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  long long b = (n + 255) / 256;
  if (b > 1024) b = 1024;
  hipLaunchKernelGGL(k_zero_u32, dim3((unsigned)b), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

}  // namespace sv
