// Device-side entry points of the library, for the host-only AddressSanitizer
// build of the runtime: the driver never launches work, so each reports that
// no device is present.
#include "../../target_model_verification_amd/csrc/sv_common.h"

namespace sv {
hipError_t launch_pass(int, bool, const PassP&, int, size_t, hipStream_t) { return hipErrorNoDevice; }
hipError_t pass_occupancy(int, bool, size_t, int*) { return hipErrorNoDevice; }
hipError_t launch_accept(const AcceptParams&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_retile(int, const void*, const void*, int, int, void*, void*, int, int, int, int, int, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_kv_import(int, const void*, int, int, int, void*, const int*, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_kv_poison(int, void*, long long, int, int, int, const int*, int, int, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_tree_commit(int, void*, long long, int, int, int, const int*, int, const int*, const int*,
                              hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_zero_u32(unsigned*, long long, hipStream_t) { return hipErrorNoDevice; }
hipError_t scratch_setup(int, void**) { return hipErrorNoDevice; }
}  // namespace sv
