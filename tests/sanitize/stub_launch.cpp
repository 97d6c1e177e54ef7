// Host-only stand-ins for the kernel launchers of kvm_kernels.hip, so that the
// C-ABI host library (kvm_api.cpp) can be built and exercised under the host
// sanitizers without device code.  Every launcher reports success and does
// nothing; the sanitizer driver only reaches them on paths that never run here
// (a state is never created without a GPU).
#include "kvm_internal.h"

namespace kvm {
int scan_lds_rows(int, bool is_bf16) { return is_bf16 ? 512 : 0; }
hipError_t scratch_address(void** out) {
  *out = nullptr;
  return hipErrorNoDevice;
}
hipError_t launch_noalloc_init(const Dims&, const Dev&, const SchedParams&, double, hipStream_t) { return hipSuccess; }
hipError_t launch_init(const Dims&, const Dev&, double, hipStream_t) { return hipSuccess; }
hipError_t launch_scan(const Dims&, const Dev&, const Src&, int, int, hipStream_t) { return hipSuccess; }
hipError_t launch_attn(const Dims&, const Dev&, const Src&, int64_t, int, int64_t, void*, int, hipStream_t) {
  return hipSuccess;
}
hipError_t launch_rope_keys(const Dims&, const Dev&, const Src&, hipStream_t) { return hipSuccess; }
hipError_t launch_ring_fill(const Dims&, const Dev&, const Src&, int64_t, int64_t, hipStream_t) { return hipSuccess; }
hipError_t launch_seq_reset(const Dims&, const Dev&, int, hipStream_t) { return hipSuccess; }
hipError_t launch_decode(const Dims&, const Dev&, const void*, const void*, const void*, const float*, int64_t, int,
                         void*, hipStream_t, const int64_t*) {
  return hipSuccess;
}
hipError_t launch_snapshot_gather(const Dims&, const Dev&, int, int64_t, int, void*, void*, float*, int*, hipStream_t) {
  return hipSuccess;
}
hipError_t launch_state_load(const Dims&, const Dev&, int, int64_t, hipStream_t) { return hipSuccess; }
hipError_t launch_proj(const ProjArgs&, bool, bool, hipStream_t) { return hipSuccess; }
hipError_t launch_backward(const Dims&, const Dev&, const BwdIn&, const Bwd&, int, hipStream_t) { return hipSuccess; }
}  // namespace kvm
