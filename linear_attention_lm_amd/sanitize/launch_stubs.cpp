// Kernel launchers replaced by stubs, for a host-only build of the C ABI's
// argument validation under AddressSanitizer and UndefinedBehaviorSanitizer
// (no device code, no GPU).  Every stub reports hipErrorNotSupported, which
// the ABI returns as BASED_ERR_HIP: the validation tests only make calls that
// the host checks reject, so no stub is reached.
#include "../csrc/launchers.h"

namespace based {

namespace {
hipError_t none() { return hipErrorNotSupported; }
}  // namespace

hipError_t launch_linattn_valu(const LinattnArgs&, bool, hipStream_t) { return none(); }
bool layer_valu_fused(const LinattnArgs&) { return false; }
hipError_t launch_layer_valu(const LinattnArgs&, float*, int, float, bool, hipStream_t) { return none(); }
hipError_t launch_linattn_mfma(const LinattnArgs&, hipStream_t) { return none(); }
hipError_t launch_linattn_decay_mfma(const LinattnArgs&, hipStream_t) { return none(); }
hipError_t launch_linattn_state_records(const void*, const void*, float*, int, int, int, int, int, int, const float*,
                                        int, hipStream_t) {
  return none();
}
hipError_t launch_layer_mfma(const LinattnArgs&, float*, int, float, hipStream_t) { return none(); }
hipError_t launch_swa_valu(const SwaArgs&, bool, hipStream_t) { return none(); }
hipError_t launch_swa_mfma(const SwaArgs&, hipStream_t) { return none(); }
hipError_t launch_swa_bwd(const SwaBwdArgs&, bool, hipStream_t) { return none(); }
bool swa_bwd_mfma_supported(int) { return false; }
hipError_t launch_swa_bwd_mfma(const SwaBwdArgs&, hipStream_t) { return none(); }
hipError_t launch_linattn_bwd_mfma(const LinattnBwdArgs&, hipStream_t) { return none(); }
hipError_t launch_linattn_bwd(const LinattnBwdArgs&, bool, hipStream_t) { return none(); }
hipError_t launch_baseconv(const BaseConvArgs&, bool, hipStream_t) { return none(); }
hipError_t launch_decode_step(const DecodeArgs&, bool, hipStream_t) { return none(); }
hipError_t launch_state_compact(const float*, const float*, float*, float*, size_t, int, hipStream_t) { return none(); }
hipError_t launch_state_expand(const float*, const float*, float*, float*, size_t, int, hipStream_t) { return none(); }
hipError_t launch_decode_prefill(const void*, const void*, void*, void*, int32_t*, int, int, int, int, int, bool,
                                 hipStream_t) {
  return none();
}

}  // namespace based
