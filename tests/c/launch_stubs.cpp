// Host-only stand-ins for the kernel launchers of libfp8bs.so, linked with
// api.cpp into a sanitizer build of the C-ABI validation layer (g++ with
// -fsanitize=address,undefined; no device code).  The validation tests only
// reach paths that fail before any launch; a stub that is reached anyway
// reports a launch failure, which the tests would see as FP8_ERR_LAUNCH.
#include "kernels.hpp"

namespace fp8bs {

#define FP8BS_STUB return hipErrorInvalidDeviceFunction

hipError_t launch_quant_rows(const uint16_t*, int64_t, int64_t, int64_t, uint8_t*, int64_t, float*, int64_t,
                             const float*, float*, uint32_t*, hipStream_t) { FP8BS_STUB; }
hipError_t launch_quant_cols(const uint16_t*, int64_t, int64_t, int64_t, uint8_t*, int64_t, float*, int64_t,
                             float*, bool, hipStream_t) { FP8BS_STUB; }
hipError_t launch_quant_dual(const uint16_t*, int64_t, int64_t, int64_t, uint8_t*, int64_t, float*, int64_t,
                             uint8_t*, int64_t, float*, int64_t, bool, hipStream_t) { FP8BS_STUB; }
hipError_t launch_quant_weight(const uint16_t*, int64_t, int64_t, int64_t, uint8_t*, int64_t, uint8_t*,
                               int64_t, float*, int64_t, bool, hipStream_t) { FP8BS_STUB; }
hipError_t launch_history_update(float*, const float*, int64_t, float, int, float*, hipStream_t) {
  FP8BS_STUB;
}
hipError_t launch_cast_e4m3(const float*, int64_t, uint8_t*, hipStream_t) { FP8BS_STUB; }
hipError_t launch_pack_tokens(const uint16_t*, int64_t, int64_t, int64_t, const int32_t*, int64_t, uint8_t*,
                              int64_t, hipStream_t) { FP8BS_STUB; }
hipError_t launch_unpack_tokens(const uint8_t*, int64_t, int64_t, int64_t, uint8_t*, int64_t, float*, int64_t,
                                hipStream_t) { FP8BS_STUB; }
hipError_t launch_dequant_tokens(const uint8_t*, int64_t, int64_t, int64_t, uint16_t*, int64_t,
                                 hipStream_t) { FP8BS_STUB; }
hipError_t launch_quant_tiles(const uint16_t*, int64_t, int64_t, int64_t, int, int, uint8_t*, int64_t, float*,
                              int64_t, uint32_t*, hipStream_t) { FP8BS_STUB; }
hipError_t launch_gemm_promotion(const uint8_t*, int64_t, const uint8_t*, int64_t, int64_t, int64_t, int64_t,
                                 int64_t, float*, int64_t, hipStream_t) { FP8BS_STUB; }
hipError_t launch_mfma_probe(int64_t, int, int, const uint8_t*, float*, hipStream_t) { FP8BS_STUB; }
hipError_t launch_recip_online_probe(const float*, float*, int64_t, hipStream_t) { FP8BS_STUB; }
hipError_t launch_gemm(const GemmProblem&, hipStream_t) { FP8BS_STUB; }
hipError_t launch_fused_quant_fprop(const FusedFpropProblem&, hipStream_t) { FP8BS_STUB; }
int device_cus() { return 0; }
hipError_t attach_static_workspace(GemmProblem&, hipStream_t) { FP8BS_STUB; }
int64_t persistent_grid(int64_t ids) { return ids; }

}  // namespace fp8bs
