// Kernel-launch entry points for a host-only build of the library's host code
// (muonh.cpp, adamw.cpp) under AddressSanitizer / UndefinedBehaviorSanitizer.
// The host tests never reach a launch (there is no device), so every stub
// reports that no device is present.
#include "../../pretraining_optimizer_amd/csrc/internal.h"

namespace muonh {

hipError_t launch_gemm(int, int, const GemmProb*, const GemmTile*, int64_t, const MatScalars*,
                       int, int, int, float, float, float, const MatPtrs*, double*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_gemm_small(int, int, const GemmProb*, const GemmTile*, int64_t,
                             const MatScalars*, int, int, float, float, float, const MatPtrs*,
                             double*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_momentum(int, const MomTile*, int64_t, int64_t, const MatGeom*, const MatPtrs*,
                           double*, ElemParams, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_finalize_norm(int32_t, const MatGeom*, const double*, MatScalars*, float,
                                hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_finalize_update(int32_t, const MatGeom*, const double*, MatScalars*,
                                  muonh_stats*, const float*, const double*, ElemParams,
                                  hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_set_eta(int32_t, const float*, float, double*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_update(int, const Chunk*, int64_t, const MatGeom*, const MatPtrs*,
                         const MatScalars*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_radius(const Chunk*, int64_t, const MatPtrs*, double*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_finalize_radius(int32_t, const MatGeom*, const double*, const int32_t*,
                                  MatScalars*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_copy_update(int, const void*, int64_t, float*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_fill_zero(void*, size_t, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_adamw(const Chunk*, int64_t, const AdamwPtrs*, AdamwParams, hipStream_t) {
  return hipErrorNoDevice;
}

}  // namespace muonh
