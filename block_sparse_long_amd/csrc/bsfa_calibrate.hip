// Calibration kernels (per-tile score maxima and kept-mass candidates), every head dimension
// and query tile.
#include "bsfa_device.h"

namespace bsfa {
template hipError_t launch_calibrate_tile<128, 128>(const CalibArgs&, int, hipStream_t);
template hipError_t launch_calibrate_tile<128, 64>(const CalibArgs&, int, hipStream_t);
template hipError_t launch_calibrate_tile<64, 128>(const CalibArgs&, int, hipStream_t);
template hipError_t launch_calibrate_tile<64, 64>(const CalibArgs&, int, hipStream_t);

hipError_t launch_kth_select(const CalibArgs& a, const float* maxima, int block_q,
                             hipStream_t stream) {
  return launch_kth_select_impl(a, maxima, block_q, stream);
}
}  // namespace bsfa
