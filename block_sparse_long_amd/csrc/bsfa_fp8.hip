// FP8 gate kernels: the Q / K quantisation (both K/V layouts) and the FP8 gate sweep, every
// head dimension and query tile.
#include "bsfa_device.h"

namespace bsfa {
template hipError_t launch_quant_tile<128, false>(const PrefillArgs&, hipStream_t);
template hipError_t launch_quant_tile<128, true>(const PrefillArgs&, hipStream_t);
template hipError_t launch_quant_tile<64, false>(const PrefillArgs&, hipStream_t);
template hipError_t launch_quant_tile<64, true>(const PrefillArgs&, hipStream_t);
template hipError_t launch_sweep_fp8_tile<128, 128>(const PrefillArgs&, int, hipStream_t);
template hipError_t launch_sweep_fp8_tile<128, 64>(const PrefillArgs&, int, hipStream_t);
template hipError_t launch_sweep_fp8_tile<64, 128>(const PrefillArgs&, int, hipStream_t);
template hipError_t launch_sweep_fp8_tile<64, 64>(const PrefillArgs&, int, hipStream_t);
}  // namespace bsfa
