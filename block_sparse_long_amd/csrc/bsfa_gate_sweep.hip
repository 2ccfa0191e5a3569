// Gate sweep kernels (absolute gate: per-tile score maxima and keep masks), every head
// dimension and query tile, both K/V layouts.
#include "bsfa_device.h"

namespace bsfa {
template hipError_t launch_sweep_tile<128, 128>(const PrefillArgs&, int, hipStream_t);
template hipError_t launch_sweep_tile<128, 64>(const PrefillArgs&, int, hipStream_t);
template hipError_t launch_sweep_tile<64, 128>(const PrefillArgs&, int, hipStream_t);
template hipError_t launch_sweep_tile<64, 64>(const PrefillArgs&, int, hipStream_t);
}  // namespace bsfa
