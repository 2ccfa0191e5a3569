// Block-mean kernels (mean correction), every head dimension, both K/V layouts.
#include "bsfa_device.h"

namespace bsfa {
template hipError_t launch_means_tile<128, false>(const PrefillArgs&, hipStream_t);
template hipError_t launch_means_tile<128, true>(const PrefillArgs&, hipStream_t);
template hipError_t launch_means_tile<64, false>(const PrefillArgs&, hipStream_t);
template hipError_t launch_means_tile<64, true>(const PrefillArgs&, hipStream_t);
}  // namespace bsfa
