// Prefill kernels for head dimension 64, 64-row query tiles, contiguous or packed K/V: every
// workgroup width and gate.
#include "bsfa_device.h"

namespace bsfa {
template hipError_t launch_prefill_tile<64, 64, false>(const PrefillArgs&, int, int,
                                        hipStream_t);
}  // namespace bsfa
