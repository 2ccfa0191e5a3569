// Prefill kernels for head dimension 64, 64-row query tiles, paged K/V (block table): every
// workgroup width and gate.
#include "bsfa_device.h"

namespace bsfa {
template hipError_t launch_prefill_tile<64, 64, true>(const PrefillArgs&, int, int,
                                        hipStream_t);
}  // namespace bsfa
