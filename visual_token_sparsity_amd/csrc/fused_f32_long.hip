// Instantiations of the one-launch decode layer for fp32 caches,
// rows of more than 2048 tokens (the parallel
// select): a translation unit of their own, so the dtype and row-mode
// variants compile in parallel.
#include "fused_kernel.h"

namespace sv {

template hipError_t launch_fused_typed<float, true>(int, int, int, const ScanArgs&,
                                                       const AttnArgs&, const FusedCtl&,
                                                       const LongSelArgs&, hipStream_t);

}  // namespace sv
