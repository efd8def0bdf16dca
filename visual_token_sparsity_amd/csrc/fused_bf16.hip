// Instantiations of the one-launch decode layer for bf16_t caches (their own
// translation unit, so the two dtypes compile in parallel).
#include "fused_kernel.h"

namespace sv {

template hipError_t launch_fused_typed<bf16_t>(int, int, int, const ScanArgs&, const AttnArgs&,
                                           const FusedCtl&, const LongSelArgs&,
                                           hipStream_t);

}  // namespace sv
