// Instantiations of the one-launch decode layer for float caches (their own
// translation unit, so the two dtypes compile in parallel).
#include "fused_kernel.h"

namespace sv {

template hipError_t launch_fused_typed<float>(int, int, int, const ScanArgs&, const AttnArgs&,
                                           const FusedCtl&, const LongSelArgs&,
                                           hipStream_t);

}  // namespace sv
