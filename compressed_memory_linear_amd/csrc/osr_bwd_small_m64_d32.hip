// osr_bwd_small_m64_d32.hip -- the small-chunk reverse walk for m = 64, d = 32 (kernels: osr_bwd_small.h;
// one translation unit per shape, so the instantiations compile in parallel).
#include "osr_bwd_small.h"

namespace osr {
template int launch_bwd_small_md<64, 32>(const BwdParams&, bool, hipStream_t);
}  // namespace osr
