// osr_bwd_small_m16_d64.hip -- the small-chunk reverse walk for m = 16, d = 64 (kernels: osr_bwd_small.h;
// one translation unit per shape, so the instantiations compile in parallel).
#include "osr_bwd_small.h"

namespace osr {
template int launch_bwd_small_md<16, 64>(const BwdParams&, bool, hipStream_t);
}  // namespace osr
