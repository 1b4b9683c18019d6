// osr_bwd_small_m128_d64.hip -- the small-chunk reverse walk for m = 128, d = 64 (kernels: osr_bwd_small.h;
// one translation unit per shape, so the instantiations compile in parallel).
#include "osr_bwd_small.h"

namespace osr {
template int launch_bwd_small_md<128, 64>(const BwdParams&, bool, hipStream_t);
}  // namespace osr
