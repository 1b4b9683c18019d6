// osr_bwd_small_m16_d128.hip -- the small-chunk reverse walk for m = 16, d = 128 (kernels: osr_bwd_small.h;
// one translation unit per shape, so the instantiations compile in parallel).
#include "osr_bwd_small.h"

namespace osr {
template int launch_bwd_small_md<16, 128>(const BwdParams&, bool, hipStream_t);
}  // namespace osr
