// osr_bwd_small_m16.hip -- the small-chunk reverse walk for m = 16 (kernels: osr_bwd_small.h).
#include "osr_bwd_small.h"

namespace osr {
template int launch_bwd_small_m<16>(int, const BwdParams&, bool, hipStream_t);
}  // namespace osr
