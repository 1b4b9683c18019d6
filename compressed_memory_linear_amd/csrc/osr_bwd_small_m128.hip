// osr_bwd_small_m128.hip -- the small-chunk reverse walk for m = 128 (kernels: osr_bwd_small.h).
#include "osr_bwd_small.h"

namespace osr {
template int launch_bwd_small_m<128>(int, const BwdParams&, bool, hipStream_t);
}  // namespace osr
