// osr_bwd_m32.hip -- backward kernels for m = 32 (one translation unit per slot
// count, so the instantiations compile in parallel).
#include "osr_bwd_kernel.h"

namespace osr {
template int launch_bwd_m<32>(int d, const BwdParams& p, bool in_bf16, hipStream_t st);
}  // namespace osr
