// osr_mfma_m128.hip -- MFMA chunk kernels instantiated for m = 128 slots.
#include "osr_mfma_inst.h"

namespace osr {
namespace mfma {
template int launch_m<128>(int d, bool split, const Params& p, hipStream_t st, const Overlap* ov);
}  // namespace mfma
}  // namespace osr
