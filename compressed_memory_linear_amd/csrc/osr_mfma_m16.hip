// osr_mfma_m16.hip -- MFMA chunk kernels instantiated for m = 16 slots.
#include "osr_mfma_inst.h"

namespace osr {
namespace mfma {
template int launch_m<16>(int d, bool split, const Params& p, hipStream_t st, const Overlap* ov);
}  // namespace mfma
}  // namespace osr
