// osr_mfma_m64.hip -- MFMA chunk kernels instantiated for m = 64 slots.
#include "osr_mfma_inst.h"

namespace osr {
namespace mfma {
template int launch_m<64>(int d, bool split, const Params& p, hipStream_t st, const Overlap* ov);
}  // namespace mfma
}  // namespace osr
