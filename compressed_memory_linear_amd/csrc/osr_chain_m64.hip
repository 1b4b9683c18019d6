// osr_chain_m64.hip -- state-passing chunk kernel instantiated for m = 64 slots.
#include "osr_chain_inst.h"

namespace osr {
namespace mfma {
template int launch_chain_m<64>(int d, const Params& p, hipStream_t st);
template int chain_subblock_m<64>(int d, int C);
}  // namespace mfma
}  // namespace osr
