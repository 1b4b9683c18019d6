// osr_mfma.hip -- MFMA chunk path (placeholder until the kernels land).
#include "osr_launch.h"

namespace osr {

bool mfma_supported(int, int, int) { return false; }
size_t mfma_workspace_bytes(int, int, int, int, int, int) { return 0; }
int launch_mfma_chunked(int, int, const Params&, hipStream_t) { return -3; }

}  // namespace osr
