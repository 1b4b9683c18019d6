// osr_bwd.hip -- dispatch and workspace size of the backward of the chunk-wise
// OSR forward (kernels: osr_bwd_kernel.h, instantiated per slot count in
// osr_bwd_m<M>.hip).
#include "osr_launch.h"

namespace osr {

template <int M>
int launch_bwd_m(int d, const BwdParams& p, bool in_bf16, hipStream_t st);
extern template int launch_bwd_m<16>(int, const BwdParams&, bool, hipStream_t);
extern template int launch_bwd_m<32>(int, const BwdParams&, bool, hipStream_t);
extern template int launch_bwd_m<64>(int, const BwdParams&, bool, hipStream_t);
extern template int launch_bwd_m<128>(int, const BwdParams&, bool, hipStream_t);

int launch_bwd(int m, int d, const BwdParams& p, bool in_bf16, hipStream_t st) {
    switch (m) {
        case 16: return launch_bwd_m<16>(d, p, in_bf16, st);
        case 32: return launch_bwd_m<32>(d, p, in_bf16, st);
        case 64: return launch_bwd_m<64>(d, p, in_bf16, st);
        case 128: return launch_bwd_m<128>(d, p, in_bf16, st);
        default: return -3;
    }
}

// Workspace floats per (b,h): the T/C + 1 chunk-start states, the running state
// before each token of one chunk, and per token c, beta (m each), |h|^2 and pad.
static size_t bwd_floats(int T, int m, int d, int C) {
    return (static_cast<size_t>(T / C) + 1 + C) * m * d + static_cast<size_t>(C) * (2 * m + 4);
}

size_t bwd_workspace_bytes(int B, int H, int T, int m, int d, int C) {
    return bwd_floats(T, m, d, C) * sizeof(float) * static_cast<size_t>(B) * static_cast<size_t>(H);
}

}  // namespace osr
