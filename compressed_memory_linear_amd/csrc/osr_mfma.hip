// osr_mfma.hip -- selection of the MFMA chunk schedule (bf16 inputs, C >= 16).
//
// Two schedules evaluate the same chunk formula (eq. recurrence_linear2, or
// eq. recurrence_linear1 on the split schedule only):
//   split: the state-passing kernel (osr_mfma_chain.h; one workgroup per
//          (b,h), sequential over chunks) stores each chunk's start state,
//          gates and h in the workspace; the read-out kernel
//          (osr_mfma_readout.h) then forms every y_t in parallel over chunks.
//   fused: one workgroup per (b,h) does both (osr_mfma_kernels.h); no
//          workspace.
// split wins when B*H alone cannot fill the 256 compute units.
#include <mutex>

#include "osr_launch.h"
#include "osr_mfma_kernels.h"

namespace osr {
namespace mfma {
template <int M>
int launch_m(int d, bool split, const Params& p, hipStream_t st, const Overlap* ov);
template <int M>
int launch_chain_m(int d, const Params& p, hipStream_t st);
template <int M>
int chain_subblock_m(int d, int C);
extern template int chain_subblock_m<16>(int, int);
extern template int chain_subblock_m<32>(int, int);
extern template int chain_subblock_m<64>(int, int);
extern template int chain_subblock_m<128>(int, int);
extern template int launch_m<16>(int, bool, const Params&, hipStream_t, const Overlap*);
extern template int launch_m<32>(int, bool, const Params&, hipStream_t, const Overlap*);
extern template int launch_m<64>(int, bool, const Params&, hipStream_t, const Overlap*);
extern template int launch_m<128>(int, bool, const Params&, hipStream_t, const Overlap*);

// Schedule choice (schedule: 0 automatic, 1 split, 2 fused; the first
// linearisation has no fused form).  The split schedule (state passing, then
// a read-out parallel over chunks) wins while the sequences leave CUs idle;
// the fused kernel, with no workspace round trip, once they fill the device:
// measured crossovers between 128 and 256 (b,h) at d = 128 and between 256
// and 512 at d = 64.
bool use_split(int B, int H, int d, int schedule, bool lin1) {
    if (lin1 || schedule == 1) return true;
    if (schedule == 2) return false;
    const int64_t bh = static_cast<int64_t>(B) * H;
    return bh < 256 || (d <= 64 && bh < 512);
}

int chain_subblock(int m, int d, int C) {
    switch (m) {
        case 16: return chain_subblock_m<16>(d, C);
        case 32: return chain_subblock_m<32>(d, C);
        case 64: return chain_subblock_m<64>(d, C);
        case 128: return chain_subblock_m<128>(d, C);
        default: return 0;
    }
}

// Workgroups per sequence of the state-passing kernel: P = C / C0 when the
// chunk is 2 or 4 of its sub-blocks and there are at most 32 sequences (so
// B*H*P workgroups, one per compute unit -- its LDS use allows no second --
// fit the 256 compute units and every workgroup of a sequence is resident
// while it waits for the others).  Measured (T = 2048 - 4096, split vs one
// workgroup per sequence): m = d = 128, C = 128: 1.49x at 16 sequences,
// 1.26x at 32, 1.00x at 64, 0.91x at 128; m64 d128 C64: 1.09x / 1.09x /
// 1.04x / 1.03x; m = d = 128, C = 64: 1.12x / 1.04x / 0.96x / 0.79x.  Eight
// workgroups of 16 tokens (m = d = 128, C = 128, 16 sequences) measured 6.49
// against 5.06 ms for four of 32: each workgroup loads every other's part of
// the chunk-end state (m d floats each), and that traffic grows with P.
int chain_split_p(int B, int H, int m, int d, int C, int chain_wgs) {
    if (chain_wgs != 0) return 1;
    const int c0 = chain_subblock(m, d, C);
    if (c0 <= 0 || C % c0 != 0) return 1;
    const int P = C / c0;
    if (P != 2 && P != 4) return 1;
    const int64_t bh = static_cast<int64_t>(B) * H;
    return bh <= 32 && bh * P <= 256 ? P : 1;
}

size_t chain_xchg_bytes(int B, int H, int m, int d, int P) {
    if (P <= 1) return 0;
    const size_t per = static_cast<size_t>(m / 16) * (d / 16) * 64 * 4 + static_cast<size_t>(m / 16) * 64;
    return static_cast<size_t>(B) * H * (2 * P * per * sizeof(float) + static_cast<size_t>(P) * (m / 16) * 32 * sizeof(int));
}

// Chunk ranges of an overlapped read-out (split schedule), for a multiple of
// 64 chunks.  With at most 64 state-passing workgroups (three quarters of the
// compute units or more left to the read-out): 4 ranges of 48, 12, 3 and 1
// 64ths of the chunks.  A range's read-out (on the side stream, where it runs
// at about a quarter of the state passing's time per chunk while sharing the
// device) then takes no longer than the next range's state passing, and the
// read-out of the last range, the only one not hidden, is 1/64 of the whole;
// each range boundary costs one event hand-off (~6.5 us), hence no more
// ranges than that.  With 65 to 128 (half the device left to the read-out,
// which then runs at about two thirds of the state passing's time per chunk):
// 4 equal ranges (B8 H16 T4096 m64 d128 C64: 0.67 -> 0.62 ms; 2 equal 0.624,
// 24/16/16/8 64ths 0.649, 20/20/16/8 0.636, 16/16/16/8/8 0.637).  Else 1 (no
// overlap).  Returns the ranges' chunk ends in `end`.
int overlap_ranges(int B, int H, int m, int d, int C, int T, int chain_wgs, int readout_overlap, int* end) {
    const int NC = T / C;
    const int64_t wgs = static_cast<int64_t>(B) * H * chain_split_p(B, H, m, d, C, chain_wgs);
    if (readout_overlap != 0 || wgs > 128 || NC < 64 || NC % 64 != 0) return 1;
    static constexpr int kFew[] = {48, 12, 3, 1}, kHalf[] = {16, 16, 16, 16};
    const int* parts = wgs > 64 ? kHalf : kFew;
    constexpr int kN = 4;
    static_assert(kN <= kMaxRanges, "ranges");
    int n = 0;
    for (int k = 0; k < kN; ++k) {
        n += parts[k] * (NC / 64);
        if (end) end[k] = n;
    }
    return kN;
}

// The side stream and events of the overlapped read-out, one set per device,
// created on first use (default priority) and kept until the process ends.
struct SideStream {
    bool tried = false, ok = false;
    hipStream_t s = nullptr;
    hipEvent_t ev_chain = nullptr, ev_side = nullptr;
};
constexpr int kMaxDev = 64;
SideStream g_side[kMaxDev];
std::mutex g_side_mu;

int device_compute_units() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    return n;
}
}  // namespace mfma

bool mfma_supported(int m, int d, int C) {
    const bool dims = (m == 16 || m == 32 || m == 64 || m == 128) && (d == 16 || d == 32 || d == 64 || d == 128);
    return dims && C >= 16 && C <= 128 && (C & (C - 1)) == 0;
}

size_t mfma_chain_workspace_bytes(int B, int H, int T, int m, int d, int C, bool lin1) {
    // per (b,h,chunk): Z [m][d], g and kappa [m][C], h [d][C] (and e [m][C]), fp32
    const size_t per_chunk = static_cast<size_t>(m) * d + (lin1 ? 3 : 2) * static_cast<size_t>(m) * C +
                             static_cast<size_t>(d) * C;
    return static_cast<size_t>(B) * H * (T / C) * per_chunk * sizeof(float);
}

// The first linearisation runs on the split schedule only.
size_t mfma_workspace_bytes(int B, int H, int T, int m, int d, int C, bool lin1, int schedule, int chain_wgs,
                            int readout_overlap) {
    if (!mfma::use_split(B, H, d, schedule, lin1)) return 0;
    // per-chunk arrays, hand-off buffers of the split state passing, the state
    // handed from one chunk range to the next
    const size_t carry = mfma::overlap_ranges(B, H, m, d, C, T, chain_wgs, readout_overlap, nullptr) > 1
                             ? static_cast<size_t>(B) * H * m * d * sizeof(float) : 0;
    return mfma_chain_workspace_bytes(B, H, T, m, d, C, lin1) +
           mfma::chain_xchg_bytes(B, H, m, d, mfma::chain_split_p(B, H, m, d, C, chain_wgs)) + carry;
}

int launch_mfma_chain_only(int m, int d, const Params& p, hipStream_t st) {
    switch (m) {
        case 16: return mfma::launch_chain_m<16>(d, p, st);
        case 32: return mfma::launch_chain_m<32>(d, p, st);
        case 64: return mfma::launch_chain_m<64>(d, p, st);
        case 128: return mfma::launch_chain_m<128>(d, p, st);
        default: return -3;
    }
}

int launch_mfma_chunked(int m, int d, const Params& p0, hipStream_t st) {
    const bool split = mfma::use_split(p0.B, p0.H, d, p0.schedule, p0.lin1 != 0);
    Params p = p0;
    Overlap ov{};
    ov.nseg = 1;
    std::unique_lock<std::mutex> side_lock;
    if (split) {
        // the state passing split over workgroups: hand-off buffers after the per-chunk arrays
        const int P = mfma::chain_split_p(p.B, p.H, m, d, p.chunk, p.chain_wgs);
        const size_t off = mfma_chain_workspace_bytes(p.B, p.H, p.T, m, d, p.chunk, p.lin1 != 0);
        const size_t xb = mfma::chain_xchg_bytes(p.B, p.H, m, d, P);
        if (P > 1 && static_cast<int64_t>(p.B) * p.H * P <= mfma::device_compute_units()) {
            const size_t per = static_cast<size_t>(m / 16) * (d / 16) * 64 * 4 + static_cast<size_t>(m / 16) * 64;
            p.xbuf = reinterpret_cast<float*>(reinterpret_cast<char*>(p.zbuf) + off);
            p.xflags = reinterpret_cast<int*>(p.xbuf + static_cast<size_t>(p.B) * p.H * 2 * P * per);
            p.chain_p = P;
        }
        // the read-out overlapped with the state passing, by chunk ranges, on the device's side stream
        const int nseg = mfma::overlap_ranges(p.B, p.H, m, d, p.chunk, p.T, p.chain_wgs, p.readout_overlap, ov.end);
        int dev = -1;
        if (nseg > 1 && hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < mfma::kMaxDev) {
            side_lock = std::unique_lock<std::mutex>(mfma::g_side_mu);
            mfma::SideStream& ss = mfma::g_side[dev];
            if (!ss.tried) {
                ss.tried = true;
                ss.ok = hipStreamCreateWithFlags(&ss.s, hipStreamNonBlocking) == hipSuccess &&
                        hipEventCreateWithFlags(&ss.ev_chain, hipEventDisableTiming) == hipSuccess &&
                        hipEventCreateWithFlags(&ss.ev_side, hipEventDisableTiming) == hipSuccess;
            }
            if (ss.ok) {
                ov.nseg = nseg;
                ov.side = ss.s;
                ov.ev_chain = ss.ev_chain;
                ov.ev_side = ss.ev_side;
                p.carry = reinterpret_cast<float*>(reinterpret_cast<char*>(p.zbuf) + off + xb);
            }
        }
    }
    const Overlap* ovp = ov.nseg > 1 ? &ov : nullptr;
    switch (m) {
        case 16: return mfma::launch_m<16>(d, split, p, st, ovp);
        case 32: return mfma::launch_m<32>(d, split, p, st, ovp);
        case 64: return mfma::launch_m<64>(d, split, p, st, ovp);
        case 128: return mfma::launch_m<128>(d, split, p, st, ovp);
        default: return -3;
    }
}

}  // namespace osr
