// lattice_osr_abi.hip -- the C ABI of liblattice_osr.so (include/lattice_osr.h):
// host-side argument checks, workspace sizing and dispatch to the kernels.
// Every check runs before any HIP call; no C++ exception crosses the ABI.
#include <limits.h>
#include <stdint.h>

#include <mutex>

#include "../../include/lattice_osr.h"
#include "osr_launch.h"

namespace {

bool pow2_dim(int x) { return x == 16 || x == 32 || x == 64 || x == 128; }
bool pow2_chunk(int c) { return c >= 1 && c <= 128 && (c & (c - 1)) == 0; }

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};

Range range_of(const void* p, size_t bytes) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return Range{a, a + bytes};
}

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi; }

// Validate a descriptor; returns 0 or a negative status.
int check_desc(const lattice_osr_desc* d) {
    if (!d) return LATTICE_OSR_ERR_NULL;
    if (d->B <= 0 || d->T <= 0 || d->H <= 0 || d->m <= 0 || d->d <= 0) return LATTICE_OSR_ERR_SHAPE;
    if (static_cast<int64_t>(d->B) * d->H > INT_MAX) return LATTICE_OSR_ERR_SHAPE;
    if (static_cast<int64_t>(d->B) * d->T * d->H > (INT64_C(1) << 40)) return LATTICE_OSR_ERR_SHAPE;
    if (!pow2_dim(d->m) || !pow2_dim(d->d)) return LATTICE_OSR_ERR_UNSUPPORTED;
    if (d->in_dtype != LATTICE_OSR_F32 && d->in_dtype != LATTICE_OSR_BF16) return LATTICE_OSR_ERR_UNSUPPORTED;
    if (d->y_dtype != LATTICE_OSR_F32 && d->y_dtype != LATTICE_OSR_BF16) return LATTICE_OSR_ERR_UNSUPPORTED;
    if (d->mode != LATTICE_OSR_MODE_DEC && d->mode != LATTICE_OSR_MODE_SIM && d->mode != LATTICE_OSR_MODE_ENC)
        return LATTICE_OSR_ERR_UNSUPPORTED;
    if (d->gamma_per_slot != 0 && d->gamma_per_slot != 1) return LATTICE_OSR_ERR_UNSUPPORTED;
    if (d->linearisation != LATTICE_OSR_LIN2 && d->linearisation != LATTICE_OSR_LIN1) return LATTICE_OSR_ERR_UNSUPPORTED;
    if (d->schedule != LATTICE_OSR_SCHED_AUTO && d->schedule != LATTICE_OSR_SCHED_SPLIT &&
        d->schedule != LATTICE_OSR_SCHED_FUSED)
        return LATTICE_OSR_ERR_UNSUPPORTED;
    if (d->chain_pairs != LATTICE_OSR_PAIRS_AUTO && d->chain_pairs != LATTICE_OSR_PAIRS_OFF)
        return LATTICE_OSR_ERR_UNSUPPORTED;
    if (d->chain_wgs != LATTICE_OSR_WGS_AUTO && d->chain_wgs != LATTICE_OSR_WGS_ONE) return LATTICE_OSR_ERR_UNSUPPORTED;
    if (d->readout_overlap != LATTICE_OSR_OVERLAP_AUTO && d->readout_overlap != LATTICE_OSR_OVERLAP_OFF)
        return LATTICE_OSR_ERR_UNSUPPORTED;
    if (d->bwd_form != LATTICE_OSR_BWD_AUTO && d->bwd_form != LATTICE_OSR_BWD_WALK && d->bwd_form != LATTICE_OSR_BWD_CHUNK)
        return LATTICE_OSR_ERR_UNSUPPORTED;
    return LATTICE_OSR_OK;
}

// Which implementation runs a chunked call.
enum class Path { TokenLoop, Mfma };

// bf16 inputs with C >= 16 run on the MFMA kernels (either linearisation).
Path chunk_path(const lattice_osr_desc* d, int C) {
    if (C > 1 && d->in_dtype == LATTICE_OSR_BF16 && osr::mfma_supported(d->m, d->d, C)) return Path::Mfma;
    return Path::TokenLoop;
}

size_t workspace_needed(const lattice_osr_desc* d, int C) {
    if (chunk_path(d, C) == Path::Mfma)
        return osr::mfma_workspace_bytes(d->B, d->H, d->T, d->m, d->d, C, d->linearisation == LATTICE_OSR_LIN1,
                                         d->schedule, d->chain_wgs, d->readout_overlap);
    return 0;
}

// Pointer, alias and workspace checks common to all entry points.
int check_buffers(const lattice_osr_desc* d, const void* q, const void* k, const void* v,
                  const void* gamma, const void* mu, const float* sin, const float* sout,
                  const void* y, const void* ws, size_t ws_bytes, size_t ws_needed) {
    if (!q || !k || !v || !gamma || !mu || !sin || !sout || !y) return LATTICE_OSR_ERR_NULL;
    if (ws_needed > 0 && !ws) return LATTICE_OSR_ERR_NULL;
    if (ws_bytes < ws_needed) return LATTICE_OSR_ERR_WORKSPACE;
    // The kernels move the per-slot and per-column tensors in 16-byte pieces;
    // mu and a per-token gamma are read element by element.
    const size_t ein_align = d->in_dtype == LATTICE_OSR_BF16 ? 2 : 4;
    const void* vec[] = {q, k, v, d->gamma_per_slot ? gamma : nullptr, sin, sout, y, ws};
    for (const void* ptr : vec)
        if (reinterpret_cast<uintptr_t>(ptr) % 16 != 0) return LATTICE_OSR_ERR_ALIGN;
    const void* elem[] = {mu, gamma};
    for (const void* ptr : elem)
        if (reinterpret_cast<uintptr_t>(ptr) % ein_align != 0) return LATTICE_OSR_ERR_ALIGN;

    const size_t ein = d->in_dtype == LATTICE_OSR_BF16 ? 2 : 4;
    const size_t ey = d->y_dtype == LATTICE_OSR_BF16 ? 2 : 4;
    const size_t tok = static_cast<size_t>(d->B) * d->T * d->H;
    const size_t st = static_cast<size_t>(d->B) * d->H * d->m * d->d * sizeof(float);
    const Range rq = range_of(q, tok * d->m * ein), rk = range_of(k, tok * d->m * ein);
    const Range rv = range_of(v, tok * d->d * ein), rmu = range_of(mu, tok * ein);
    const Range rg = range_of(gamma, tok * (d->gamma_per_slot ? d->m : 1) * ein);
    const Range rin = range_of(sin, st), rout = range_of(sout, st);
    const Range ry = range_of(y, tok * d->d * ey);
    const Range rw = range_of(ws, ws_needed);

    if (rin.lo != rout.lo && overlap(rin, rout)) return LATTICE_OSR_ERR_ALIAS;
    const Range others[] = {rq, rk, rv, rg, rmu, rin, rout, rw};
    for (const Range& r : others)
        if (overlap(ry, r)) return LATTICE_OSR_ERR_ALIAS;
    const Range outs_vs_in[] = {rq, rk, rv, rg, rmu};
    for (const Range& r : outs_vs_in)
        if (overlap(rout, r) || overlap(rw, r)) return LATTICE_OSR_ERR_ALIAS;
    if (overlap(rw, rin) || overlap(rw, rout)) return LATTICE_OSR_ERR_ALIAS;
    return LATTICE_OSR_OK;
}

osr::Params make_params(const lattice_osr_desc* d, int C, const void* q, const void* k,
                        const void* v, const void* gamma, const void* mu, const float* sin,
                        float* sout, void* y, void* ws) {
    osr::Params p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.gamma = gamma;
    p.mu = mu;
    p.state_in = sin;
    p.state_out = sout;
    p.y = y;
    p.zbuf = static_cast<float*>(ws);
    p.raw = nullptr;
    p.raw_stride = 0;
    p.raw_c = p.raw_b = p.raw_hh = nullptr;
    p.hrec = nullptr;
    p.B = d->B;
    p.T = d->T;
    p.H = d->H;
    p.chunk = C;
    p.gamma_per_slot = d->gamma_per_slot;
    p.mode = d->mode;
    p.lin1 = d->linearisation == LATTICE_OSR_LIN1 ? 1 : 0;
    p.y_bf16 = d->y_dtype == LATTICE_OSR_BF16 ? 1 : 0;
    p.schedule = d->schedule;
    p.chain_pairs = d->chain_pairs;
    p.chain_wgs = d->chain_wgs;
    p.readout_overlap = d->readout_overlap;
    p.chain_p = 1;
    p.xbuf = nullptr;
    p.xflags = nullptr;
    p.gate = nullptr;
    p.n_begin = 0;
    p.n_end = 0;
    p.carry = nullptr;
    return p;
}

// Backward: pointer, alignment and overlap checks.  Every gradient buffer and
// the workspace is an output; none may overlap another output or any input.
int check_bwd_buffers(const lattice_osr_desc* d, const void* q, const void* k, const void* v,
                      const void* gamma, const void* mu, const float* sin, const void* dy,
                      const float* dso, const float* dq, const float* dk, const float* dv,
                      const float* dgamma, const float* dmu, const float* dsi, const void* ws,
                      size_t ws_bytes, size_t ws_needed) {
    if (!q || !k || !v || !gamma || !mu || !sin || !dy || !dso || !dq || !dk || !dv || !dgamma || !dmu || !dsi)
        return LATTICE_OSR_ERR_NULL;
    if (ws_needed > 0 && !ws) return LATTICE_OSR_ERR_NULL;
    if (ws_bytes < ws_needed) return LATTICE_OSR_ERR_WORKSPACE;
    const size_t ein_align = d->in_dtype == LATTICE_OSR_BF16 ? 2 : 4;
    const void* vec[] = {q, k, v, d->gamma_per_slot ? gamma : nullptr, sin, dy, dso, dv, dsi, ws};
    for (const void* ptr : vec)
        if (reinterpret_cast<uintptr_t>(ptr) % 16 != 0) return LATTICE_OSR_ERR_ALIGN;
    const void* elem[] = {mu, gamma};
    for (const void* ptr : elem)
        if (reinterpret_cast<uintptr_t>(ptr) % ein_align != 0) return LATTICE_OSR_ERR_ALIGN;
    const void* f32s[] = {dq, dk, dgamma, dmu};
    for (const void* ptr : f32s)
        if (reinterpret_cast<uintptr_t>(ptr) % 4 != 0) return LATTICE_OSR_ERR_ALIGN;

    const size_t ein = d->in_dtype == LATTICE_OSR_BF16 ? 2 : 4;
    const size_t ey = d->y_dtype == LATTICE_OSR_BF16 ? 2 : 4;
    const size_t tok = static_cast<size_t>(d->B) * d->T * d->H;
    const size_t gsz = tok * (d->gamma_per_slot ? d->m : 1);
    const size_t st = static_cast<size_t>(d->B) * d->H * d->m * d->d * sizeof(float);
    const Range ins[] = {range_of(q, tok * d->m * ein), range_of(k, tok * d->m * ein),
                         range_of(v, tok * d->d * ein), range_of(gamma, gsz * ein), range_of(mu, tok * ein),
                         range_of(sin, st), range_of(dy, tok * d->d * ey), range_of(dso, st)};
    const Range outs[] = {range_of(dq, tok * d->m * 4), range_of(dk, tok * d->m * 4),
                          range_of(dv, tok * d->d * 4), range_of(dgamma, gsz * 4), range_of(dmu, tok * 4),
                          range_of(dsi, st), range_of(ws, ws_needed)};
    const int nout = sizeof(outs) / sizeof(outs[0]);
    for (int i = 0; i < nout; ++i) {
        for (const Range& r : ins)
            if (overlap(outs[i], r)) return LATTICE_OSR_ERR_ALIAS;
        for (int j = i + 1; j < nout; ++j)
            if (overlap(outs[i], outs[j])) return LATTICE_OSR_ERR_ALIAS;
    }
    return LATTICE_OSR_OK;
}

// The backward takes its chunk-start states from the matrix-core state-passing
// kernel where the forward would run on it (bf16 inputs, C >= 16), except for
// the encoding layer, whose gradient is too sensitive to the split products'
// rounding; otherwise its own fp32 forward pass finds them.
// Compute units of the current device (0 if the query fails: no split then).
int64_t device_cus() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    return n;
}

bool bwd_uses_chain(const lattice_osr_desc* d, int C) {
    return d->in_dtype == LATTICE_OSR_BF16 && C >= 16 && osr::mfma_supported(d->m, d->d, C) &&
           d->mode != LATTICE_OSR_MODE_ENC;
}

// With the state-passing kernel, the backward's workspace is its own part, then
// that kernel's per-chunk arrays (Z, g, kappa, h[, e]), then c, beta (m x C)
// and |h|^2 (C) of every chunk.
size_t bwd_chain_extra_bytes(const lattice_osr_desc* d, int C) {
    const size_t nch = static_cast<size_t>(d->B) * d->H * (d->T / C);
    return nch * (2 * static_cast<size_t>(d->m) * C + C) * sizeof(float);
}

// The small-chunk reverse walk where it is built, not turned off, and the fewest
// workgroups per sequence it needs fit 256 compute units: C <= 8 after the token
// loop, C = 16 after the state-passing kernel (bf16 inputs, not the encoding layer).
bool bwd_small_form(const lattice_osr_desc* d, int C) {
    return d->bwd_form == LATTICE_OSR_BWD_AUTO && (C <= 8 || (C == 16 && bwd_uses_chain(d, C))) &&
           osr::bwd_small_supported(d->m, d->d, C, d->linearisation == LATTICE_OSR_LIN1) &&
           static_cast<int64_t>(d->B) * d->H * osr::bwd_small_min_p(d->m, d->d, C) <= 256;
}

// With the small-chunk walk and the decoding objective, the backward's part is
// followed by every token's h (fp32 [B*H][T][d]).
size_t bwd_small_h_bytes(const lattice_osr_desc* d, int C) {
    if (C > 8 || !bwd_small_form(d, C) || d->mode != LATTICE_OSR_MODE_DEC) return 0;
    return static_cast<size_t>(d->B) * d->H * d->T * d->d * sizeof(float);
}

// Workgroups per sequence that the workspace provides hand-off buffers for (the
// launch may use fewer where the device has fewer compute units).
int bwd_parts(const lattice_osr_desc* d, int C) {
    if (bwd_small_form(d, C)) return osr::bwd_small_split_p(d->B, d->H, d->m, d->d, C, d->chain_wgs);
    return osr::bwd_split_p(d->B, d->H, d->m, d->d, C, bwd_uses_chain(d, C), d->chain_wgs);
}

// ... then, where the slot rows of a sequence split over several workgroups,
// their hand-off buffers.
size_t bwd_workspace_needed(const lattice_osr_desc* d, int C) {
    size_t n = osr::bwd_workspace_bytes(d->B, d->H, d->T, d->m, d->d, C);
    const bool chain = bwd_uses_chain(d, C);
    if (chain)
        n += osr::mfma_chain_workspace_bytes(d->B, d->H, d->T, d->m, d->d, C, d->linearisation == LATTICE_OSR_LIN1) +
             bwd_chain_extra_bytes(d, C);
    n += bwd_small_h_bytes(d, C);
    if (bwd_small_form(d, C)) return n + osr::bwd_small_xchg_bytes(d->B, d->H, d->d, bwd_parts(d, C), C);
    return n + osr::bwd_xchg_bytes(d->B, d->H, d->d, bwd_parts(d, C));
}

// Parameters of the small-chunk backward's phase 1 (the forward's small-chunk
// token loop): every chunk-start state before projection, and the end state,
// into the backward's workspace layout and, decoding objective, every token's
// h after the backward's part; y and state_out as given (null: not written).
osr::Params small_phase1_params(const lattice_osr_desc* desc, int C, const void* q, const void* k, const void* v,
                                const void* gamma, const void* mu, const float* state_in, float* state_out,
                                void* y, void* workspace) {
    const size_t bwd_bytes = osr::bwd_workspace_bytes(desc->B, desc->H, desc->T, desc->m, desc->d, C);
    osr::Params pf = make_params(desc, C, q, k, v, gamma, mu, state_in, state_out, y, nullptr);
    pf.raw = static_cast<float*>(workspace);
    pf.raw_stride = static_cast<int64_t>(bwd_bytes / sizeof(float)) / (static_cast<int64_t>(desc->B) * desc->H);
    pf.hrec = bwd_small_h_bytes(desc, C) ? reinterpret_cast<float*>(static_cast<char*>(workspace) + bwd_bytes)
                                         : nullptr;
    return pf;
}

// The chunk-parallel backward where it is built and not turned off.
bool bwd_chunk_form(const lattice_osr_desc* d, int C) {
    return d->bwd_form != LATTICE_OSR_BWD_WALK && bwd_uses_chain(d, C) &&
           osr::bwd_chunk_supported(d->m, d->d, C, d->in_dtype == LATTICE_OSR_BF16,
                                    d->linearisation == LATTICE_OSR_LIN1, d->mode);
}

// Shape rules of the backward: those of the chunked forward.
int check_bwd_desc(const lattice_osr_desc* d, int C) {
    int rc = check_desc(d);
    if (rc) return rc;
    if (C <= 0 || d->T % C != 0) return LATTICE_OSR_ERR_SHAPE;
    if (!pow2_chunk(C)) return LATTICE_OSR_ERR_UNSUPPORTED;
    if (d->bwd_form == LATTICE_OSR_BWD_CHUNK && !bwd_chunk_form(d, C)) return LATTICE_OSR_ERR_UNSUPPORTED;
    return LATTICE_OSR_OK;
}

}  // namespace

extern "C" {

int lattice_osr_abi_version(void) { return LATTICE_OSR_ABI_VERSION; }

const char* lattice_osr_status_string(int status) {
    switch (status) {
        case LATTICE_OSR_OK: return "ok";
        case LATTICE_OSR_ERR_NULL: return "null pointer argument";
        case LATTICE_OSR_ERR_SHAPE: return "bad shape (non-positive dimension, T % chunk_size != 0, or T != 1 for decode)";
        case LATTICE_OSR_ERR_UNSUPPORTED: return "unsupported configuration (m, d, chunk size, dtype, mode or gamma layout)";
        case LATTICE_OSR_ERR_WORKSPACE: return "workspace too small";
        case LATTICE_OSR_ERR_LAUNCH: return "kernel launch failed";
        case LATTICE_OSR_ERR_ALIAS: return "forbidden overlap between arguments";
        case LATTICE_OSR_ERR_ALIGN: return "misaligned pointer argument";
        default: return "unknown status";
    }
}

size_t lattice_osr_workspace_bytes(const lattice_osr_desc* desc, int32_t chunk_size) {
    if (check_desc(desc) != LATTICE_OSR_OK || !pow2_chunk(chunk_size) || desc->T % chunk_size != 0)
        return static_cast<size_t>(-1);
    return workspace_needed(desc, chunk_size);
}

int lattice_osr_fwd_chunked(const lattice_osr_desc* desc, int32_t chunk_size, const void* q,
                            const void* k, const void* v, const void* gamma, const void* mu,
                            const float* state_in, float* state_out, void* y, void* workspace,
                            size_t workspace_bytes, void* hip_stream) {
    int rc = check_desc(desc);
    if (rc) return rc;
    if (chunk_size <= 0 || desc->T % chunk_size != 0) return LATTICE_OSR_ERR_SHAPE;
    if (!pow2_chunk(chunk_size)) return LATTICE_OSR_ERR_UNSUPPORTED;
    const size_t need = workspace_needed(desc, chunk_size);
    rc = check_buffers(desc, q, k, v, gamma, mu, state_in, state_out, y, workspace, workspace_bytes, need);
    if (rc) return rc;
    const osr::Params p = make_params(desc, chunk_size, q, k, v, gamma, mu, state_in, state_out, y, workspace);
    hipStream_t st = static_cast<hipStream_t>(hip_stream);
    if (chunk_path(desc, chunk_size) == Path::Mfma) return osr::launch_mfma_chunked(desc->m, desc->d, p, st);
    return osr::launch_valu(false, desc->m, desc->d, p, desc->in_dtype == LATTICE_OSR_BF16, st);
}

int lattice_osr_fwd_chunked_gated(const lattice_osr_desc* desc, int32_t chunk_size, const void* q,
                                  const void* k, const void* v, const void* gamma, const void* mu,
                                  const void* gate, const float* state_in, float* state_out, void* y,
                                  void* workspace, size_t workspace_bytes, void* hip_stream) {
    int rc = check_desc(desc);
    if (rc) return rc;
    if (chunk_size <= 0 || desc->T % chunk_size != 0) return LATTICE_OSR_ERR_SHAPE;
    if (!pow2_chunk(chunk_size)) return LATTICE_OSR_ERR_UNSUPPORTED;
    const size_t need = workspace_needed(desc, chunk_size);
    rc = check_buffers(desc, q, k, v, gamma, mu, state_in, state_out, y, workspace, workspace_bytes, need);
    if (rc) return rc;
    // the gate is one more input: [B,T,H,d] in_dtype, 16-byte aligned, overlapping no output
    if (!gate) return LATTICE_OSR_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(gate) % 16 != 0) return LATTICE_OSR_ERR_ALIGN;
    const size_t ein = desc->in_dtype == LATTICE_OSR_BF16 ? 2 : 4;
    const size_t ey = desc->y_dtype == LATTICE_OSR_BF16 ? 2 : 4;
    const size_t tok = static_cast<size_t>(desc->B) * desc->T * desc->H;
    const size_t st = static_cast<size_t>(desc->B) * desc->H * desc->m * desc->d * sizeof(float);
    const Range rg = range_of(gate, tok * desc->d * ein);
    if (overlap(rg, range_of(y, tok * desc->d * ey)) || overlap(rg, range_of(state_out, st)) ||
        overlap(rg, range_of(workspace, need)))
        return LATTICE_OSR_ERR_ALIAS;
    osr::Params p = make_params(desc, chunk_size, q, k, v, gamma, mu, state_in, state_out, y, workspace);
    p.gate = gate;
    hipStream_t hs = static_cast<hipStream_t>(hip_stream);
    if (chunk_path(desc, chunk_size) == Path::Mfma) return osr::launch_mfma_chunked(desc->m, desc->d, p, hs);
    return osr::launch_valu(false, desc->m, desc->d, p, desc->in_dtype == LATTICE_OSR_BF16, hs);
}

}  // extern "C"

// Scratch of lattice_osr_fwd_chunked_noalloc: the workspace of the split
// schedule in device memory the library owns, one copy per GPU (held until
// the process ends).  In host code `scratch` names a host-side stand-in, not
// a device address: its address on a device comes from hipGetSymbolAddress,
// taken once per device with that device current and kept here.
namespace {
constexpr size_t kScratchBytes = static_cast<size_t>(64) << 20;  // LATTICE_OSR_NOALLOC_SCRATCH_BYTES
__device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
void* scratch_dev[kMaxDevices];
std::mutex scratch_mu;

// The current device's copy of the scratch array (its address, looked up on
// the first use on that device).
int scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return LATTICE_OSR_ERR_LAUNCH;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_dev[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return LATTICE_OSR_ERR_LAUNCH;
        scratch_dev[dev] = ptr;
    }
    *out = scratch_dev[dev];
    return LATTICE_OSR_OK;
}
}  // namespace

extern "C" {

int lattice_osr_fwd_chunked_noalloc(const lattice_osr_desc* desc, int32_t chunk_size, const void* q,
                                    const void* k, const void* v, const void* gamma, const void* mu,
                                    const float* state_in, float* state_out, void* y, void* hip_stream) {
    int rc = check_desc(desc);
    if (rc) return rc;
    if (chunk_size <= 0 || desc->T % chunk_size != 0) return LATTICE_OSR_ERR_SHAPE;
    if (!pow2_chunk(chunk_size)) return LATTICE_OSR_ERR_UNSUPPORTED;
    // everything on the caller's stream: no side stream or events are touched
    lattice_osr_desc dl = *desc;
    dl.readout_overlap = LATTICE_OSR_OVERLAP_OFF;
    desc = &dl;
    const size_t need = workspace_needed(desc, chunk_size);
    if (need > kScratchBytes) return LATTICE_OSR_ERR_WORKSPACE;
    // inputs and outputs as for lattice_osr_fwd_chunked (the scratch overlaps nothing of the caller's)
    rc = check_buffers(desc, q, k, v, gamma, mu, state_in, state_out, y, nullptr, 0, 0);
    if (rc) return rc;
    void* ws = nullptr;
    if (need > 0) {
        rc = scratch_address(&ws);
        if (rc) return rc;
    }
    const osr::Params p = make_params(desc, chunk_size, q, k, v, gamma, mu, state_in, state_out, y, ws);
    hipStream_t st = static_cast<hipStream_t>(hip_stream);
    if (chunk_path(desc, chunk_size) == Path::Mfma) return osr::launch_mfma_chunked(desc->m, desc->d, p, st);
    return osr::launch_valu(false, desc->m, desc->d, p, desc->in_dtype == LATTICE_OSR_BF16, st);
}

int lattice_osr_fwd_recurrent(const lattice_osr_desc* desc, const void* q, const void* k,
                              const void* v, const void* gamma, const void* mu,
                              const float* state_in, float* state_out, void* y, void* workspace,
                              size_t workspace_bytes, void* hip_stream) {
    int rc = check_desc(desc);
    if (rc) return rc;
    rc = check_buffers(desc, q, k, v, gamma, mu, state_in, state_out, y, workspace, workspace_bytes, 0);
    if (rc) return rc;
    const osr::Params p = make_params(desc, 1, q, k, v, gamma, mu, state_in, state_out, y, workspace);
    return osr::launch_valu(false, desc->m, desc->d, p, desc->in_dtype == LATTICE_OSR_BF16,
                            static_cast<hipStream_t>(hip_stream));
}

int lattice_osr_decode_step(const lattice_osr_desc* desc, const void* q, const void* k,
                            const void* v, const void* gamma, const void* mu,
                            const float* state_in, float* state_out, void* y, void* workspace,
                            size_t workspace_bytes, void* hip_stream) {
    int rc = check_desc(desc);
    if (rc) return rc;
    if (desc->T != 1) return LATTICE_OSR_ERR_SHAPE;
    rc = check_buffers(desc, q, k, v, gamma, mu, state_in, state_out, y, workspace, workspace_bytes, 0);
    if (rc) return rc;
    const osr::Params p = make_params(desc, 1, q, k, v, gamma, mu, state_in, state_out, y, workspace);
    return osr::launch_valu(true, desc->m, desc->d, p, desc->in_dtype == LATTICE_OSR_BF16,
                            static_cast<hipStream_t>(hip_stream));
}

}  // extern "C"

extern "C" {

size_t lattice_osr_bwd_workspace_bytes(const lattice_osr_desc* desc, int32_t chunk_size) {
    if (check_bwd_desc(desc, chunk_size) != LATTICE_OSR_OK) return static_cast<size_t>(-1);
    return bwd_workspace_needed(desc, chunk_size);
}

}  // extern "C"

namespace {

// saved: the workspace already holds what lattice_osr_fwd_chunked_save stored
// (small-chunk form only): the forward pass of phase 1 is skipped.
int bwd_chunked_impl(const lattice_osr_desc* desc, int32_t chunk_size, const void* q, const void* k, const void* v,
                     const void* gamma, const void* mu, const float* state_in, const void* dy,
                     const float* dstate_out, float* dq, float* dk, float* dv, float* dgamma, float* dmu,
                     float* dstate_in, void* workspace, size_t workspace_bytes, void* hip_stream, bool saved) {
    int rc = check_bwd_desc(desc, chunk_size);
    if (rc) return rc;
    if (saved && (chunk_size > 8 || !bwd_small_form(desc, chunk_size))) return LATTICE_OSR_ERR_UNSUPPORTED;
    const size_t need = bwd_workspace_needed(desc, chunk_size);
    rc = check_bwd_buffers(desc, q, k, v, gamma, mu, state_in, dy, dstate_out, dq, dk, dv, dgamma, dmu,
                           dstate_in, workspace, workspace_bytes, need);
    if (rc) return rc;
    hipStream_t st = static_cast<hipStream_t>(hip_stream);
    const bool chain = bwd_uses_chain(desc, chunk_size);
    if (chain) {
        // chunk-start states (before projection) straight into the backward's part of the
        // workspace; the state-passing kernel's own per-chunk arrays follow it
        const size_t bwd_bytes = osr::bwd_workspace_bytes(desc->B, desc->H, desc->T, desc->m, desc->d, chunk_size);
        const bool lin1 = desc->linearisation == LATTICE_OSR_LIN1;
        const size_t chain_bytes =
            osr::mfma_chain_workspace_bytes(desc->B, desc->H, desc->T, desc->m, desc->d, chunk_size, lin1);
        const int64_t nch = static_cast<int64_t>(desc->B) * desc->H * (desc->T / chunk_size);
        osr::Params pc = make_params(desc, chunk_size, q, k, v, gamma, mu, state_in, nullptr, nullptr,
                                     static_cast<char*>(workspace) + bwd_bytes);
        pc.raw = static_cast<float*>(workspace);
        pc.raw_stride = static_cast<int64_t>(bwd_bytes / sizeof(float)) / (static_cast<int64_t>(desc->B) * desc->H);
        pc.raw_c = reinterpret_cast<float*>(static_cast<char*>(workspace) + bwd_bytes + chain_bytes);
        pc.raw_b = pc.raw_c + nch * desc->m * chunk_size;
        pc.raw_hh = pc.raw_b + nch * desc->m * chunk_size;
        rc = osr::launch_mfma_chain_only(desc->m, desc->d, pc, st);
        if (rc) return rc;
    }
    osr::BwdParams p;
    p.f = make_params(desc, chunk_size, q, k, v, gamma, mu, state_in, nullptr, nullptr, nullptr);
    p.dy = dy;
    p.dstate_out = dstate_out;
    p.dq = dq;
    p.dk = dk;
    p.dv = dv;
    p.dgamma = dgamma;
    p.dmu = dmu;
    p.dstate_in = dstate_in;
    p.ws = static_cast<float*>(workspace);
    p.dy_bf16 = desc->y_dtype == LATTICE_OSR_BF16 ? 1 : 0;
    p.states_ready = chain ? 1 : 0;
    p.stage_gk = 0;  // set by the launch where LDS allows
    p.chain_g = p.chain_k = p.chain_h = p.chain_e = p.chain_c = p.chain_b = p.chain_hh = nullptr;
    if (chain) {
        // the state-passing kernel's arrays: Z [m][d], g, kappa [m][C], h [d][C] (e [m][C]) per
        // chunk, then c, beta [m][C] and |h|^2 [C] per chunk
        const bool lin1 = desc->linearisation == LATTICE_OSR_LIN1;
        const size_t bwd_bytes = osr::bwd_workspace_bytes(desc->B, desc->H, desc->T, desc->m, desc->d, chunk_size);
        const size_t chain_bytes =
            osr::mfma_chain_workspace_bytes(desc->B, desc->H, desc->T, desc->m, desc->d, chunk_size, lin1);
        const int64_t nch = static_cast<int64_t>(desc->B) * desc->H * (desc->T / chunk_size);
        const int64_t mc = static_cast<int64_t>(desc->m) * chunk_size, dc = static_cast<int64_t>(desc->d) * chunk_size;
        const float* zb = reinterpret_cast<const float*>(static_cast<const char*>(workspace) + bwd_bytes);
        p.chain_g = zb + nch * desc->m * desc->d;
        p.chain_k = p.chain_g + nch * mc;
        p.chain_h = p.chain_k + nch * mc;
        p.chain_e = lin1 ? p.chain_h + nch * dc : nullptr;
        p.chain_c = reinterpret_cast<const float*>(static_cast<const char*>(workspace) + bwd_bytes + chain_bytes);
        p.chain_b = p.chain_c + nch * mc;
        p.chain_hh = p.chain_b + nch * mc;
    }
    if (bwd_chunk_form(desc, chunk_size)) return osr::launch_bwd_chunk(desc->m, desc->d, p, true, st);
    const bool in_bf16 = desc->in_dtype == LATTICE_OSR_BF16;
    if (bwd_small_form(desc, chunk_size)) {
        // phase 1: the forward's small-chunk token loop, keeping every chunk-start state
        // (before projection) in the backward's layout and, decoding objective, every h
        // (unless lattice_osr_fwd_chunked_save stored them there already)
        const osr::Params pf =
            small_phase1_params(desc, chunk_size, q, k, v, gamma, mu, state_in, nullptr, nullptr, workspace);
        if (!saved && !chain) {
            rc = osr::launch_tokenloop_small(desc->m, desc->d, pf, in_bf16, st);
            if (rc) return rc;
        }
        p.f.hrec = pf.hrec;
        // the rows of a sequence over P workgroups where all of them can be resident (a
        // smaller P fits in the buffers sized for the policy's); on a device with too
        // few compute units for the fewest the shape needs, the general walk takes the
        // chunk-start states from phase 1 instead
        const int64_t bh = static_cast<int64_t>(desc->B) * desc->H, cus = device_cus();
        const int pmin = osr::bwd_small_min_p(desc->m, desc->d, chunk_size);
        p.split_p = bwd_parts(desc, chunk_size);
        p.xbuf = nullptr;
        p.xflags = nullptr;
        while (p.split_p > pmin && bh * p.split_p > cus) p.split_p /= 2;
        if (p.split_p > 1 && bh * p.split_p > cus) {
            p.split_p = 1;
            p.states_ready = 1;
            return osr::launch_bwd(desc->m, desc->d, p, in_bf16, st);
        }
        if (p.split_p > 1) {
            const size_t xoff = need - osr::bwd_small_xchg_bytes(desc->B, desc->H, desc->d, p.split_p, chunk_size);
            p.xbuf = reinterpret_cast<float*>(static_cast<char*>(workspace) + xoff);
        }
        return osr::launch_bwd_small(desc->m, desc->d, p, in_bf16, st);
    }
    // slot rows split over workgroups: every workgroup of a sequence must be resident
    // at once (they wait for each other), so no more workgroups than compute units
    p.split_p = osr::bwd_split_p(desc->B, desc->H, desc->m, desc->d, chunk_size, chain, desc->chain_wgs);
    p.xbuf = nullptr;
    p.xflags = nullptr;
    if (p.split_p > 1) {
        const size_t xoff = need - osr::bwd_xchg_bytes(desc->B, desc->H, desc->d, p.split_p);
        const int64_t cus = device_cus();
        while (p.split_p > 1 && (static_cast<int64_t>(desc->B) * desc->H * p.split_p > cus ||
                                 !osr::bwd_split_fits(desc->m, desc->d, chunk_size, p.split_p)))
            p.split_p /= 2;
        if (p.split_p > 1) {
            p.xbuf = reinterpret_cast<float*>(static_cast<char*>(workspace) + xoff);
            p.xflags = reinterpret_cast<int*>(p.xbuf + static_cast<size_t>(desc->B) * desc->H * 2 * p.split_p * 8 *
                                                           (desc->d + 4));
        }
    }
    return osr::launch_bwd(desc->m, desc->d, p, in_bf16, st);
}

}  // namespace

extern "C" {

int lattice_osr_bwd_chunked(const lattice_osr_desc* desc, int32_t chunk_size, const void* q, const void* k,
                            const void* v, const void* gamma, const void* mu, const float* state_in,
                            const void* dy, const float* dstate_out, float* dq, float* dk, float* dv,
                            float* dgamma, float* dmu, float* dstate_in, void* workspace,
                            size_t workspace_bytes, void* hip_stream) {
    return bwd_chunked_impl(desc, chunk_size, q, k, v, gamma, mu, state_in, dy, dstate_out, dq, dk, dv, dgamma, dmu,
                            dstate_in, workspace, workspace_bytes, hip_stream, false);
}

int lattice_osr_bwd_chunked_saved(const lattice_osr_desc* desc, int32_t chunk_size, const void* q, const void* k,
                                  const void* v, const void* gamma, const void* mu, const float* state_in,
                                  const void* dy, const float* dstate_out, float* dq, float* dk, float* dv,
                                  float* dgamma, float* dmu, float* dstate_in, void* workspace,
                                  size_t workspace_bytes, void* hip_stream) {
    return bwd_chunked_impl(desc, chunk_size, q, k, v, gamma, mu, state_in, dy, dstate_out, dq, dk, dv, dgamma, dmu,
                            dstate_in, workspace, workspace_bytes, hip_stream, true);
}

int lattice_osr_fwd_chunked_save(const lattice_osr_desc* desc, int32_t chunk_size, const void* q, const void* k,
                                 const void* v, const void* gamma, const void* mu, const float* state_in,
                                 float* state_out, void* y, void* bwd_workspace, size_t bwd_workspace_bytes,
                                 void* hip_stream) {
    int rc = check_bwd_desc(desc, chunk_size);
    if (rc) return rc;
    if (chunk_size > 8 || !bwd_small_form(desc, chunk_size)) return LATTICE_OSR_ERR_UNSUPPORTED;
    const size_t need = bwd_workspace_needed(desc, chunk_size);
    rc = check_buffers(desc, q, k, v, gamma, mu, state_in, state_out, y, bwd_workspace, bwd_workspace_bytes, need);
    if (rc) return rc;
    const osr::Params pf =
        small_phase1_params(desc, chunk_size, q, k, v, gamma, mu, state_in, state_out, y, bwd_workspace);
    return osr::launch_tokenloop_small(desc->m, desc->d, pf, desc->in_dtype == LATTICE_OSR_BF16,
                                       static_cast<hipStream_t>(hip_stream));
}

}  // extern "C"

// Layer glue: shape rules are those of the descriptor; every buffer is the
// caller's device memory, outputs overlap nothing.
namespace {

bool aligned(const void* p, size_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

}  // namespace

extern "C" {

int lattice_osr_glue_pre(const lattice_osr_desc* desc, const void* xq, const void* xk, const void* gamma_logit,
                         const float* conv_wq, const float* conv_wk, const float* conv_bq, const float* conv_bk,
                         const void* hist_q_in, const void* hist_k_in, void* q, void* k, void* gamma,
                         void* hist_q_out, void* hist_k_out, void* hip_stream) {
    int rc = check_desc(desc);
    if (rc) return rc;
    if (!xq || !xk || !gamma_logit || !conv_wq || !conv_wk || !q || !k || !gamma) return LATTICE_OSR_ERR_NULL;
    if ((hist_q_in == nullptr) != (hist_k_in == nullptr) || (hist_q_out == nullptr) != (hist_k_out == nullptr))
        return LATTICE_OSR_ERR_NULL;
    const size_t ein = desc->in_dtype == LATTICE_OSR_BF16 ? 2 : 4;
    const void* vec[] = {xq, xk, conv_wq, conv_wk, hist_q_in, hist_k_in, q, k, hist_q_out, hist_k_out,
                         desc->gamma_per_slot ? gamma_logit : nullptr, desc->gamma_per_slot ? gamma : nullptr};
    for (const void* ptr : vec)
        if (!aligned(ptr, 16)) return LATTICE_OSR_ERR_ALIGN;
    if (!aligned(gamma_logit, ein) || !aligned(gamma, ein) || !aligned(conv_bq, 4) || !aligned(conv_bk, 4))
        return LATTICE_OSR_ERR_ALIGN;

    const size_t N = static_cast<size_t>(desc->H) * desc->m;
    const size_t G = desc->gamma_per_slot ? N : static_cast<size_t>(desc->H);
    const size_t rows = static_cast<size_t>(desc->B) * desc->T;
    const size_t hist = static_cast<size_t>(desc->B) * 3 * N * ein;
    const Range ins[] = {range_of(xq, rows * N * ein),       range_of(xk, rows * N * ein),
                         range_of(gamma_logit, rows * G * ein), range_of(conv_wq, N * 4 * sizeof(float)),
                         range_of(conv_wk, N * 4 * sizeof(float)), range_of(conv_bq, conv_bq ? N * sizeof(float) : 0),
                         range_of(conv_bk, conv_bk ? N * sizeof(float) : 0), range_of(hist_q_in, hist_q_in ? hist : 0),
                         range_of(hist_k_in, hist_k_in ? hist : 0)};
    const Range outs[] = {range_of(q, rows * N * ein), range_of(k, rows * N * ein), range_of(gamma, rows * G * ein),
                          range_of(hist_q_out, hist_q_out ? hist : 0), range_of(hist_k_out, hist_k_out ? hist : 0)};
    const int nout = sizeof(outs) / sizeof(outs[0]);
    for (int i = 0; i < nout; ++i) {
        for (const Range& r : ins)
            if (overlap(outs[i], r)) return LATTICE_OSR_ERR_ALIAS;
        for (int j = i + 1; j < nout; ++j)
            if (overlap(outs[i], outs[j])) return LATTICE_OSR_ERR_ALIAS;
    }

    osr::GlueParams p;
    p.xq = xq;
    p.xk = xk;
    p.glogit = gamma_logit;
    p.wq = conv_wq;
    p.wk = conv_wk;
    p.bq = conv_bq;
    p.bk = conv_bk;
    p.hq_in = hist_q_in;
    p.hk_in = hist_k_in;
    p.q = q;
    p.k = k;
    p.gamma = gamma;
    p.hq_out = hist_q_out;
    p.hk_out = hist_k_out;
    p.B = desc->B;
    p.T = desc->T;
    p.N = static_cast<int>(N);
    p.G = static_cast<int>(G);
    p.gvec = desc->gamma_per_slot;
    if (N > static_cast<size_t>(INT_MAX) / 2) return LATTICE_OSR_ERR_SHAPE;
    return osr::launch_glue_pre(p, desc->in_dtype == LATTICE_OSR_BF16, static_cast<hipStream_t>(hip_stream));
}

int lattice_osr_glue_post(const lattice_osr_desc* desc, const void* y, const void* gate, void* out,
                          void* hip_stream) {
    int rc = check_desc(desc);
    if (rc) return rc;
    if (!y || !gate || !out) return LATTICE_OSR_ERR_NULL;
    if (!aligned(y, 16) || !aligned(gate, 16) || !aligned(out, 16)) return LATTICE_OSR_ERR_ALIGN;
    const size_t n = static_cast<size_t>(desc->B) * desc->T * desc->H * desc->d;
    const size_t ey = desc->y_dtype == LATTICE_OSR_BF16 ? 2 : 4;
    const size_t eg = desc->in_dtype == LATTICE_OSR_BF16 ? 2 : 4;
    const Range ry = range_of(y, n * ey), rg = range_of(gate, n * eg), ro = range_of(out, n * ey);
    if (overlap(ro, rg) || (ro.lo != ry.lo && overlap(ro, ry))) return LATTICE_OSR_ERR_ALIAS;
    return osr::launch_glue_post(y, desc->y_dtype == LATTICE_OSR_BF16, gate, desc->in_dtype == LATTICE_OSR_BF16, out,
                                 static_cast<int64_t>(n), static_cast<hipStream_t>(hip_stream));
}

}  // extern "C"
