/*
 * lattice_osr.h -- C ABI of the MI355X (gfx950) Orthogonal State Recurrence
 * (OSR) library, liblattice_osr.so.
 *
 * The operation is the state update and read-out of the Lattice compression
 * layer ("Lattice: Learning to Efficiently Compress the Memory", Karami,
 * Pascanu, Mirrokni, arXiv 2504.05646).  A state of m slots, each a vector of
 * length d, is updated per token t by writing into every slot only the part of
 * the token's vector h_t that is orthogonal to that slot (eq. OSR), scaled by
 * the per-slot writing intensity gamma_t * k_t, after decaying the slot by the
 * forget gate mu_t (eq. dacay_recurrence); each slot is then projected back
 * onto the unit sphere (eq. normalized_recurrence).  The output is the
 * read-out y_t = S_t q_t of the updated state (general form of the layer).
 *   decoding objective:   h_t = phi(S) k_t - v_t   (eq. decoding_recurrence)
 *   similarity objective: h_t = -v_t               (eq. similarity_recurrence)
 *   encoding layer:       h_t = v_t, each slot writing with its encoding error
 *                         phi(S)^T v_t - k_t in place of k_t
 *                         (subsection "Encoding layer", eq. encoding_recurrence)
 * Chunked evaluation takes the update's projections at the chunk-start state
 * (section "Parallel and Hardware Efficient Form", eq. recurrence_linear2);
 * with chunk size 1 it is the exact recurrence.
 *
 * Layouts (all contiguous, row-major, as in the implementation appendix):
 *   q, k        [B, T, H, m]     in_dtype
 *   gamma       [B, T, H, m]     in_dtype   (gamma_per_slot = 1)
 *               [B, T, H]        in_dtype   (gamma_per_slot = 0)
 *   v           [B, T, H, d]     in_dtype
 *   mu          [B, T, H]        in_dtype
 *   y           [B, T, H, d]     y_dtype
 *   state_in/out[B, H, m, d]     float32, row i = slot s_i
 * Alignment: q, k, v, a per-slot gamma, state_in, state_out, y and the
 * workspace must be 16-byte aligned; mu and a per-token gamma need only
 * element alignment (any token slice of a contiguous tensor qualifies).
 * Slots of state_in must be non-zero; every slot is projected onto the unit
 * sphere at each chunk start and once more on the returned state.
 *
 * Ownership: every pointer is a device pointer owned by the caller, including
 * the workspace.  The library never allocates, frees or retains device memory
 * (the no-allocation entry's static scratch array aside).  Its only other
 * global state is one side stream and two events per device, created on the
 * first call that overlaps the read-out (LATTICE_OSR_OVERLAP_AUTO) and kept
 * until the process ends; calls on distinct streams may run concurrently.  state_out may alias state_in exactly (in-place update); any
 * partial overlap between state_in and state_out, or any overlap of y with
 * another argument, is rejected.
 *
 * Errors: every entry point returns LATTICE_OSR_OK (0) or a negative status.
 * All argument checks run on the host before any HIP call; on error nothing
 * is enqueued.  LATTICE_OSR_ERR_LAUNCH reports hipGetLastError() after the
 * launch.  Non-finite input values are not detected; they propagate.
 *
 * Asynchrony: work is enqueued on `hip_stream` (a hipStream_t; NULL = the
 * default stream).  No call synchronises.  Inputs must stay valid and
 * unmodified until the stream reaches the end of the enqueued work.
 */
#ifndef LATTICE_OSR_H
#define LATTICE_OSR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LATTICE_OSR_ABI_VERSION 6

#if defined(__GNUC__) || defined(__clang__)
#define LATTICE_OSR_API __attribute__((visibility("default")))
#else
#define LATTICE_OSR_API
#endif

/* Element types of the token inputs (in_dtype) and of y (y_dtype). */
#define LATTICE_OSR_F32 0
#define LATTICE_OSR_BF16 1

/* Objective that defines h_t. */
#define LATTICE_OSR_MODE_DEC 0 /* decoding (l2 reconstruction): h = phi(S)k - v */
#define LATTICE_OSR_MODE_SIM 1 /* dot-product similarity:       h = -v        */
#define LATTICE_OSR_MODE_ENC 2 /* encoding layer: h = v, and each slot writes with the
                                  error of its encoding, e_i = (s_i . v)/|s_i| - k_i,
                                  in place of k_i ("Encoding layer" subsection,
                                  eq. encoding_stateNorm_loss / encoding_recurrence) */

/* Chunk linearisation (section "Parallel and Hardware Efficient Form"): how
 * the update inside a chunk uses the chunk-start state.  Irrelevant at chunk
 * size 1, where both are the exact recurrence. */
#define LATTICE_OSR_LIN2 0 /* eq. recurrence_linear2 (default): the projection term
                              rides on the running slot, gate mu beta + h~ k^       */
#define LATTICE_OSR_LIN1 1 /* eq. recurrence_linear1: gate mu beta on the running
                              slot, the projection term h~ k^ on the chunk-start slot */

/* Matrix-core chunk schedule (bf16 inputs, chunk_size >= 16).  A choice of
 * speed only: every schedule evaluates the same chunk formula (the results
 * agree to the rounding of the split-bf16 products).  Ignored where the
 * token-loop kernel runs (fp32 inputs, chunk_size < 16). */
#define LATTICE_OSR_SCHED_AUTO 0  /* split while the (b,h) sequences leave compute units idle
                                     (fewer than 256 sequences, 512 at d <= 64), else fused */
#define LATTICE_OSR_SCHED_SPLIT 1 /* a state-passing kernel (sequential over chunks) stores each
                                     chunk's start state, gates and h in the workspace; a read-out
                                     kernel then forms every y_t in parallel over chunks */
#define LATTICE_OSR_SCHED_FUSED 2 /* one kernel per sequence does both; no workspace.  The first
                                     linearisation has no fused form and takes the split schedule */

/* Wave layout of the state-passing kernel (split schedule). */
#define LATTICE_OSR_PAIRS_AUTO 0 /* two waves per block of 16 slots, one per token half of the
                                    chunk, where that measured faster (m <= 32 with the chunk as
                                    one sub-block of >= 32 tokens); one wave elsewhere */
#define LATTICE_OSR_PAIRS_OFF 1  /* always one wave per block of 16 slots */

/* Workgroups per (b,h) sequence in the state-passing kernel (split schedule). */
#define LATTICE_OSR_WGS_AUTO 0 /* where a chunk is 2 or 4 (P) of that kernel's sub-blocks and
                                  the sequences are few (B*H <= 32, and B*H*P no more than the
                                  device's compute units), one workgroup per sub-block of the
                                  chunk, exchanging their parts of the chunk-end state through
                                  the workspace; else one workgroup */
#define LATTICE_OSR_WGS_ONE 1  /* always one workgroup per sequence */

/* Read-out of the split schedule overlapped with its state passing. */
#define LATTICE_OSR_OVERLAP_AUTO 0 /* where the state passing takes at most 128 workgroups and
                                      there are at least 64 chunks (a multiple of 64): the chunks
                                      in 4 ranges (up to 64 workgroups: of shrinking length, 48,
                                      12, 3 and 1 64ths of the chunks; from 65: equal quarters);
                                      each range's read-out runs on the
                                      library's side stream for the device while the next range's
                                      state passing runs on hip_stream, which waits for the side
                                      stream before the call's work ends.  Same results, bit for
                                      bit, as _OFF.  A caller capturing the call into a HIP graph
                                      may prefer _OFF (or the no-allocation entry), which keeps
                                      all work on hip_stream */
#define LATTICE_OSR_OVERLAP_OFF 1  /* state passing, then read-out, both on hip_stream */

/*
 * Form of the backward (lattice_osr_bwd_chunked; the forward ignores it).
 * WALK: the general reverse walk over the tokens, in fp32 on the vector units.
 * CHUNK: the chunk-parallel form on the fp32 matrix cores (built for
 * m = d = chunk_size = 64, bf16 inputs, the default linearisation, the
 * decoding and similarity objectives; elsewhere the call returns
 * LATTICE_OSR_ERR_UNSUPPORTED).  AUTO: CHUNK where it is built; at
 * chunk_size 2, 4 or 8 with the default linearisation and m d <= 4096 (and
 * d <= 64 at chunk_size 8), a reverse walk that keeps a chunk's per-token
 * states in registers; else WALK.  All compute the same gradient up to fp32
 * rounding.
 */
#define LATTICE_OSR_BWD_AUTO 0
#define LATTICE_OSR_BWD_WALK 1
#define LATTICE_OSR_BWD_CHUNK 2

/* Status codes. */
#define LATTICE_OSR_OK 0
#define LATTICE_OSR_ERR_NULL (-1)        /* a required pointer is NULL              */
#define LATTICE_OSR_ERR_SHAPE (-2)       /* non-positive dims, T % C != 0, T != 1 for decode */
#define LATTICE_OSR_ERR_UNSUPPORTED (-3) /* m, d not in {16,32,64,128}; C not a power of two <= 128; bad enum */
#define LATTICE_OSR_ERR_WORKSPACE (-4)   /* workspace smaller than lattice_osr_workspace_bytes() */
#define LATTICE_OSR_ERR_LAUNCH (-5)      /* the HIP launch reported an error        */
#define LATTICE_OSR_ERR_ALIAS (-6)       /* forbidden overlap between arguments      */
#define LATTICE_OSR_ERR_ALIGN (-7)       /* a pointer is misaligned (see Alignment)  */

typedef struct {
    int32_t B;              /* batch (decode: number of sequences)               */
    int32_t T;              /* tokens per sequence                               */
    int32_t H;              /* heads                                             */
    int32_t m;              /* slots per head: 16, 32, 64 or 128                 */
    int32_t d;              /* slot / value width: 16, 32, 64 or 128             */
    int32_t gamma_per_slot; /* 1: gamma is [B,T,H,m]; 0: gamma is [B,T,H]        */
    int32_t in_dtype;       /* LATTICE_OSR_F32 or LATTICE_OSR_BF16               */
    int32_t y_dtype;        /* LATTICE_OSR_F32 or LATTICE_OSR_BF16               */
    int32_t mode;           /* LATTICE_OSR_MODE_DEC, _SIM or _ENC                */
    int32_t linearisation;  /* LATTICE_OSR_LIN2 (0) or LATTICE_OSR_LIN1 (1)      */
    int32_t schedule;       /* LATTICE_OSR_SCHED_AUTO (0), _SPLIT (1), _FUSED (2) */
    int32_t chain_pairs;    /* LATTICE_OSR_PAIRS_AUTO (0) or _OFF (1)            */
    int32_t chain_wgs;      /* LATTICE_OSR_WGS_AUTO (0) or _ONE (1)              */
    int32_t readout_overlap; /* LATTICE_OSR_OVERLAP_AUTO (0) or _OFF (1)         */
    int32_t bwd_form;       /* LATTICE_OSR_BWD_AUTO (0), _WALK (1), _CHUNK (2)   */
} lattice_osr_desc;

/*
 * Chunk-wise forward (training / prefill).  Each chunk of C = chunk_size
 * tokens takes its projections, gates and (decoding objective) h_t from the
 * chunk-start state (eq. recurrence_linear2, the gated-linear-attention form
 * of the section "Parallel and Hardware Efficient Form", or eq.
 * recurrence_linear1 with desc->linearisation = LATTICE_OSR_LIN1); C = 1 is
 * the exact recurrence.  Requires T % chunk_size == 0 and chunk_size a power
 * of two in [1, 128].  workspace must hold lattice_osr_workspace_bytes(desc,
 * chunk_size) bytes (it may be NULL when that is 0; bf16 inputs with
 * chunk_size >= 16 need one unless many sequences take the default
 * linearisation's fused kernel); its contents on entry are ignored.
 */
LATTICE_OSR_API int lattice_osr_fwd_chunked(const lattice_osr_desc* desc, int32_t chunk_size,
                            const void* q, const void* k, const void* v, const void* gamma,
                            const void* mu, const float* state_in, float* state_out, void* y,
                            void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * Chunk-wise forward with the layer's GeLU post-gate fused into the output
 * (section "Experiments", paragraph on the Lattice block, where a GeLU
 * post-gate follows the recurrence): y_t = (S_t q_t) * GeLU(gate_t)
 * elementwise, GeLU(x) = x Phi(x) in its exact form, in fp32 before y is
 * rounded to y_dtype.  The same as lattice_osr_fwd_chunked followed by
 * lattice_osr_glue_post, without writing and reading back the ungated y.
 *   gate  [B, T, H, d]  in_dtype, 16-byte aligned; an input (it may overlap
 *                       other inputs, no output: ERR_ALIAS otherwise)
 * Every other argument, rule and status is that of lattice_osr_fwd_chunked
 * (the same workspace size).
 */
LATTICE_OSR_API int lattice_osr_fwd_chunked_gated(const lattice_osr_desc* desc, int32_t chunk_size,
                                                  const void* q, const void* k, const void* v,
                                                  const void* gamma, const void* mu, const void* gate,
                                                  const float* state_in, float* state_out, void* y,
                                                  void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * lattice_osr_fwd_chunked for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation and arguments without the workspace.  The
 * split schedule's per-chunk arrays (and the state passing's hand-off
 * buffers) live in a scratch array the library keeps in device memory, one
 * per GPU, allocated with the library's code object and held until the
 * process ends; the call itself allocates nothing.  Limit: configurations
 * whose lattice_osr_workspace_bytes() exceeds
 * LATTICE_OSR_NOALLOC_SCRATCH_BYTES return LATTICE_OSR_ERR_WORKSPACE.  The
 * scratch is shared by every call on one GPU and keeps the last call's
 * contents: calls that overlap in time on one GPU (distinct streams, or
 * another thread) race on it and must be serialised by the caller.  The
 * first call on a device looks up that device's copy (hipGetSymbolAddress,
 * the device that is current); LATTICE_OSR_ERR_LAUNCH if that fails.  The
 * read-out never overlaps here (desc->readout_overlap is taken as
 * LATTICE_OSR_OVERLAP_OFF, and the workspace limit is that of _OFF): all work
 * stays on hip_stream.
 */
#define LATTICE_OSR_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
LATTICE_OSR_API int lattice_osr_fwd_chunked_noalloc(const lattice_osr_desc* desc, int32_t chunk_size,
                                                    const void* q, const void* k, const void* v,
                                                    const void* gamma, const void* mu, const float* state_in,
                                                    float* state_out, void* y, void* hip_stream);

/*
 * Exact recurrent forward: the recurrence of eq. recurrence_detailed applied
 * token by token (chunk size 1), the state held on chip across tokens.
 * Needs no workspace (workspace may be NULL, workspace_bytes 0).
 */
LATTICE_OSR_API int lattice_osr_fwd_recurrent(const lattice_osr_desc* desc, const void* q, const void* k,
                              const void* v, const void* gamma, const void* mu,
                              const float* state_in, float* state_out, void* y,
                              void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * One exact decode step for B sequences x H heads (desc->T must be 1): read
 * each state once, apply one update, write it once, emit y.  In place
 * (state_out == state_in) is allowed.  Needs no workspace.
 */
LATTICE_OSR_API int lattice_osr_decode_step(const lattice_osr_desc* desc, const void* q, const void* k,
                            const void* v, const void* gamma, const void* mu,
                            const float* state_in, float* state_out, void* y,
                            void* workspace, size_t workspace_bytes, void* hip_stream);

/* Workspace bytes lattice_osr_fwd_chunked needs for this descriptor (shape,
 * linearisation and schedule) and chunk size (0 if none); (size_t)-1 if the
 * arguments are invalid.  Pass the same descriptor to the forward. */
LATTICE_OSR_API size_t lattice_osr_workspace_bytes(const lattice_osr_desc* desc, int32_t chunk_size);

/*
 * Backward of the chunk-wise forward (training).  The pages train the layer
 * through its chunk-wise form (section "Parallel and Hardware Efficient
 * Form"); this call returns the gradient of
 *     L = sum(dy * y) + sum(dstate_out * state_out)
 * with respect to q, k, v, gamma, mu and state_in, where (y, state_out) is
 * lattice_osr_fwd_chunked at the same desc (either linearisation) and
 * chunk_size.  The forward is recomputed inside the call: the forward's y and
 * state_out are not needed.
 *   dy          [B,T,H,d]   y_dtype            (16-byte aligned)
 *   dstate_out  [B,H,m,d]   float32            (16-byte aligned)
 *   dq, dk      [B,T,H,m]   float32            (4-byte aligned)
 *   dv          [B,T,H,d]   float32            (16-byte aligned)
 *   dgamma      gamma's shape, float32         (4-byte aligned)
 *   dmu         [B,T,H]     float32            (4-byte aligned)
 *   dstate_in   [B,H,m,d]   float32            (16-byte aligned)
 * Every gradient is written in full (no accumulation into existing values).
 * The gradient buffers and the workspace must not overlap one another or any
 * input.  workspace must hold lattice_osr_bwd_workspace_bytes(desc,
 * chunk_size) bytes: per (b,h), 4 (T/C + 1 + C) m d bytes of states plus
 * 4 C (2m + 4) bytes of per-token values, and, for bf16 inputs with
 * chunk_size >= 16 (decoding and similarity objectives, whose chunk-start
 * states then come from the matrix-core state-passing kernel), that kernel's
 * per-chunk arrays: 4 (m d + 4 m C + d C + C) bytes per chunk (4 m C more
 * with LATTICE_OSR_LIN1).  On that path, with desc->chain_wgs =
 * LATTICE_OSR_WGS_AUTO, the slot rows of each sequence are split over P
 * workgroups (the largest P in {1, 2, 4, 8} with m / P >= 16, B*H*P <= 256 and
 * a workgroup's working set within its 160 KiB of LDS; fewer if the device has
 * fewer compute units) that exchange each batch of
 * tokens' sums over slots: the workspace then ends with their hand-off
 * buffers, B*H*(2 P 8 (d + 4) * 4 + 128 P) bytes.  The result equals one
 * workgroup's (LATTICE_OSR_WGS_ONE) up to the order of those fp32 sums;
 * reruns are bit-identical.  Where desc->bwd_form allows it (AUTO or CHUNK;
 * built for m = d = chunk_size = 64 on that same path), the gradient is
 * instead taken in its chunk-parallel form on the fp32 matrix cores, one
 * workgroup per (b,h): per chunk the vector-Jacobian products of the
 * chunk's matrix form (16-token tiles), the gate gradients by recursions
 * over the tile's tokens; the same workspace and the same result up to fp32
 * rounding (the token walk's to 1e-4 of RMS; with forget gates mu near 0 the
 * tile's gate products span many decades and the two agree to 5e-3).
 *
 * Small chunks: with desc->bwd_form AUTO, at chunk_size 1, 2, 4 or 8 (at
 * most 4 at d = 128 and at m d = 8192, 2 at m = d = 128; either linearisation)
 * and at chunk_size 16 on the state-passing path above (the default
 * linearisation), where a chunk fits, a reverse walk that keeps each chunk's per-token states in
 * registers runs after a forward pass that stores the chunk-start states
 * (at chunk_size 16 the state-passing kernel's pass, which also supplies h;
 * below 16 the token loop's, and for the decoding objective every token's h
 * goes to the workspace too, 4 T d bytes per (b,h)).  With desc->chain_wgs =
 * LATTICE_OSR_WGS_AUTO, chunk_size >= 4, m >= 32 and B*H*P <= 256, the slot
 * rows of each sequence are split over P workgroups (4 at chunk_size 8 where
 * a quarter of the rows has the threads to stage a chunk, else 2) that
 * exchange each chunk's sums over slots through hand-off buffers at the end
 * of the workspace: B*H*16 P max(chunk_size, 8) (d + 4) bytes (value and tag
 * pairs).  Fewer workgroups on devices with fewer than B*H*P compute units,
 * one with LATTICE_OSR_WGS_ONE.  At m d = 8192, m = d = 128 and (chunk_size
 * 16) m = d = 64 the chunk's states fit only split, over at least 2, 4 and 2
 * workgroups: the form needs B*H*P <= 256 there, WGS_ONE gives that fewest
 * P, and a device with fewer compute units runs the general walk within the
 * same workspace.  The result equals the general walk's up to fp32 rounding.
 *
 * The remaining rules (shapes, chunk sizes, alignment of the inputs, status
 * codes, asynchrony) are those of lattice_osr_fwd_chunked.
 */
LATTICE_OSR_API int lattice_osr_bwd_chunked(const lattice_osr_desc* desc, int32_t chunk_size,
                            const void* q, const void* k, const void* v, const void* gamma,
                            const void* mu, const float* state_in, const void* dy,
                            const float* dstate_out, float* dq, float* dk, float* dv, float* dgamma,
                            float* dmu, float* dstate_in, void* workspace, size_t workspace_bytes,
                            void* hip_stream);

/* Workspace bytes lattice_osr_bwd_chunked needs for this shape; (size_t)-1 if
 * the arguments are invalid or the configuration has no backward. */
LATTICE_OSR_API size_t lattice_osr_bwd_workspace_bytes(const lattice_osr_desc* desc, int32_t chunk_size);

/*
 * Training at small chunks without the backward's forward pass.  Where the
 * backward takes its small-chunk form at chunk_size 1, 2, 4 or 8 (above;
 * elsewhere both calls return LATTICE_OSR_ERR_UNSUPPORTED):
 *
 * lattice_osr_fwd_chunked_save computes y and state_out exactly as
 * lattice_osr_fwd_chunked does (the same kernel, bit for bit; arguments and
 * rules as there, no workspace) and also stores, in bwd_workspace
 * (lattice_osr_bwd_workspace_bytes(desc, chunk_size) bytes, 16-byte aligned,
 * overlapping no argument), every chunk-start state before projection and,
 * for the decoding objective, every token's h.
 *
 * lattice_osr_bwd_chunked_saved returns what lattice_osr_bwd_chunked returns,
 * bit for bit (arguments and rules as there), taking those values from its
 * workspace instead of recomputing them: the workspace must hold what a
 * lattice_osr_fwd_chunked_save call with the same inputs, chunk_size and desc
 * (y_dtype aside) stored, unchanged since (work on one stream, or ordered).
 * The backward reads them and writes only the workspace's hand-off buffers,
 * so the saved values serve any number of backward calls.  The forward pass
 * this skips is about a third of the backward (B4 H8 T2048 m = d = 64 C4:
 * ~1.5 of 4.2 ms).
 */
LATTICE_OSR_API int lattice_osr_fwd_chunked_save(const lattice_osr_desc* desc, int32_t chunk_size,
                            const void* q, const void* k, const void* v, const void* gamma,
                            const void* mu, const float* state_in, float* state_out, void* y,
                            void* bwd_workspace, size_t bwd_workspace_bytes, void* hip_stream);
LATTICE_OSR_API int lattice_osr_bwd_chunked_saved(const lattice_osr_desc* desc, int32_t chunk_size,
                            const void* q, const void* k, const void* v, const void* gamma,
                            const void* mu, const float* state_in, const void* dy,
                            const float* dstate_out, float* dq, float* dk, float* dv, float* dgamma,
                            float* dmu, float* dstate_in, void* workspace, size_t workspace_bytes,
                            void* hip_stream);

/*
 * Layer glue before the recurrence (section "Experiments", paragraph on the
 * Lattice block: a pair of short convolutions for q and k, which share one
 * projection, and the writing intensity gamma_t = sigmoid(W_gamma x_t); the
 * experiment-details appendix sets the convolution width to 4).  The
 * projections are the caller's; this call does, in one pass:
 *   q = conv4(xq), k = conv4(xk)  depthwise and causal along T, one filter per
 *                                 channel (h, i): out_t = b + sum_j w[j] x_{t-3+j},
 *                                 j = 0..3 (w[3] weighs the current token);
 *                                 the three rows before t = 0 come from the
 *                                 history (zeros when it is NULL: sequence start);
 *   gamma = sigmoid(gamma_logit)  elementwise.
 * The outputs are ready for lattice_osr_fwd_chunked with the same desc (which
 * supplies B, T, H, m, gamma_per_slot and in_dtype; every element buffer is
 * in_dtype, the weights fp32; d, y_dtype, mode, linearisation are validated
 * but unused).  Arithmetic is fp32.
 *   xq, xk, q, k            [B, T, H, m]
 *   gamma_logit, gamma      [B, T, H, m] (gamma_per_slot = 1) or [B, T, H]
 *   conv_wq, conv_wk        [H, m, 4]  float32
 *   conv_bq, conv_bk        [H, m]     float32, or NULL (no bias)
 *   hist_q_in, hist_k_in    [B, 3, H, m], the raw xq / xk rows of the three
 *                           tokens before this call, oldest first; both NULL
 *                           at a sequence start
 *   hist_q_out, hist_k_out  [B, 3, H, m] receive the last three raw rows
 *                           (of the history followed by x), for the next call;
 *                           both NULL: not written
 * Alignment: 16 bytes for every buffer except the biases (4 bytes) and a
 * per-token gamma_logit / gamma (element alignment).  No output may overlap
 * another output or any input (ERR_ALIAS); pass a second history buffer
 * rather than updating one in place.  Errors and asynchrony as above.
 */
LATTICE_OSR_API int lattice_osr_glue_pre(const lattice_osr_desc* desc, const void* xq, const void* xk,
                                         const void* gamma_logit, const float* conv_wq, const float* conv_wk,
                                         const float* conv_bq, const float* conv_bk, const void* hist_q_in,
                                         const void* hist_k_in, void* q, void* k, void* gamma, void* hist_q_out,
                                         void* hist_k_out, void* hip_stream);

/*
 * Layer glue after the recurrence: the GeLU post-gate on the layer's output
 * (section "Experiments", paragraph on the Lattice block),
 *   out = y * GeLU(gate),  GeLU(x) = x Phi(x), Phi the standard normal CDF
 * (the exact form), elementwise in fp32.
 *   y, out  [B, T, H, d]  y_dtype;  gate  [B, T, H, d]  in_dtype
 * out may be y itself (in place); any other overlap is ERR_ALIAS.  All three
 * must be 16-byte aligned.  Errors and asynchrony as above.
 */
LATTICE_OSR_API int lattice_osr_glue_post(const lattice_osr_desc* desc, const void* y, const void* gate, void* out,
                                          void* hip_stream);

/* Static text for a status code (never NULL). */
LATTICE_OSR_API const char* lattice_osr_status_string(int status);

/* LATTICE_OSR_ABI_VERSION of the loaded library. */
LATTICE_OSR_API int lattice_osr_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LATTICE_OSR_H */
