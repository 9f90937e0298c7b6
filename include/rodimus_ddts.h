/*
 * rodimus_ddts.h -- C ABI of the MI355X (gfx950) DDTS recurrence library.
 *
 * The operation (per batch element b and head h; dk = expansion factor n,
 * dv = value width m):
 *
 *   alpha_t     = exp(-g_t * tau_t)            forget gate, over dk
 *   alpha_hat_t = g_t ^ tau_t                   input gate, over dk
 *   S_t = diag(alpha_t) S_{t-1} + (alpha_hat_t * k_t) (beta_hat_t * v_t)^T
 *   o_t = S_t^T q_t                             readout after the update
 *
 * Cited from the pages on Rodimus* (arXiv 2410.06577):
 *  - gate formulas alpha = exp(-g*tau), alpha_hat = g^tau: the digest page
 *    (digest.lyk-ai.com), section "Method";
 *  - beta_hat is the low-rank gate on the value side: same section;
 *  - selection acts only along n (the dk rows of S), which is what allows the
 *    chunkwise-parallel form: the authors' rebuttal (paperhub.cn), bullet
 *    "Efficient Parallelization";
 *  - training runs chunkwise in parallel and inference sequentially over a
 *    cached fixed-size state: the same rebuttal, answer on sequential
 *    processing bottlenecks (Q2 of the first review);
 *  - the state is n x m per head: the same rebuttal, answer on the
 *    "State size n x m" column of Table 4.
 * The recurrence's own equation (the paper's Eq. 11) is not on the pages; the
 * readout-after-update order and the absence of any scaling of q inside the
 * operation are the readings taken.
 *
 * Conventions shared by every entry point
 *  - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *    allocates no memory and keeps no state beyond a per-device flag for each
 *    kernel (the first launch of a kernel on a device raises its LDS limit
 *    with hipFuncSetAttribute) and the fixed per-device scratch array of
 *    rodimus_ddts_chunk_fwd_static_scratch (part of its code object); calls
 *    are reentrant, except that calls of that one entry point on one GPU
 *    share its scratch.  Work is enqueued on
 *    `stream` and the call returns before it completes.  Only kernel launches
 *    are enqueued (no memsets, allocations or synchronisation), so calls can
 *    be captured in a HIP graph; make one call of the same shape and dtype
 *    outside the capture first, so that the attribute is already set.
 *  - Every argument check happens on the host, synchronously, BEFORE any HIP
 *    call; a failed check returns a status and enqueues nothing.
 *  - Layouts are dense row-major: per-token tensors [B, T, H, D] with the
 *    feature dimension contiguous; states [B, H, dk, dv] fp32 with dv
 *    contiguous (the same layout for prefill and decode, so a prefill's final
 *    state is a decode state).
 *  - Supported widths: dk, dv in {16, 32, 64, 128}.  Pointers must be 16-byte
 *    aligned.
 *  - Domain (documented, not checked on the device): g >= 0 and tau >= 0.
 *    NaN and Inf propagate.  The chunked form multiplies by exp(+-partial
 *    sums of g*tau) inside a chunk; results are exact up to rounding while the
 *    sum of g*tau over any half chunk stays below about 80 (true for gates in
 *    [0, 1] at any supported chunk size).
 */
#ifndef RODIMUS_DDTS_H
#define RODIMUS_DDTS_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RODIMUS_ABI_VERSION 1

/* The two enums carry sentinel members that make every int a valid value of
 * their type: a caller's out-of-range code (e.g. a dtype of 7) then reaches
 * the library's checks, which reject it, instead of being undefined in the
 * C++ implementation.  The sentinels are not statuses or dtypes. */
typedef enum {
    RODIMUS_OK = 0,
    RODIMUS_ERR_INVALID_ARG = 1,   /* null pointer, bad size, misalignment, overlap */
    RODIMUS_ERR_UNSUPPORTED = 2,   /* width, chunk or dtype outside the supported set */
    RODIMUS_ERR_WORKSPACE = 3,     /* workspace missing or smaller than required */
    RODIMUS_ERR_HIP = 4,           /* a HIP launch or runtime call failed */
    RODIMUS_STATUS_RANGE_MIN_ = -2147483647 - 1,
    RODIMUS_STATUS_RANGE_MAX_ = 2147483647
} rodimus_status;

typedef enum {
    RODIMUS_DTYPE_F32 = 0,
    RODIMUS_DTYPE_BF16 = 1,
    RODIMUS_DTYPE_RANGE_MIN_ = -2147483647 - 1,
    RODIMUS_DTYPE_RANGE_MAX_ = 2147483647
} rodimus_dtype;

/* ABI version of the loaded library (RODIMUS_ABI_VERSION). */
int rodimus_abi_version(void);

/* Static, human-readable text for a status code. */
const char *rodimus_status_string(rodimus_status status);

/*
 * Bytes of device workspace rodimus_ddts_chunk_fwd needs for these sizes
 * (0 when the single-sweep path is used).  Returns 0 as well for arguments
 * the forward would reject.  Deterministic: depends only on the arguments.
 */
size_t rodimus_ddts_chunk_fwd_workspace_bytes(int B, int T, int H, int dk, int dv, int chunk);

/*
 * Chunkwise-parallel forward (prefill / training pass) over whole sequences.
 *
 *   B, T, H, dk, dv  sizes; B, H >= 1, T >= 0 (T == 0 only copies the state).
 *   chunk            tokens per chunk: 0 = library's choice, else 16, 32 or 64.
 *                    Results do not depend on it beyond rounding.  It is an
 *                    upper bound: a shorter chunk is used where the tile does
 *                    not fit in LDS (fp32 inputs with dk = 128 and 64), and
 *                    32-token chunks where the library splits the sequences
 *                    into segments (few (b, h) pairs; bf16 inputs, dk <= 64).
 *   in_dtype         dtype of all six per-token inputs (bf16 or fp32); the
 *                    state and the output are always fp32.
 *   q, k, g, tau     [B, T, H, dk]
 *   v, beta_hat      [B, T, H, dv]
 *   initial_state    [B, H, dk, dv] fp32, or NULL for a zero state.
 *   out              [B, T, H, dv] fp32; must not overlap any input or state.
 *   final_state      [B, H, dk, dv] fp32, or NULL.  May be the same pointer as
 *                    initial_state (carry-over in place), may not overlap it
 *                    partially, and may not overlap any other tensor.
 *   workspace        device scratch of at least
 *                    rodimus_ddts_chunk_fwd_workspace_bytes(...) bytes (NULL
 *                    allowed when that is 0); its contents on entry are ignored.
 *   stream           HIP stream the kernels are launched on.
 *
 * Returns RODIMUS_OK, or an error status with nothing enqueued (argument
 * errors) or with a HIP launch error (RODIMUS_ERR_HIP).
 */
rodimus_status rodimus_ddts_chunk_fwd(
    int B, int T, int H, int dk, int dv, int chunk, rodimus_dtype in_dtype,
    const void *q, const void *k, const void *g, const void *tau,
    const void *v, const void *beta_hat,
    const float *initial_state, float *out, float *final_state,
    void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * As rodimus_ddts_chunk_fwd, with the sequence split into `segments` pieces
 * per (b, h) that run in parallel: each piece's state transfer is computed
 * from a zero state, the transfers are combined in order, and each piece then
 * produces its outputs from its true incoming state.  segments = 0 lets the
 * library choose (what rodimus_ddts_chunk_fwd does); 1 forces one sequential
 * sweep per (b, h); values above the number of chunks are clamped.
 * Workspace: rodimus_ddts_chunk_fwd_ex_workspace_bytes with the same arguments.
 */
rodimus_status rodimus_ddts_chunk_fwd_ex(
    int B, int T, int H, int dk, int dv, int chunk, int segments, rodimus_dtype in_dtype,
    const void *q, const void *k, const void *g, const void *tau,
    const void *v, const void *beta_hat,
    const float *initial_state, float *out, float *final_state,
    void *workspace, size_t workspace_bytes, hipStream_t stream);

size_t rodimus_ddts_chunk_fwd_ex_workspace_bytes(int B, int T, int H, int dk, int dv,
                                                 int chunk, int segments);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * call as rodimus_ddts_chunk_fwd_ex with identical results, but the scratch
 * of the segmented path comes from a fixed buffer inside the library instead
 * of a workspace argument.  The caller still passes inputs and outputs.
 *
 *   Limit: the plan's workspace (rodimus_ddts_chunk_fwd_plan) must be at most
 *   RODIMUS_STATIC_SCRATCH_BYTES, else RODIMUS_ERR_WORKSPACE is returned with
 *   nothing enqueued (e.g. B * H = 16 heads of 64 x 128 split into 16
 *   segments, 30 transfer pieces, need 15.9 MB).
 *   The buffer is one per GPU, held by every GPU the library runs on until
 *   the process ends, and shared by every call on that GPU: calls that
 *   overlap on one GPU (several streams or host threads) race on it and must
 *   be serialised by the caller.  Its contents carry nothing from one call
 *   to the next.
 *   Allocation: none (no hipMalloc, hipFree or allocating library call); the
 *   first call on a device looks up the buffer's device address once.
 * Other arguments, checks and errors as rodimus_ddts_chunk_fwd_ex.
 */
#define RODIMUS_STATIC_SCRATCH_BYTES ((size_t)32 << 20)

rodimus_status rodimus_ddts_chunk_fwd_static_scratch(
    int B, int T, int H, int dk, int dv, int chunk, int segments, rodimus_dtype in_dtype,
    const void *q, const void *k, const void *g, const void *tau,
    const void *v, const void *beta_hat,
    const float *initial_state, float *out, float *final_state, hipStream_t stream);

/*
 * Tracing aid (the profiler's view of one forward call, on its own stream):
 * until called again with count = 0, every forward call made by the calling
 * host thread records the caller's events (hipEventCreate) on its stream
 * around its launches: one sweep: events[0] before the launch, events[1]
 * after it; segmented: events[0] before the transfer pass, events[1] after
 * it, events[2] after the ordered combine, events[3] after the output pass.
 * count must be 4 (RODIMUS_ERR_INVALID_ARG otherwise), or 0 to stop.  The
 * events array must stay valid while set.  No event is recorded by a call
 * that fails its checks.
 */
rodimus_status rodimus_trace_forward_events(hipEvent_t *events, int count);

/*
 * How rodimus_ddts_chunk_fwd_ex runs for these arguments and input dtype:
 *   chunk            tokens per chunk (16, 32 or 64) of the outputs (the
 *                    segment transfers of a whole-head plan may run chunks
 *                    of half that length over the same token ranges);
 *   dv_tile          dv columns per workgroup (128: one workgroup per head);
 *   segments         pieces each (b, h) sequence is split into (1: one
 *                    sequential sweep);
 *   transfer_pieces  pieces each state transfer (one per segment but the
 *                    last) is cut into; 0 for one sweep;
 *   workspace_bytes  device workspace the call needs (the *_workspace_bytes
 *                    queries return the larger need over both dtypes).
 * Host only: no HIP call, no GPU needed; deterministic.  Returns the status
 * the forward would return for invalid or unsupported arguments (the plan is
 * then left untouched), RODIMUS_ERR_INVALID_ARG for a NULL plan.
 */
typedef struct {
    int chunk, dv_tile, segments, transfer_pieces;
    size_t workspace_bytes;
} rodimus_chunk_plan;

rodimus_status rodimus_ddts_chunk_fwd_plan(int B, int T, int H, int dk, int dv, int chunk,
                                           int segments, rodimus_dtype in_dtype,
                                           rodimus_chunk_plan *plan);

/*
 * The steps on either side of the recurrence, fused into its kernels.  The
 * pages name them without giving their equations; the readings taken:
 *  - beta_hat from low-rank factors (digest page, "Method", low-rank
 *    bullet): beta_hat_t = sigmoid(u_t w), u_t the rank-r factor of token t
 *    and head h, w [r, dv] per head, no scaling;
 *  - ShortConv (digest page, "Method", ShortConv + GLU bullet): a causal
 *    depthwise convolution along time of q, k and v, conv_width taps per head
 *    and channel, no bias, no activation:
 *        x'_t[i] = sum_{j < conv_width} c[h][i][j] x_{t-j}[i];
 *  - the feedthrough d (rebuttal page, answer to "How significant is d_t in
 *    Eq. (11)?": the SSM feedthrough matrix): o_t += d .* v_t, d a vector over
 *    dv per head, constant in t, v_t the value entering the recurrence (after
 *    the convolution, before beta_hat).
 * Fields (NULL / 0 / 1 switch a step off):
 *   u, w        [B, T, H, rank] (decode: [N, H, rank]) and [H, rank, dv], in
 *               in_dtype; rank 16 or 32.  When u is set, beta_hat is not read
 *               and may be NULL.
 *   d           [H, dv] fp32.
 *   conv_width  1 (none), 2, 3 or 4; conv_q, conv_k [H, dk, conv_width] and
 *               conv_v [H, dv, conv_width] fp32, tap j multiplying the input
 *               j tokens back.  q, k and v then hold conv_width - 1 raw rows
 *               before token 0: [B, T + conv_width - 1, H, D] (zeros at a
 *               sequence start; the last conv_width - 1 raw rows of the
 *               previous call to continue a sequence).  Decode: q, k, v are the
 *               windows of the last conv_width raw tokens, oldest first,
 *               [N, conv_width, H, D].
 * All pointers 16-byte aligned, outputs overlapping none of them.
 */
typedef struct {
    const void *u, *w;
    int rank;
    const float *d;
    int conv_width;
    const float *conv_q, *conv_k, *conv_v;
} rodimus_fused;

/*
 * rodimus_ddts_chunk_fwd_ex with the fused steps of `fused` (not NULL).
 * Workspace: rodimus_ddts_chunk_fwd_fused_workspace_bytes (the fused kernels
 * may plan differently: fp32 inputs run 16-token chunks).
 */
rodimus_status rodimus_ddts_chunk_fwd_fused(
    int B, int T, int H, int dk, int dv, int chunk, int segments, rodimus_dtype in_dtype,
    const void *q, const void *k, const void *g, const void *tau,
    const void *v, const void *beta_hat, const rodimus_fused *fused,
    const float *initial_state, float *out, float *final_state,
    void *workspace, size_t workspace_bytes, hipStream_t stream);

size_t rodimus_ddts_chunk_fwd_fused_workspace_bytes(int B, int T, int H, int dk, int dv,
                                                    int chunk, int segments);

/*
 * One recurrent step (sequential inference) for N independent sequences over
 * their resident states, updated in place.
 *
 *   N, H, dk, dv     sizes; N, H >= 1.
 *   in_dtype         dtype of the six per-token inputs.
 *   q, k, g, tau     [N, H, dk]
 *   v, beta_hat      [N, H, dv]
 *   state            [N, H, dk, dv] fp32, read and overwritten with S_t.
 *   out              [N, H, dv] fp32 (o_t); must not overlap the state or inputs.
 *   stream           HIP stream.
 */
rodimus_status rodimus_ddts_decode_step(
    int N, int H, int dk, int dv, rodimus_dtype in_dtype,
    const void *q, const void *k, const void *g, const void *tau,
    const void *v, const void *beta_hat,
    float *state, float *out, hipStream_t stream);

/*
 * rodimus_ddts_decode_step with the fused steps of `fused` (not NULL); q, k,
 * v are [N, conv_width, H, D] windows when conv_width > 1.
 */
rodimus_status rodimus_ddts_decode_step_fused(
    int N, int H, int dk, int dv, rodimus_dtype in_dtype,
    const void *q, const void *k, const void *g, const void *tau,
    const void *v, const void *beta_hat, const rodimus_fused *fused,
    float *state, float *out, hipStream_t stream);

/*
 * Sliding-window attention with one key shared by all heads (SW-SKA, the
 * second token mixer of Rodimus+): the summary page ("Approach") and the
 * digest page ("Method", Rodimus+ bullets) describe sliding-window attention
 * whose keys are shared across heads; the rebuttal (answer on the Rodimus+
 * parameter count) splits its projections into multi-head, multi-query and
 * output ones, so q and v have a head each and k one for all.  Per batch b,
 * head h and token t:
 *     o[b,t,h] = sum over t - window < s <= t of softmax_s(scale q[b,t,h] . k[b,s]) v[b,s,h]
 *
 *   B, T, H       sizes; B, H >= 1, T >= 0 (T == 0 does nothing); B * T and
 *                 64 * H * dv * 2 below 2^31 (RODIMUS_ERR_INVALID_ARG).
 *   dk, dv        64 or 128.
 *   window        tokens each query attends to, itself included (>= 1).
 *   scale         score scale; 0 = 1 / sqrt(dk).  Negative, Inf or NaN:
 *                 RODIMUS_ERR_INVALID_ARG.
 *   in_dtype      RODIMUS_DTYPE_BF16 (others: RODIMUS_ERR_UNSUPPORTED).
 *   q             [B, T, H, dk]; k [B, T, dk] (shared); v [B, T, H, dv].
 *   out           [B, T, H, dv] fp32; must not overlap the inputs.
 * Precision: q . k on bf16 MFMA with fp32 accumulation (exact products), the
 * softmax in fp32, the probabilities split into two bf16 terms for the
 * product with v.  No workspace.
 */
rodimus_status rodimus_swska_fwd(int B, int T, int H, int dk, int dv, int window, float scale,
                                 rodimus_dtype in_dtype, const void *q, const void *k,
                                 const void *v, float *out, hipStream_t stream);

/*
 * Backward of rodimus_ddts_chunk_fwd (the training pass's other half): the
 * gradients of a loss L with respect to every input of the forward, given
 * dL/d out and optionally dL/d final_state.  The pages state that training
 * runs the recurrence chunkwise in parallel (rebuttal page, bullet "Efficient
 * Parallelization", and the answer on sequential processing bottlenecks);
 * the gradients are those of the recurrence in the header comment.  At g = 0,
 * where g^tau has no derivative, its terms in dg and dtau are taken as 0.
 *
 *   B, T, H, dk, dv  as rodimus_ddts_chunk_fwd (every dk, dv in {16, 32, 64, 128}).
 *   in_dtype, q, k, g, tau, v, beta_hat, initial_state
 *                    the forward's inputs (initial_state may be NULL = zeros).
 *   d_out            [B, T, H, dv] fp32, dL/d out.
 *   d_final_state    [B, H, dk, dv] fp32 or NULL (= zeros).
 *   dq, dk_, dg, dtau  [B, T, H, dk] fp32 outputs.
 *   dv_, dbeta_hat   [B, T, H, dv] fp32 outputs.
 *   d_initial_state  [B, H, dk, dv] fp32 output or NULL.
 *   workspace        device buffer of rodimus_ddts_chunk_bwd_workspace_bytes:
 *                    the forward's state entering every chunk (64 tokens; 32 at
 *                    dk = 128), its final state, and dL/dS leaving every chunk,
 *                    all recomputed here.
 * Outputs must not overlap each other, the inputs or the workspace.
 * Precision: as the forward (bf16 MFMA products on split operands, fp32
 * accumulation and state).
 */
rodimus_status rodimus_ddts_chunk_bwd(
    int B, int T, int H, int dk, int dv, rodimus_dtype in_dtype,
    const void *q, const void *k, const void *g, const void *tau,
    const void *v, const void *beta_hat, const float *initial_state,
    const float *d_out, const float *d_final_state,
    float *dq, float *dk_, float *dg, float *dtau, float *dv_, float *dbeta_hat,
    float *d_initial_state, void *workspace, size_t workspace_bytes, hipStream_t stream);

size_t rodimus_ddts_chunk_bwd_workspace_bytes(int B, int T, int H, int dk, int dv);

#ifdef __cplusplus
}
#endif

#endif /* RODIMUS_DDTS_H */
