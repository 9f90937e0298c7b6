// internal.h -- declarations shared by the library's translation units
// (host-side launchers; kernels stay private to their .hip file).
#pragma once

#include <atomic>
#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime.h>

namespace rodimus {

// Raise a kernel's dynamic-LDS limit to `bytes` once per device (the first
// launch on each device sets it; `done` is that kernel's per-device flags).
// Host threads may race on a first launch: both then set the same attribute
// (idempotent) and both store the flag, which is atomic.  Device indices at
// or beyond kMaxDevices are refused (hipErrorInvalidDevice) rather than
// setting the attribute on every call.
constexpr int kMaxDevices = 64;
inline hipError_t set_lds_limit_once(const void *fn, size_t bytes, std::atomic<bool> *done)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    if (done[dev].load(std::memory_order_acquire)) return hipSuccess;
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e == hipSuccess) done[dev].store(true, std::memory_order_release);
    return e;
}

// Per-token input pointers (device), typed as the storage dtype by the kernels.
struct TokenInputs {
    const void *q, *k, *g, *tau, *v, *beta;
};

// How one chunk-forward call is executed.
struct ChunkPlan {
    int C;          // tokens per chunk
    int Ct;         // tokens per chunk of the segment transfers (C, or C / 2)
    int DVT;        // dv columns per workgroup
    int segments;   // pieces per (b, h) sequence run in parallel (1 = one sweep)
    int n_chunks;   // ceil(T / C)
    int chunks_per_seg;
    // segmented runs: transfers over the chunks before the last segment, in
    // tr_per_seg pieces per segment (tr_per_seg * (segments - 1) of them)
    int tr_per_seg;
    int ws_slots;   // state slots per (b, h) in the workspace
    size_t lds_bytes;
    size_t ws_bytes;
};

// Bytes of LDS the chunk kernel needs for a tile shape (0 if not instantiated),
// with or without the fused steps.
size_t chunk_lds_bytes(int dk, int dvt, int C, bool f32_inputs, bool fused = false);
// Workgroups of the output mode (outputs true) or of the segment-transfer
// mode one CU holds for a tile shape.
int chunk_per_cu(int dk, int dvt, int C, bool f32_inputs, bool outputs, bool fused = false);

// The steps fused around the recurrence (kernels instantiated with them):
// beta_hat = sigmoid(u w) when u is set (u [B][T][H][rank], w [H][rank][dv],
// the inputs' dtype), the feedthrough o += d * v (d [H][dv] fp32, or null),
// and a ShortConv of q, k, v with conv_w taps (1: none; c* [H][D][conv_w]
// fp32; q, k, v then hold conv_w - 1 history rows before token 0).
struct FusedSteps {
    const void *u = nullptr, *w = nullptr;
    int rank = 0;
    const float *d = nullptr;
    int conv_w = 1;
    const float *cq = nullptr, *ck = nullptr, *cv = nullptr;
};

// Chunk sweep / segment pass.  mode 0: outputs from S_in; mode 1: segment
// state transfer (dS from a zero state, and the product of decays).
struct ChunkLaunch {
    int B, T, H, dk, dv;
    int C, DVT, n_seg, chunks_per_seg;
    int mode;
    bool f32_inputs;
    TokenInputs in;
    const float *s_in; long long s_in_bh_stride, s_in_seg_stride;
    float *out;
    float *s_out; long long s_out_bh_stride, s_out_seg_stride; int s_out_last_only;
    float *gam_out;         // mode 1: segment p's decay of head bh at bh * gam_bh_stride + p * dk
    long long gam_bh_stride;
    bool fused = false;     // run the kernels with the fused steps compiled in
    FusedSteps fu;
};
hipError_t launch_chunk(const ChunkLaunch &L, hipStream_t stream);

// Ordered combination of segment transfers: S_in[p] of every segment, in
// place over the transfers (per transfers for each segment but the last;
// slots state slots per head).
hipError_t launch_segment_combine(int BH, int n_seg, int per, int slots, int dk, int dv,
                                  const float *s0, float *ds_inout, const float *gam,
                                  hipStream_t stream);

// Copy or zero a [count] fp32 array (T == 0 forwards).
hipError_t launch_state_copy(const float *src, float *dst, size_t count, hipStream_t stream);

hipError_t launch_decode(int N, int H, int dk, int dv, bool f32_inputs, const TokenInputs &in,
                         float *state, float *out, hipStream_t stream,
                         const FusedSteps *fused = nullptr);

// Backward of the chunk forward: one launch runs the forward state sweep
// (the state entering every chunk, and S_T) and the reverse adjoint sweep
// (dL/dS leaving every chunk, and dL/dS_0) side by side; then one workgroup
// per (b, h, chunk) forms the chunk's gradients.
struct ChunkBwdLaunch {
    int B, T, H, dk, dv;
    bool f32_inputs;
    TokenInputs in;
    const float *s0;        // [B*H][dk][dv] initial state or null
    const float *dout, *dsf;
    float *s_chunks;        // [B*H][ceil(T / chunk)][dk][dv] chunk-start states (written)
    float *s_final;         // [B*H][dk][dv] final state (written)
    float *d_chunks;        // [B*H][ceil(T / chunk)][dk][dv] dL/dS leaving every chunk (written)
    float *dq, *dk_, *dg, *dtau, *dv_, *dbeta, *ds0;
};
// Sliding-window shared-key attention (bf16 inputs, fp32 out), dk, dv in {64, 128}.
hipError_t launch_swska(int B, int T, int H, int dk, int dv, int window, float scale,
                        const void *q, const void *k, const void *v, float *out,
                        hipStream_t stream);

size_t chunk_bwd_lds_bytes(int dk, int dv, bool f32_inputs);   // 0 if the shape is not instantiated
int chunk_bwd_chunk(int dk);                   // tokens per chunk of the backward
hipError_t launch_chunk_bwd(const ChunkBwdLaunch &L, hipStream_t stream);

}  // namespace rodimus
