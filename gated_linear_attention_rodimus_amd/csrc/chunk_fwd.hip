// chunk_fwd.hip -- dispatch of the chunk-forward kernels by dk, and the two
// small kernels of the segmented path: the ordered combination of segment
// state transfers and the state copy used when T == 0.
//
// Segmented path (long sequences with few heads): the sequence of one (b, h)
// is cut into P pieces.  Chaining the recurrence over a piece from state X
// gives diag(G_p) X + dS_p, where G_p is the product of the piece's forget
// gates and dS_p the piece's result from a zero state.  These affine maps
// compose in order, so S_in[p] = diag(G_{p-1}) S_in[p-1] + dS_{p-1}; the
// pieces then run in parallel from their true incoming states.  This only
// reorders the recurrence's own products and sums (the chunkwise-parallel
// training form of the rebuttal page, paperhub.cn, answer on sequential
// processing bottlenecks).
#include "internal.h"

namespace rodimus {

size_t chunk_lds_bytes_dk16(int, int, bool);
size_t chunk_lds_bytes_dk32(int, int, bool);
size_t chunk_lds_bytes_dk64(int, int, bool);
size_t chunk_lds_bytes_dk128(int, int, bool);
int chunk_per_cu_dk16(int, int, bool, bool);
int chunk_per_cu_dk32(int, int, bool, bool);
int chunk_per_cu_dk64(int, int, bool, bool);
int chunk_per_cu_dk128(int, int, bool, bool);
hipError_t launch_chunk_dk16(const ChunkLaunch &, hipStream_t);
hipError_t launch_chunk_dk32(const ChunkLaunch &, hipStream_t);
hipError_t launch_chunk_dk64(const ChunkLaunch &, hipStream_t);
hipError_t launch_chunk_dk128(const ChunkLaunch &, hipStream_t);
size_t chunk_lds_bytes_dk16_fu(int, int, bool);
size_t chunk_lds_bytes_dk32_fu(int, int, bool);
size_t chunk_lds_bytes_dk64_fu(int, int, bool);
size_t chunk_lds_bytes_dk128_fu(int, int, bool);
int chunk_per_cu_dk16_fu(int, int, bool, bool);
int chunk_per_cu_dk32_fu(int, int, bool, bool);
int chunk_per_cu_dk64_fu(int, int, bool, bool);
int chunk_per_cu_dk128_fu(int, int, bool, bool);
hipError_t launch_chunk_dk16_fu(const ChunkLaunch &, hipStream_t);
hipError_t launch_chunk_dk32_fu(const ChunkLaunch &, hipStream_t);
hipError_t launch_chunk_dk64_fu(const ChunkLaunch &, hipStream_t);
hipError_t launch_chunk_dk128_fu(const ChunkLaunch &, hipStream_t);
hipError_t launch_chunk_dk16_fn(const ChunkLaunch &, hipStream_t);
hipError_t launch_chunk_dk32_fn(const ChunkLaunch &, hipStream_t);
hipError_t launch_chunk_dk64_fn(const ChunkLaunch &, hipStream_t);
hipError_t launch_chunk_dk128_fn(const ChunkLaunch &, hipStream_t);

namespace {

// ---------------------------------------------------------------- segment combine
// S_in[0] = S0 (or 0); S_in[p + 1] = the transfers p * per .. p * per + per - 1
// applied in order to S_in[p] (each: S <- diag(gam[j]) S + dS[j]); S_in[p] is
// written to slot p, after every transfer in that slot has been read.  One
// thread per state element, sequential over the transfers.  Up to 32
// transfers are all loaded first (one memory latency for the whole chain);
// beyond that, the next segment's transfers (per <= 4) are loaded while the
// current ones are applied.
__global__ __launch_bounds__(256) void segment_combine_kernel(
    int n_seg, int per, int slots, int dk, int dv, const float *__restrict__ s0,
    float *__restrict__ ds, const float *__restrict__ gam)
{
    const int bh = blockIdx.y;
    const int e = blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= dk * dv) return;
    const int i = e / dv;
    const size_t st = (size_t)dk * dv;
    float run = s0 ? s0[(size_t)bh * st + e] : 0.f;
    float *d = ds + (size_t)bh * slots * st + e;
    const float *gm = gam + (size_t)bh * slots * dk + i;
    const int ntr = (n_seg - 1) * per;
    if (ntr <= 32) {
        float dd[32], gg[32];
#pragma unroll
        for (int j = 0; j < 32; ++j)
            if (j < ntr) {
                dd[j] = d[(size_t)j * st];
                gg[j] = gm[(size_t)j * dk];
            }
#pragma unroll
        for (int j = 0; j < 32; ++j)
            if (j < ntr) {
                if ((j & (per - 1)) == 0) d[(size_t)(j / per) * st] = run;   // S_in of segment j / per
                run = gg[j] * run + dd[j];
            }
        d[(size_t)(n_seg - 1) * st] = run;
        return;
    }
    float nd[4] = {0.f, 0.f, 0.f, 0.f}, ng[4] = {0.f, 0.f, 0.f, 0.f};
    auto fetch = [&](int p) {
#pragma unroll
        for (int f = 0; f < 4; ++f)
            if (f < per) {
                const int j = p * per + f;
                nd[f] = d[(size_t)j * st];
                ng[f] = gm[(size_t)j * dk];
            }
    };
    fetch(0);
    for (int p = 0; p < n_seg; ++p) {
        const float cur = run;
        if (p + 1 < n_seg) {
            float cd[4], cg[4];
#pragma unroll
            for (int f = 0; f < 4; ++f) { cd[f] = nd[f]; cg[f] = ng[f]; }
            if (p + 2 < n_seg) fetch(p + 1);
#pragma unroll
            for (int f = 0; f < 4; ++f)
                if (f < per) run = cg[f] * run + cd[f];
        }
        d[(size_t)p * st] = cur;
    }
}

__global__ __launch_bounds__(256) void state_copy_kernel(const float *__restrict__ src,
                                                         float *__restrict__ dst, size_t n)
{
    const size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e < n) dst[e] = src ? src[e] : 0.f;
}

}  // namespace

size_t chunk_lds_bytes(int dk, int dvt, int C, bool f32_inputs, bool fused)
{
    switch (dk) {
    case 16: return fused ? chunk_lds_bytes_dk16_fu(dvt, C, f32_inputs) : chunk_lds_bytes_dk16(dvt, C, f32_inputs);
    case 32: return fused ? chunk_lds_bytes_dk32_fu(dvt, C, f32_inputs) : chunk_lds_bytes_dk32(dvt, C, f32_inputs);
    case 64: return fused ? chunk_lds_bytes_dk64_fu(dvt, C, f32_inputs) : chunk_lds_bytes_dk64(dvt, C, f32_inputs);
    case 128: return fused ? chunk_lds_bytes_dk128_fu(dvt, C, f32_inputs) : chunk_lds_bytes_dk128(dvt, C, f32_inputs);
    }
    return 0;
}

int chunk_per_cu(int dk, int dvt, int C, bool f32_inputs, bool outputs, bool fused)
{
    switch (dk) {
    case 16: return fused ? chunk_per_cu_dk16_fu(dvt, C, f32_inputs, outputs) : chunk_per_cu_dk16(dvt, C, f32_inputs, outputs);
    case 32: return fused ? chunk_per_cu_dk32_fu(dvt, C, f32_inputs, outputs) : chunk_per_cu_dk32(dvt, C, f32_inputs, outputs);
    case 64: return fused ? chunk_per_cu_dk64_fu(dvt, C, f32_inputs, outputs) : chunk_per_cu_dk64(dvt, C, f32_inputs, outputs);
    case 128: return fused ? chunk_per_cu_dk128_fu(dvt, C, f32_inputs, outputs) : chunk_per_cu_dk128(dvt, C, f32_inputs, outputs);
    }
    return 1;
}

// The fused steps without a ShortConv run the kernels compiled without it (no
// window rows, taps or padding; their LDS layout is no larger and they are
// compiled for the same shapes, so the plan made for the fused kernels holds).
hipError_t launch_chunk(const ChunkLaunch &Lc, hipStream_t stream)
{
    const bool conv = Lc.fused && Lc.fu.conv_w > 1;
    switch (Lc.dk) {
    case 16: return !Lc.fused ? launch_chunk_dk16(Lc, stream)
                              : conv ? launch_chunk_dk16_fu(Lc, stream) : launch_chunk_dk16_fn(Lc, stream);
    case 32: return !Lc.fused ? launch_chunk_dk32(Lc, stream)
                              : conv ? launch_chunk_dk32_fu(Lc, stream) : launch_chunk_dk32_fn(Lc, stream);
    case 64: return !Lc.fused ? launch_chunk_dk64(Lc, stream)
                              : conv ? launch_chunk_dk64_fu(Lc, stream) : launch_chunk_dk64_fn(Lc, stream);
    case 128: return !Lc.fused ? launch_chunk_dk128(Lc, stream)
                               : conv ? launch_chunk_dk128_fu(Lc, stream) : launch_chunk_dk128_fn(Lc, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_segment_combine(int BH, int n_seg, int per, int slots, int dk, int dv,
                                  const float *s0, float *ds_inout, const float *gam,
                                  hipStream_t stream)
{
    // the kernel holds 4 transfers per segment, and masks slots with per - 1
    if (per != 1 && per != 2 && per != 4) return hipErrorInvalidValue;
    const int elems = dk * dv;
    dim3 grid((elems + 255) / 256, BH);
    hipLaunchKernelGGL(segment_combine_kernel, grid, dim3(256), 0, stream, n_seg, per, slots, dk,
                       dv, s0, ds_inout, gam);
    return hipGetLastError();
}

hipError_t launch_state_copy(const float *src, float *dst, size_t count, hipStream_t stream)
{
    if (count == 0) return hipSuccess;
    const size_t blocks = (count + 255) / 256;
    hipLaunchKernelGGL(state_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, src, dst,
                       count);
    return hipGetLastError();
}

}  // namespace rodimus
