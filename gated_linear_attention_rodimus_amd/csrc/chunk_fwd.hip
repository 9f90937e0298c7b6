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

namespace {

// ---------------------------------------------------------------- segment combine
// S_in[0] = S0 (or 0); S_in[p + 1] = the transfers p * per .. p * per + per - 1
// applied in order to S_in[p] (each: S <- diag(gam[j]) S + dS[j]); S_in[p] is
// written to slot p, after every transfer in that slot has been read.  One
// thread per state element, sequential over segments.
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
    for (int p = 0; p < n_seg; ++p) {
        const float cur = run;
        if (p + 1 < n_seg)
            for (int f = 0; f < per; ++f) {
                const int j = p * per + f;
                run = gm[(size_t)j * dk] * run + d[(size_t)j * st];
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

size_t chunk_lds_bytes(int dk, int dvt, int C, bool f32_inputs)
{
    switch (dk) {
    case 16: return chunk_lds_bytes_dk16(dvt, C, f32_inputs);
    case 32: return chunk_lds_bytes_dk32(dvt, C, f32_inputs);
    case 64: return chunk_lds_bytes_dk64(dvt, C, f32_inputs);
    case 128: return chunk_lds_bytes_dk128(dvt, C, f32_inputs);
    }
    return 0;
}

int chunk_per_cu(int dk, int dvt, int C, bool f32_inputs, bool outputs)
{
    switch (dk) {
    case 16: return chunk_per_cu_dk16(dvt, C, f32_inputs, outputs);
    case 32: return chunk_per_cu_dk32(dvt, C, f32_inputs, outputs);
    case 64: return chunk_per_cu_dk64(dvt, C, f32_inputs, outputs);
    case 128: return chunk_per_cu_dk128(dvt, C, f32_inputs, outputs);
    }
    return 1;
}

hipError_t launch_chunk(const ChunkLaunch &Lc, hipStream_t stream)
{
    switch (Lc.dk) {
    case 16: return launch_chunk_dk16(Lc, stream);
    case 32: return launch_chunk_dk32(Lc, stream);
    case 64: return launch_chunk_dk64(Lc, stream);
    case 128: return launch_chunk_dk128(Lc, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_segment_combine(int BH, int n_seg, int per, int slots, int dk, int dv,
                                  const float *s0, float *ds_inout, const float *gam,
                                  hipStream_t stream)
{
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
