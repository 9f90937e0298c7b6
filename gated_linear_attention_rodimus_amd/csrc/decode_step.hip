// decode_step.hip -- one recurrent DDTS step over a batch of resident states.
//
// Sequential inference over a cached fixed-size state (Rodimus* rebuttal page,
// paperhub.cn, answer on sequential processing bottlenecks): per (n, h)
//   S <- diag(exp(-g*tau)) S + (g^tau * k)(beta_hat * v)^T,   o = S^T q
// with the gates of the Rodimus* digest page (digest.lyk-ai.com), "Method".
//
// The step is bound by HBM: the fp32 state (dk*dv*4 bytes per head) is read
// and written once, the inputs are ~3% of the traffic.  One workgroup of 256
// threads owns one (or, for small heads, several) state slices:
//  - each thread owns one float4 column group c (dv/4 of them per row) and a
//    fixed set of rows, so every wave-wide load or store touches whole 128-byte
//    lines (coalesced 128-bit accesses), all loads issued before any math;
//  - per-row gates (alpha_i, alpha_hat_i*k_i) and per-column v'_j are computed
//    once per slice into LDS while the state loads are in flight;
//  - o_j = sum_i q_i S_ij is reduced over the row groups through LDS.
#include "internal.h"

namespace rodimus {
namespace {

constexpr int kThreads = 256;
typedef float f4v __attribute__((ext_vector_type(4)));
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float ld_in(const __bf16 *p, size_t i) { return (float)p[i]; }
__device__ __forceinline__ float ld_in(const float *p, size_t i) { return p[i]; }

// alpha_hat = g^tau with pow semantics at g = 0 (0^0 = 1, 0^tau = 0).
__device__ __forceinline__ float gate_pow(float g, float tau) {
    if (g > 0.f) return __builtin_amdgcn_exp2f(tau * __builtin_amdgcn_logf(g));
    return tau == 0.f ? 1.f : 0.f;
}

// The fused steps of a decode step (FU kernels): beta_hat = sigmoid(u w)
// when u is set (u [N][H][rank], w [H][rank][dv]), o += d * v when d is set,
// and a ShortConv of q, k, v over the window of their last conv_w raw tokens
// ([N][conv_w][H][D], oldest first) when conv_w > 1.
struct DecodeFused {
    const void *u, *w;
    int rank, H, conv_w;
    const float *d, *cq, *ck, *cv;
};

template <typename TIn>
__device__ __forceinline__ float conv_at(const TIn *x, const float *c, int n, int h, int H, int D,
                                         int i, int W)
{
    // y = sum_j c[j] x[newest - j]; window row r holds raw token r (oldest first)
    float acc = 0.f;
    for (int j = 0; j < W; ++j)
        acc = __builtin_fmaf(c[((size_t)h * D + i) * W + j],
                             ld_in(x, (((size_t)n * W + (W - 1 - j)) * H + h) * D + i), acc);
    return acc;
}

template <int DK, int DV, typename TIn, bool FU>
__global__ __launch_bounds__(kThreads) void decode_step_kernel(
    int pairs, const TIn *__restrict__ q, const TIn *__restrict__ k, const TIn *__restrict__ g,
    const TIn *__restrict__ tau, const TIn *__restrict__ v, const TIn *__restrict__ beta,
    float *__restrict__ state, float *__restrict__ out, DecodeFused f)
{
    constexpr int CG = DV / 4;                       // float4 column groups per row
    constexpr int F4 = DK * DV / 4;                  // float4s per slice
    constexpr int PPB = F4 >= kThreads ? 1 : kThreads / F4;   // slices per block
    constexpr int TPP = kThreads / PPB;              // threads per slice
    constexpr int PER = F4 / TPP;                    // float4s per thread
    constexpr int RG = TPP / CG;                     // row groups per slice
    static_assert(PER >= 1 && F4 % TPP == 0 && TPP % CG == 0, "tile shape");

    __shared__ float s_a[PPB][DK], s_kk[PPB][DK], s_q[PPB][DK], s_vv[PPB][DV];
    __shared__ float s_vf[FU ? PPB : 1][FU ? DV : 1];    // FU: v entering the recurrence
    __shared__ float s_red[PPB][RG][DV];

    const int t = threadIdx.x;
    const int slot = t / TPP, lt = t % TPP;
    const int pair = blockIdx.x * PPB + slot;
    const bool active = pair < pairs;
    const int c = lt % CG, rg = lt / CG;

    float4 *S = reinterpret_cast<float4 *>(state) + (size_t)(active ? pair : 0) * F4;
    float4 s[PER];
    // the slice is read once per step: non-temporal loads keep it from
    // displacing other data in the caches
#pragma unroll
    for (int m = 0; m < PER; ++m) {
        const f4v y = active ? __builtin_nontemporal_load((const f4v *)&S[lt + m * TPP])
                             : f4v{0.f, 0.f, 0.f, 0.f};
        s[m] = make_float4(y[0], y[1], y[2], y[3]);
    }

    // gates for this slice (rows over dk, columns over dv)
    if (active && !FU) {
        const size_t rk = (size_t)pair * DK, rv = (size_t)pair * DV;
        for (int i = lt; i < DK; i += TPP) {
            const float gi = ld_in(g, rk + i), ti = ld_in(tau, rk + i);
            s_a[slot][i] = __builtin_amdgcn_exp2f(-gi * ti * kLog2e);
            s_kk[slot][i] = gate_pow(gi, ti) * ld_in(k, rk + i);
            s_q[slot][i] = ld_in(q, rk + i);
        }
        for (int j = lt; j < DV; j += TPP)
            s_vv[slot][j] = ld_in(beta, rv + j) * ld_in(v, rv + j);
    }
    if constexpr (FU) {
        if (active) {
            const int n = pair / f.H, h = pair % f.H;
            const size_t rk = (size_t)pair * DK, rv = (size_t)pair * DV;
            for (int i = lt; i < DK; i += TPP) {
                const float gi = ld_in(g, rk + i), ti = ld_in(tau, rk + i);
                const float ki = f.conv_w > 1 ? conv_at(k, f.ck, n, h, f.H, DK, i, f.conv_w) : ld_in(k, rk + i);
                const float qi = f.conv_w > 1 ? conv_at(q, f.cq, n, h, f.H, DK, i, f.conv_w) : ld_in(q, rk + i);
                s_a[slot][i] = __builtin_amdgcn_exp2f(-gi * ti * kLog2e);
                s_kk[slot][i] = gate_pow(gi, ti) * ki;
                s_q[slot][i] = qi;
            }
            const TIn *u = (const TIn *)f.u, *w = (const TIn *)f.w;
            for (int j = lt; j < DV; j += TPP) {
                const float vj = f.conv_w > 1 ? conv_at(v, f.cv, n, h, f.H, DV, j, f.conv_w) : ld_in(v, rv + j);
                float bj;
                if (u) {
                    float z = 0.f;
                    for (int r = 0; r < f.rank; ++r)
                        z = __builtin_fmaf(ld_in(u, (size_t)pair * f.rank + r),
                                           ld_in(w, ((size_t)h * f.rank + r) * DV + j), z);
                    bj = __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-kLog2e * z));
                } else {
                    bj = ld_in(beta, rv + j);
                }
                s_vv[slot][j] = bj * vj;
                s_vf[slot][j] = vj;
            }
        }
    }
    __syncthreads();

    if (active) {
        const float v0 = s_vv[slot][4 * c], v1 = s_vv[slot][4 * c + 1];
        const float v2 = s_vv[slot][4 * c + 2], v3 = s_vv[slot][4 * c + 3];
        float o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f;
#pragma unroll
        for (int m = 0; m < PER; ++m) {
            const int i = rg + m * RG;               // row of this float4
            const float a = s_a[slot][i], kk = s_kk[slot][i], qi = s_q[slot][i];
            float4 x = s[m];
            x.x = a * x.x + kk * v0;
            x.y = a * x.y + kk * v1;
            x.z = a * x.z + kk * v2;
            x.w = a * x.w + kk * v3;
            // streamed back with the non-temporal policy: the next read of this
            // slice is a whole step (every other layer's state) away
            __builtin_nontemporal_store(f4v{x.x, x.y, x.z, x.w}, (f4v *)&S[lt + m * TPP]);
            o0 += qi * x.x; o1 += qi * x.y; o2 += qi * x.z; o3 += qi * x.w;
        }
        s_red[slot][rg][4 * c] = o0;
        s_red[slot][rg][4 * c + 1] = o1;
        s_red[slot][rg][4 * c + 2] = o2;
        s_red[slot][rg][4 * c + 3] = o3;
    }
    __syncthreads();
    if (active) {
        for (int j = lt; j < DV; j += TPP) {
            float acc = 0.f;
#pragma unroll
            for (int r = 0; r < RG; ++r) acc += s_red[slot][r][j];
            if constexpr (FU) {
                if (f.d) acc = __builtin_fmaf(f.d[(size_t)(pair % f.H) * DV + j], s_vf[slot][j], acc);
            }
            out[(size_t)pair * DV + j] = acc;
        }
    }
}

template <int DK, int DV, typename TIn>
hipError_t launch_typed(int pairs, const TokenInputs &in, float *state, float *out,
                        const DecodeFused *f, hipStream_t stream)
{
    constexpr int F4 = DK * DV / 4;
    constexpr int PPB = F4 >= kThreads ? 1 : kThreads / F4;
    const int blocks = (pairs + PPB - 1) / PPB;
    if (f) {
        hipLaunchKernelGGL((decode_step_kernel<DK, DV, TIn, true>), dim3(blocks), dim3(kThreads), 0,
                           stream, pairs, (const TIn *)in.q, (const TIn *)in.k, (const TIn *)in.g,
                           (const TIn *)in.tau, (const TIn *)in.v, (const TIn *)in.beta, state, out,
                           *f);
    } else {
        hipLaunchKernelGGL((decode_step_kernel<DK, DV, TIn, false>), dim3(blocks), dim3(kThreads), 0,
                           stream, pairs, (const TIn *)in.q, (const TIn *)in.k, (const TIn *)in.g,
                           (const TIn *)in.tau, (const TIn *)in.v, (const TIn *)in.beta, state, out,
                           DecodeFused{});
    }
    return hipGetLastError();
}

template <typename TIn>
hipError_t launch_dtype(int pairs, int dk, int dv, const TokenInputs &in, float *state,
                        float *out, const DecodeFused *f, hipStream_t stream)
{
#define RODIMUS_DEC_DV(DK)                                                              \
    switch (dv) {                                                                       \
    case 16: return launch_typed<DK, 16, TIn>(pairs, in, state, out, f, stream);        \
    case 32: return launch_typed<DK, 32, TIn>(pairs, in, state, out, f, stream);        \
    case 64: return launch_typed<DK, 64, TIn>(pairs, in, state, out, f, stream);        \
    case 128: return launch_typed<DK, 128, TIn>(pairs, in, state, out, f, stream);      \
    }                                                                                   \
    break;
    switch (dk) {
    case 16: RODIMUS_DEC_DV(16)
    case 32: RODIMUS_DEC_DV(32)
    case 64: RODIMUS_DEC_DV(64)
    case 128: RODIMUS_DEC_DV(128)
    }
#undef RODIMUS_DEC_DV
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(int N, int H, int dk, int dv, bool f32_inputs, const TokenInputs &in,
                         float *state, float *out, hipStream_t stream, const FusedSteps *fused)
{
    const int pairs = N * H;
    DecodeFused f{};
    if (fused) {
        f.u = fused->u; f.w = fused->w; f.rank = fused->rank; f.H = H;
        f.conv_w = fused->conv_w; f.d = fused->d;
        f.cq = fused->cq; f.ck = fused->ck; f.cv = fused->cv;
    }
    const DecodeFused *fp = fused ? &f : nullptr;
    return f32_inputs ? launch_dtype<float>(pairs, dk, dv, in, state, out, fp, stream)
                      : launch_dtype<__bf16>(pairs, dk, dv, in, state, out, fp, stream);
}

}  // namespace rodimus
