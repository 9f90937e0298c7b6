// chunk_bwd.hip -- backward of the chunkwise DDTS forward on gfx950 MFMA.
//
// The training claim of the pages rests on the chunkwise form (Rodimus* rebuttal
// page, paperhub.cn, bullet "Efficient Parallelization"); the backward below is
// derived from the same chunk identity (the one chunk_kernel.h evaluates):
//   O   = tril(Qt Kt^T) V' + Qt S',        S' = diag(e^{b_m}) S_in
//   S_o = diag(e^{b_L}) S_in + diag(f) Kt^T V',   f = e^{b_L - b_m}
// with Qt = q e^{b - b_m}, Kt = k' e^{b_m - b}, k' = g^tau k, V' = beta_hat v,
// b the chunk-local inclusive cumulative sum of lambda = -g tau.  Given
// dO = dL/dO and D = dL/dS_o of a chunk:
//   dA   = tril(dO V'^T)                       A = tril(Qt Kt^T)
//   dQt  = diag-cols(e^{b_m}) (dO S_in^T) + dA Kt
//   dKt  = diag-cols(f) (V' D^T) + dA^T Qt
//   dV'  = A^T dO + (Kt diag(f)) D
//   dL/dS_in = diag(e^{b_L}) D + (q e^{b})^T dO          (the previous chunk's D)
//   dq = e^{b - b_m} dQt,  dk' = e^{b_m - b} dKt,  dk = g^tau dk',  d(g^tau) = k dk',
//   dv = beta_hat dV',  dbeta_hat = v dV'
//   dlambda_r = sum_{u >= r} (q_u dq_u - k'_u dk'_u) + rowsum(S_o * D)   (per dk column;
//               the sum runs over the chunk's tokens u >= r)
//   dg = -tau dlambda + tau g^(tau-1) d(g^tau),  dtau = -g dlambda + ln(g) g^tau d(g^tau)
// (the g^tau terms taken as 0 at g = 0).  The dlambda identity replaces the
// per-token state products of a token-level backward: every output and the
// chunk-end state depend on lambda_r only through e^{b_u - b_s} with s < r <= u
// and through e^{b_u}, e^{b_L}, which is what the two sums count.
//
// Only two things are sequential over chunks: the forward state S (entering
// each chunk) and the state adjoint D (leaving each chunk).  So a call runs
//   (1, 2) state_sweeps_kernel: S forwards and D backwards over the chunks
//       (the S_o and dL/dS_in lines above), side by side in one launch, one
//       workgroup per (b, h, dv tile) and direction, writing S_in and D of
//       every chunk, S_T and dL/dS_0;
//   (3) chunk_grad_kernel: one workgroup per (b, h, chunk), every chunk in
//       parallel, forming all of the chunk's gradients from S_in and D (the
//       rowsum(S_o * D) term from S_in and the state term of dKt).
// Every product is a 16x16-tile MFMA (v_mfma_f32_16x16x32_bf16, fp32
// accumulate) whose fp32 operands are split into NS bf16 terms (NS = 2 for
// bf16 inputs, 3 for fp32), as in the forward.  Tail tokens read as zero
// (inert) and their gradients are not stored.
#include "chunk_kernel.h"

namespace rodimus {
namespace bwd_detail {

using chunk_detail::bf16x4;
using chunk_detail::bf16x8;
using chunk_detail::f32x4;
using chunk_detail::kLog2e;
using chunk_detail::mma_split;

// tokens per chunk: the forward's chunk length for the same dk (64, or 32 at
// dk = 128 where a 64-token forward chunk does not fit in LDS)
template <int DK> struct ChunkOf { static constexpr int C = DK == 128 ? 32 : 64; };

using chunk_detail::make_rsrc;
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Per-token tensors are read and written through buffer resources based at
// the chunk's first token of head h and ending with the sequence (tokens past
// T read as zero and their stores are dropped by the range check), so no
// load sits behind a branch and offsets stay 32-bit.
template <typename TIn>
__device__ __forceinline__ typename chunk_detail::InRaw<TIn>::type ld_raw(rsrc_t r, unsigned off_elems) {
    typedef typename chunk_detail::InRaw<TIn>::type Raw;
    return chunk_detail::buf_load(r, off_elems * (unsigned)sizeof(TIn), Raw());
}
template <typename TIn>
__device__ __forceinline__ float ld_tok(rsrc_t r, unsigned off_elems) {
    return chunk_detail::in_to_f32(ld_raw<TIn>(r, off_elems));
}

// g^tau with pow semantics at g = 0
__device__ __forceinline__ float gate_pow(float g, float tau) {
    if (g > 0.f) return __builtin_amdgcn_exp2f(tau * __builtin_amdgcn_logf(g));
    return tau == 0.f ? 1.f : 0.f;
}

template <int NS>
__device__ __forceinline__ void split8(const float *x, bf16x8 *out) {
    unsigned w[4][NS];
#pragma unroll
    for (int p = 0; p < 4; ++p) chunk_detail::split_pair<NS>(x[2 * p], x[2 * p + 1], w[p]);
#pragma unroll
    for (int n = 0; n < NS; ++n) out[n] = chunk_detail::pack8(w[0][n], w[1][n], w[2][n], w[3][n]);
}

// k-slot e (0..7) of lane group lg in a 32-deep MFMA step: lane group lg takes
// k = 4 lg .. 4 lg + 3 and 16 + 4 lg .. 16 + 4 lg + 3, for both operands.
__device__ __forceinline__ int kslot(int lg, int e) { return e < 4 ? 4 * lg + e : 12 + 4 * lg + e; }

// The 8 operand values of one lane for the step k0 of a length-K contraction,
// from a row-major array whose rows run along k: x[e] = p[row * pitch + k0 +
// kslot(lg, e)] (two 16-byte reads; zero past K when K = 16).
template <int K>
__device__ __forceinline__ void op_rows(const float *p, int pitch, int row, int k0, int lg, float *x) {
    const float *s = p + (size_t)row * pitch + k0 + 4 * lg;
    const f32x4 a = *(const f32x4 *)s;
    x[0] = a[0]; x[1] = a[1]; x[2] = a[2]; x[3] = a[3];
    if constexpr (K >= 32) {
        const f32x4 b = *(const f32x4 *)(s + 16);
        x[4] = b[0]; x[5] = b[1]; x[6] = b[2]; x[7] = b[3];
    } else {
        x[4] = x[5] = x[6] = x[7] = 0.f;
    }
}

// ------------------------------------------------------------------ (1, 2) state sweeps

struct SweepArgs {
    int T, H, dv, n_chunks;
    const void *q, *k, *g, *tau, *v, *beta;
    const float *s0;           // [B*H][DK][dv] initial state or null (zeros)
    const float *dout, *dsf;   // dL/d out, dL/dS_T (or null)
    float *s_chunks;           // [B*H][n_chunks][DK][dv]: S entering every chunk
    float *s_final;            // [B*H][DK][dv]: S_T
    float *d_chunks;           // [B*H][n_chunks][DK][dv]: D = dL/dS leaving every chunk
    float *ds0;                // [B*H][DK][dv] or null
};

// The two sequential parts, one the mirror of the other, for one (b, h) and JT
// columns of dv:
//   forward (REV = false), chunks first to last:  store X = S entering the
//     chunk, then S <- diag(e^{b_L}) S + (k' e^{b_L - b})^T V';
//   reverse (REV = true), chunks last to first:  store X = D leaving the
//     chunk, then D <- diag(e^{b_L}) D + (q e^{b})^T dO;
// with b the chunk's inclusive cumulative sum of -g tau, so both factors are
// at most 1 in size.  Two roles: NP producer waves turn a chunk into the
// token-side factor and the staged operand (V' or dO), both split into NS
// bf16 planes, token-major, in LDS buffer it & 1 of pipeline step it, while
// the DK/16 state waves store X and add the product of the previous chunk
// from the other buffer.  Two workgroup barriers per step:
//   phase 1  producers: issue the next chunk's loads; cumulative sums of
//            g tau over their tokens, scanned over the wave's token groups;
//            the wave's per-column totals to LDS.
//            state waves: X to the workspace (through LDS, whole rows).
//   phase 2  producers: the other waves' totals complete the sums; factor
//            planes, e^{b_L} per row, the staged operand planes.
//            state waves: X decays by e^{b_L} and takes the MFMA product.
// Memory access is by whole 128-byte lines where the layout allows: a
// producer wave's lanes cover every dk column pair of GW tokens per load (one
// 32-bit load per bf16 pair), the staged operand is read 16 bytes a lane along
// rows, and each state wave's 16 rows of X (one contiguous block when JT = dv)
// are written 16 bytes a lane after a pass through LDS.
//   State waves: wave w owns dk rows 16 w .. 16 w + 15 of the state as MFMA
// C-layout tiles of X^T (lane (lc, lg) holds row 16 w + lc at columns
// 16 jt + 4 lg .. + 3, so the row decay is one scalar per lane).  Both MFMA
// operands come from the planes through the transposing LDS read, which hands
// lane (lc, lg) tokens 4 lg .. + 3 and 16 + 4 lg .. + 3 of a 32-token step,
// the same k-slots for both.
template <int DK, int JT, int NS_>
struct SweepCfg {
    static constexpr int NS = NS_;
    static constexpr int C = ChunkOf<DK>::C;
    // 4 producer waves; 8 at dk = 128, where two register sets of pair loads
    // of 4-wave producers would not fit the registers that a 12-wave
    // workgroup leaves each wave (170) and spill
    static constexpr int NP = DK == 128 ? 8 : 4;
    static constexpr int NRB = DK / 16, NW = NP + NRB, NT = 64 * NW;
    static constexpr int PP = DK / 2;                          // dk column pairs
    static constexpr int GW = 64 / PP;                         // token groups per producer wave
    static constexpr int G = GW * NP, TPG = C / G;             // token groups, tokens per group
    // plane row strides (bf16): four consecutive rows of a transposing read
    // fall in distinct banks
    static constexpr int RSA = DK == 16 ? 20 : DK == 32 ? 36 : DK == 64 ? 76 : 148;
    static constexpr int RSB = JT + 16;
    static constexpr int XS = JT + 4;                          // X staging row stride (fp32)
    static constexpr size_t a_bytes = (size_t)NS * C * RSA * 2;     // factor planes
    static constexpr size_t b_bytes = (size_t)NS * C * RSB * 2;     // staged operand planes
    static constexpr size_t buf = a_bytes + b_bytes + (size_t)DK * 4;   // + e^{b_L} per row
    static constexpr size_t t_off = 2 * buf;                   // [NP][DK] per-wave sums of g tau
    static constexpr size_t x_off = t_off + (size_t)NP * DK * 4;    // [NRB][16][XS] X staging
    static constexpr size_t bytes = x_off + (size_t)NRB * 16 * XS * 4;
    static_assert(GW * PP == 64 && TPG * G == C && TPG >= 1, "producer lanes");
    static_assert(C % 32 == 0 && JT % 16 == 0, "tile multiples");
};

// The dv tile of a sweep workgroup: the full dv, halved where the buffers
// would not fit in LDS (fp32 inputs, dk = 64, dv = 128) or the registers of a
// 16-wave workgroup (fp32 inputs, dk = dv = 128).
template <int DK, int DV, int NS>
struct SweepTile {
    static constexpr bool halve = SweepCfg<DK, DV, NS>::bytes > 160 * 1024 || (NS == 3 && DK == 128 && DV == 128);
    static constexpr int JT = halve ? DV / 2 : DV;
};

// acc[t] += the split product of A[t] and the shared operand Bv (term pairs
// of total order < NS, smallest first) for NT independent tiles, issued
// term-major so consecutive MFMAs never depend on each other.
template <int NS, int NT>
__device__ __forceinline__ void mma_split_shared(const bf16x8 (*A)[NS], const bf16x8 *Bv, f32x4 *acc) {
    if constexpr (NS == 3) {
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[t][1], Bv[1], acc[t], 0, 0, 0);
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[t][0], Bv[2], acc[t], 0, 0, 0);
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[t][2], Bv[0], acc[t], 0, 0, 0);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[t][0], Bv[1], acc[t], 0, 0, 0);
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[t][1], Bv[0], acc[t], 0, 0, 0);
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[t][0], Bv[0], acc[t], 0, 0, 0);
}

template <int DK, int JT, typename TIn, bool REV>
__device__ __forceinline__ void state_sweep(const SweepArgs &a, unsigned char *smem)
{
    constexpr int NS = std::is_same<TIn, float>::value ? 3 : 2;
    typedef SweepCfg<DK, JT, NS> L;
    constexpr int C = L::C, NP = L::NP, NRB = L::NRB, PP = L::PP, GW = L::GW, TPG = L::TPG;
    constexpr int RSA = L::RSA, RSB = L::RSB, XS = L::XS, NJ = JT / 16, KSC = C / 32, NPT = 64 * NP;
    constexpr int JG = NJ < 4 ? NJ : NRB >= 8 ? 2 : 4;     // fewer operands live at 8 state waves
    typedef typename std::conditional<REV, float, TIn>::type TB;   // staged operand input type
    constexpr int EPB = 16 / (int)sizeof(TB), NPB = C * JT / EPB, LB = (NPB + NPT - 1) / NPT;
    typedef chunk_detail::Pair<TIn> PR;
    typedef typename PR::type Raw2;
    typedef unsigned u32x4v __attribute__((ext_vector_type(4)));

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int bh = blockIdx.x, j0 = blockIdx.y * JT;
    const int b = bh / a.H, h = bh % a.H, dv = a.dv, nc = a.n_chunks;
    auto planeA = [&](int buf, int n) { return (__bf16 *)(smem + buf * L::buf) + (size_t)n * C * RSA; };
    auto planeB = [&](int buf, int n) {
        return (__bf16 *)(smem + buf * L::buf + L::a_bytes) + (size_t)n * C * RSB;
    };
    auto ebl_of = [&](int buf) { return (float *)(smem + buf * L::buf + L::a_bytes + L::b_bytes); };
    float *tots = (float *)(smem + L::t_off);
    auto chunk_of = [&](int it) { return REV ? nc - 1 - it : it; };

    if (wave >= NRB) {
        // ------------------------------------------------ producers
        const long long T = a.T, H = a.H, row0 = (long long)b * T * H + h;
        const int ptid = tid - 64 * NRB, pw = wave - NRB, gw = lane / PP, pl = lane % PP;
        const int gi = pw * GW + gw, c0 = 2 * pl;       // token group; dk columns c0, c0 + 1
        const TIn *gx = (const TIn *)(REV ? a.q : a.k), *gg = (const TIn *)a.g, *gt = (const TIn *)a.tau;
        const TB *gb0 = REV ? (const TB *)a.dout : (const TB *)a.v, *gb1 = (const TB *)a.beta;
        struct Regs {
            Raw2 x[TPG], g[TPG], t[TPG];
            u32x4v b0[LB], b1[REV ? 1 : LB];
        };
        auto load = [&](int c, Regs &R) {
            const long long t0 = (long long)c * C, lim = (T - t0) * H - h;
            const size_t bk = (size_t)(row0 + t0 * H) * DK, bv = (size_t)(row0 + t0 * H) * dv;
            const rsrc_t Rx = make_rsrc(gx + bk, lim * DK * (long long)sizeof(TIn));
            const rsrc_t Rg = make_rsrc(gg + bk, lim * DK * (long long)sizeof(TIn));
            const rsrc_t Rt = make_rsrc(gt + bk, lim * DK * (long long)sizeof(TIn));
#pragma unroll
            for (int m = 0; m < TPG; ++m) {
                const unsigned o = (unsigned)(((gi * TPG + m) * H * DK + c0) * (long long)sizeof(TIn));
                R.g[m] = PR::load(Rg, o);
                R.t[m] = PR::load(Rt, o);
                R.x[m] = PR::load(Rx, o);
            }
            const rsrc_t Rb0 = make_rsrc(gb0 + bv, lim * dv * (long long)sizeof(TB));
            const rsrc_t Rb1 = make_rsrc(gb1 + bv, REV ? 0 : lim * dv * (long long)sizeof(TB));
#pragma unroll
            for (int m = 0; m < LB; ++m) {
                const int p = ptid + m * NPT, u = p / (JT / EPB), j = (p % (JT / EPB)) * EPB;
                const unsigned o = p < NPB ? (unsigned)((u * H * dv + j0 + j) * (long long)sizeof(TB)) : 0x80000000u;
                R.b0[m] = __builtin_amdgcn_raw_buffer_load_b128(Rb0, o, 0, 0);
                if constexpr (!REV) R.b1[m] = __builtin_amdgcn_raw_buffer_load_b128(Rb1, o, 0, 0);
            }
        };
        auto step = [&](int it, const Regs &R, Regs &nxt) {
            const bool work = it < nc;
            const int pb = it & 1;
            // ---- phase 1: sums of g tau over the thread's tokens, scanned over
            // the wave's GW token groups (lanes pl + PP gw); the wave totals to LDS
            float cum0[TPG], cum1[TPG], ex0 = 0.f, ex1 = 0.f;
            if (work) {
                if (it + 1 < nc) load(chunk_of(it + 1), nxt);
                float run0 = 0.f, run1 = 0.f;
#pragma unroll
                for (int m = 0; m < TPG; ++m) {
                    run0 = PR::gt_lo(R.g[m], R.t[m], run0);
                    run1 = PR::gt_hi(R.g[m], R.t[m], run1);
                    cum0[m] = run0;
                    cum1[m] = run1;
                }
                float in0 = run0, in1 = run1;
#pragma unroll
                for (int s = 1; s < GW; s <<= 1) {
                    const float y0 = __shfl_up(in0, s * PP), y1 = __shfl_up(in1, s * PP);
                    if (gw >= s) { in0 += y0; in1 += y1; }
                }
                ex0 = in0 - run0;
                ex1 = in1 - run1;
                if (gw == GW - 1) *(float2 *)(tots + pw * DK + c0) = make_float2(in0, in1);
            }
            __syncthreads();
            // ---- phase 2: the earlier waves' totals complete the sums; planes
            if (work) {
                float tot0 = 0.f, tot1 = 0.f;
#pragma unroll
                for (int w = 0; w < NP; ++w) {
                    const float2 x = *(const float2 *)(tots + w * DK + c0);
                    if (w < pw) { ex0 += x.x; ex1 += x.y; }
                    tot0 += x.x;
                    tot1 += x.y;
                }
#pragma unroll
                for (int m = 0; m < TPG; ++m) {
                    const float s0 = ex0 + cum0[m], s1 = ex1 + cum1[m];      // -b_u (nats)
                    float f0, f1;
                    if constexpr (REV) {                                          // q e^{b}
                        f0 = PR::lo(R.x[m]) * __builtin_amdgcn_exp2f(-kLog2e * s0);
                        f1 = PR::hi(R.x[m]) * __builtin_amdgcn_exp2f(-kLog2e * s1);
                    } else {                                                      // k' e^{b_L - b}
                        const float la0 = chunk_detail::log2_gate_pow(PR::lo(R.g[m]), PR::lo(R.t[m]));
                        const float la1 = chunk_detail::log2_gate_pow(PR::hi(R.g[m]), PR::hi(R.t[m]));
                        f0 = PR::lo(R.x[m]) * __builtin_amdgcn_exp2f(__builtin_fmaf(-kLog2e, tot0 - s0, la0));
                        f1 = PR::hi(R.x[m]) * __builtin_amdgcn_exp2f(__builtin_fmaf(-kLog2e, tot1 - s1, la1));
                    }
                    unsigned w[NS];
                    chunk_detail::split_pair<NS>(f0, f1, w);
                    const int u = gi * TPG + m;
#pragma unroll
                    for (int n = 0; n < NS; ++n) *(unsigned *)(planeA(pb, n) + u * RSA + c0) = w[n];
                }
                if (gi == 0)
                    *(float2 *)(ebl_of(pb) + c0) = make_float2(__builtin_amdgcn_exp2f(-kLog2e * tot0),
                                                               __builtin_amdgcn_exp2f(-kLog2e * tot1));
                // the staged operand: V' = beta_hat v (forward) or dO (reverse)
#pragma unroll
                for (int m = 0; m < LB; ++m) {
                    const int p = ptid + m * NPT, u = p / (JT / EPB), j = (p % (JT / EPB)) * EPB;
                    if (p < NPB) {
                        unsigned w[EPB / 2][NS];
#pragma unroll
                        for (int e = 0; e < EPB / 2; ++e) {
                            float x0, x1;
                            if constexpr (REV) {
                                x0 = __uint_as_float(R.b0[m][2 * e]);
                                x1 = __uint_as_float(R.b0[m][2 * e + 1]);
                            } else if constexpr (EPB == 8) {
                                x0 = __uint_as_float(R.b0[m][e] << 16) * __uint_as_float(R.b1[m][e] << 16);
                                x1 = __uint_as_float(R.b0[m][e] & 0xffff0000u) *
                                     __uint_as_float(R.b1[m][e] & 0xffff0000u);
                            } else {
                                x0 = __uint_as_float(R.b0[m][2 * e]) * __uint_as_float(R.b1[m][2 * e]);
                                x1 = __uint_as_float(R.b0[m][2 * e + 1]) * __uint_as_float(R.b1[m][2 * e + 1]);
                            }
                            chunk_detail::split_pair<NS>(x0, x1, w[e]);
                        }
#pragma unroll
                        for (int n = 0; n < NS; ++n) {
                            __bf16 *dst = planeB(pb, n) + u * RSB + j;
                            if constexpr (EPB == 8) *(u32x4v *)dst = u32x4v{w[0][n], w[1][n], w[2][n], w[3][n]};
                            else *(uint2 *)dst = make_uint2(w[0][n], w[1][n]);
                        }
                    }
                }
            }
            __syncthreads();
        };
        Regs R0, R1;
        if (nc > 0) load(chunk_of(0), R0);
        for (int it = 0; it <= nc; it += 2) {
            step(it, R0, R1);
            if (it + 1 <= nc) step(it + 1, R1, R0);
        }
    } else {
        // ------------------------------------------------ state waves
        const int lc = lane & 15, lg = lane >> 4, r = 16 * wave + lc;
        const int trow = 4 * lg + (lc >> 2), tcol = 4 * (lc & 3);
        const float *x0 = REV ? a.dsf : a.s0;
        float *xs = REV ? a.d_chunks : a.s_chunks;
        float *xend = REV ? a.ds0 : a.s_final;
        float *xst = (float *)(smem + L::x_off) + wave * 16 * XS;    // this wave's staging rows
        auto xoff = [&](int jt) { return (size_t)r * dv + j0 + 16 * jt + 4 * lg; };
        f32x4 X[NJ];
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt) X[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (x0)
#pragma unroll
            for (int jt = 0; jt < NJ; ++jt) X[jt] = *(const f32x4 *)(x0 + (size_t)bh * DK * dv + xoff(jt));
        for (int it = 0; it <= nc; ++it) {
            const int cb = (it - 1) & 1;
            if (it >= 1) {
                // X -> LDS -> rows 16 w .. 16 w + 15 of the chunk's slot, 16 bytes a lane
                float *dst = xs + ((size_t)bh * nc + chunk_of(it - 1)) * DK * dv + (size_t)16 * wave * dv + j0;
#pragma unroll
                for (int jt = 0; jt < NJ; ++jt) *(f32x4 *)(xst + lc * XS + 16 * jt + 4 * lg) = X[jt];
#pragma unroll
                for (int i = 0; i < NJ; ++i) {
                    const int e = i * 256 + 4 * lane, row = e / JT, col = e % JT;
                    __builtin_nontemporal_store(*(const f32x4 *)(xst + row * XS + col),
                                                (f32x4 *)(dst + (size_t)row * dv + col));
                }
            }
            __syncthreads();
            if (it >= 1) {
                const float ebl = ebl_of(cb)[r];
#pragma unroll
                for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) X[jt][i] *= ebl;            // row r's decay
#pragma unroll
                for (int ks = 0; ks < KSC; ++ks) {
                    bf16x8 Fa[NS];
#pragma unroll
                    for (int n = 0; n < NS; ++n) {
                        const __bf16 *pa = planeA(cb, n) + (32 * ks + trow) * RSA + 16 * wave + tcol;
                        Fa[n] = chunk_detail::cat(chunk_detail::lds_read_tr(pa),
                                                  chunk_detail::lds_read_tr(pa + 16 * RSA));
                    }
                    // JG independent tiles at a time (term-major MFMA issue)
#pragma unroll
                    for (int jg = 0; jg < NJ; jg += JG) {
                        bf16x8 Bt[JG][NS];
#pragma unroll
                        for (int q = 0; q < JG; ++q)
#pragma unroll
                            for (int n = 0; n < NS; ++n) {
                                const __bf16 *pb = planeB(cb, n) + (32 * ks + trow) * RSB + 16 * (jg + q) + tcol;
                                Bt[q][n] = chunk_detail::cat(chunk_detail::lds_read_tr(pb),
                                                             chunk_detail::lds_read_tr(pb + 16 * RSB));
                            }
                        mma_split_shared<NS, JG>(Bt, Fa, X + jg);           // X^T += B^T factor
                    }
                }
            }
            __syncthreads();
        }
        if (xend)
#pragma unroll
            for (int jt = 0; jt < NJ; ++jt) *(f32x4 *)(xend + (size_t)bh * DK * dv + xoff(jt)) = X[jt];
    }
}

// Both sweeps in one launch (blockIdx.z: 0 forward, 1 reverse); they are
// independent and latency-bound, so their workgroups share the CUs.
template <int DK, int JT, typename TIn>
__global__ __launch_bounds__((SweepCfg<DK, JT, std::is_same<TIn, float>::value ? 3 : 2>::NT))
void state_sweeps_kernel(SweepArgs a)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    if (blockIdx.z == 0) state_sweep<DK, JT, TIn, false>(a, smem);
    else state_sweep<DK, JT, TIn, true>(a, smem);
}

// ------------------------------------------------------------------ (3) chunk gradients

struct GradArgs {
    int T, H, n_chunks, n_work;
    const void *q, *k, *g, *tau, *v, *beta;
    const float *dout;
    const float *s_chunks;     // [B*H][n_chunks][DK][DV] S entering every chunk
    const float *d_chunks;     // [B*H][n_chunks][DK][DV] D leaving every chunk
    float *dq, *dk, *dg, *dtau, *dv, *dbeta;
};

typedef unsigned short u16;

// The matrices the waves share go to LDS already split: NS planes of bf16
// terms per matrix (plane n holds term n of every element), rows padded by 4
// elements.  A row-wise MFMA operand is then two 8-byte reads per plane and no
// arithmetic; a column-wise one two transposing 8-byte reads per plane.
template <int NS>
__device__ __forceinline__ void split1(float x, u16 *t) {
    unsigned w[NS];
    chunk_detail::split_pair<NS>(x, 0.f, w);
#pragma unroll
    for (int n = 0; n < NS; ++n) t[n] = (u16)(w[n] & 0xffffu);
}

// x[e] = element (row, k0 + kslot(lg, e)) of a split matrix with planes pl
// elements apart: operand A[n] for each term n
template <int NS, int K>
__device__ __forceinline__ void sop_rows(const u16 *p0, int pl, int pitch, int row, int k0, int lg, bf16x8 *A) {
#pragma unroll
    for (int n = 0; n < NS; ++n) {
        const u16 *p = p0 + n * pl + row * pitch + k0 + 4 * lg;
        const uint2 a = *(const uint2 *)p;
        const uint2 b = K >= 32 ? *(const uint2 *)(p + 16) : uint2{0u, 0u};
        A[n] = chunk_detail::pack8(a.x, a.y, b.x, b.y);
    }
}

// x[e] = element (k0 + kslot(lg, e), col) for col = 16 tile + lc: two
// transposing reads per plane (lane lc takes column col of tokens k0 + 4 lg
// .. + 3 and k0 + 16 + 4 lg .. + 3, the k-slots of lane group lg)
template <int NS, int K>
__device__ __forceinline__ void sop_cols(const u16 *p0, int pl, int pitch, int col, int k0, int lg, bf16x8 *A) {
    static_assert(K >= 32, "a column-wise operand spans a whole 32-deep step");
    const int lc = col & 15;
    const int row = k0 + 4 * lg + (lc >> 2), c4 = (col - lc) + 4 * (lc & 3);
#pragma unroll
    for (int n = 0; n < NS; ++n) {
        const __bf16 *b = (const __bf16 *)(p0 + n * pl) + row * pitch + c4;
        A[n] = chunk_detail::cat(chunk_detail::lds_read_tr(b), chunk_detail::lds_read_tr(b + 16 * pitch));
    }
}

// LDS layout (bytes).  Split planes: Kt [C][DK]; Qt [C][DK], then A^T [C][C]
// over it; one slab of JS dv columns of dO and V' [C][JS], then dA^T [C][C]
// over dO.  The same area stages output rows as fp32: dV' of a slab
// [C][JS + 4] over the dO and V' planes, then dq, dk, dg, dtau [4][C][DK + 4]
// over everything.
template <int DK, int DV, int NS>
struct GradCfg {
    static constexpr int C = ChunkOf<DK>::C, NU = C / 16, NRB = DK / 16;
    static constexpr int JS = DV < 64 ? DV : 64, NSL = DV / JS, NJS = JS / 16;   // dv slabs
    static constexpr int NW = NRB > 4 ? NRB : 4, NT = 64 * NW;
    static constexpr int PK = DK + 4, PS = JS + 4, PC = C + 4;            // bf16 elements
    static constexpr int LK = C * PK, LS = C * PS, LC = C * PC;           // plane sizes
    static constexpr size_t o_kt = 0, o_qt = o_kt + (size_t)NS * LK * 2;
    static constexpr size_t o_do = o_qt + (size_t)NS * LK * 2, o_vp = o_do + (size_t)NS * LS * 2;
    static constexpr size_t end0 = o_vp + (size_t)NS * LS * 2;
    static constexpr size_t o_at = PC <= PK ? o_qt : end0;
    static constexpr size_t end1 = PC <= PK ? end0 : end0 + (size_t)NS * LC * 2;
    static constexpr size_t o_dat = PC <= PS ? o_do : end1;
    static constexpr size_t end2 = PC <= PS ? end1 : end1 + (size_t)NS * LC * 2;
    static constexpr size_t o_f = end2;
    static constexpr size_t end3 = o_f + (size_t)DK * 4;
    static constexpr int OK = DK + 4, OS = JS + 4;                        // fp32 staging rows
    static constexpr size_t stage_k = (size_t)4 * C * OK * 4;             // at 0
    static constexpr size_t stage_v = (size_t)C * OS * 4;                 // at o_do
    static constexpr size_t need_v = o_do + stage_v;
    static constexpr size_t m01 = end3 > stage_k ? end3 : stage_k;
    static constexpr size_t m02 = m01 > need_v ? m01 : need_v;
    // raw bf16 gates q, k, g, tau [4][C][DK] staged for the transposing read:
    // in phase A over the dO / V' planes (not yet written; past the f vector
    // where those are small), in phase C over the Kt / Qt planes (no longer read)
    static constexpr size_t gs_bytes = (size_t)4 * C * DK * 2;
    static constexpr size_t o_gsa = o_do + gs_bytes <= o_f ? o_do : (end3 + 15) / 16 * 16;
    static constexpr size_t o_gsc = 0;
    static constexpr size_t bytes = m02 > o_gsa + gs_bytes ? m02 : o_gsa + gs_bytes;
    static_assert(o_gsc + gs_bytes <= o_do, "phase C gate staging vs dA^T");
    // the f vector must survive the dv staging
    static_assert(o_f >= need_v || o_f + DK * 4 <= o_do, "f vs dv staging");
};

// Raw bf16 gates of the chunk through LDS: the whole [4][C][DK] block (q, k,
// g, tau) is read by all threads with 16-byte loads, every load instruction
// covering whole 128-byte rows, and stored row-major with the 16-byte pieces
// of row u permuted by (u ^ u >> 2) (which spreads both the stores and the
// transposing reads below over all banks); a state-row wave then reads its 16
// columns in the MFMA C-layout with one transposing read per array and token
// tile.
template <int DK, int C>
__device__ __forceinline__ int gate_slot(int u, int col) {
    constexpr int PCH = DK / 8;
    return u * DK + (((col >> 3) ^ ((u ^ (u >> 2)) & (PCH - 1))) << 3) + (col & 7);
}

template <int DK, int C, int NT>
struct GateStage {
    static constexpr int PCH = DK / 8, NPC = 4 * C * PCH, LPC = (NPC + NT - 1) / NT;
    chunk_detail::u32x4 x[LPC];
    // issue the loads (the array index is uniform over a wave: C * PCH is a
    // multiple of 64)
    __device__ __forceinline__ void load(const rsrc_t *R, unsigned HK, int tid) {
#pragma unroll
        for (int m = 0; m < LPC; ++m) {
            const int p = tid + m * NT;
            const int arr = __builtin_amdgcn_readfirstlane(p / (C * PCH));
            const int u = (p / PCH) % C, c = p % PCH;
            const rsrc_t Ra = arr == 0 ? R[0] : arr == 1 ? R[1] : arr == 2 ? R[2] : R[3];
            x[m] = __builtin_amdgcn_raw_buffer_load_b128(Ra, p < NPC ? (u * HK + 8 * c) * 2u : 0x80000000u, 0, 0);
        }
    }
    __device__ __forceinline__ void store(__bf16 *dst, int tid) const {
#pragma unroll
        for (int m = 0; m < LPC; ++m) {
            const int p = tid + m * NT;
            if (p < NPC) {
                const int arr = p / (C * PCH), u = (p / PCH) % C, c = p % PCH;
                *(chunk_detail::u32x4 *)(dst + arr * C * DK + gate_slot<DK, C>(u, 8 * c)) = x[m];
            }
        }
    }
};

// x_[arr][t][i] = gate arr at token 16 t + 4 lg + i, column 16 w + lc
template <int DK, int C>
__device__ __forceinline__ void read_gates(const __bf16 *src, int w, int lc, int lg, float (*q_)[4], float (*k_)[4],
                                           float (*g_)[4], float (*t_)[4]) {
    const int col = 16 * w + 4 * (lc & 3);
#pragma unroll
    for (int t = 0; t < C / 16; ++t) {
        const int u = 16 * t + 4 * lg + (lc >> 2), o = gate_slot<DK, C>(u, col);
        const bf16x4 a = chunk_detail::lds_read_tr(src + o);
        const bf16x4 b = chunk_detail::lds_read_tr(src + C * DK + o);
        const bf16x4 c = chunk_detail::lds_read_tr(src + 2 * C * DK + o);
        const bf16x4 d = chunk_detail::lds_read_tr(src + 3 * C * DK + o);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            q_[t][i] = (float)a[i]; k_[t][i] = (float)b[i]; g_[t][i] = (float)c[i]; t_[t][i] = (float)d[i];
        }
    }
}

// One workgroup per (b, h, chunk).  Roles of wave w:
//   dk block w (w < DK/16): the gates of columns 16w..16w+15 over the chunk's
//     tokens (lane (lc, lg): column 16 w + lc, tokens 16 t + 4 lg + i, which is
//     also the MFMA C-layout of a [token tile t] x [dk block w] tile and, for
//     t = 2 ks, 2 ks + 1, the k-slots of step ks), then dQt and dKt of the block
//     and the elementwise tail (dq, dk, dlambda, dg, dtau);
//   token tile w (w < C/16): rows w of A^T and dA^T;
//   dv tile w of each slab: dV' of those 16 columns (every thread then forms
//     dv and dbeta_hat from it in the slab's row-store pass).
// bf16 gates reach the dk blocks through LDS (whole-row loads by all threads,
// transposing reads), once for Qt / Kt and again for the elementwise tail.
// The dv slabs are processed one after the other (dA^T, dQt and dKt
// accumulate over them), which keeps the LDS small enough for two workgroups
// per CU: one computes while the other waits for memory.
template <int DK, int DV, typename TIn>
__global__ __launch_bounds__((GradCfg<DK, DV, 2>::NT), (DK <= 64 && !std::is_same<TIn, float>::value ? 2 : 1))
void chunk_grad_kernel(GradArgs a)
{
    constexpr int NS = std::is_same<TIn, float>::value ? 3 : 2;
    typedef GradCfg<DK, DV, NS> L;
    constexpr int C = L::C, NU = L::NU, NRB = L::NRB, NT = L::NT;
    constexpr int JS = L::JS, NSL = L::NSL, NJS = L::NJS;
    constexpr int PK = L::PK, PS = L::PS, PC = L::PC, LK = L::LK, LS = L::LS, LC = L::LC;
    constexpr int KSC = C / 32, KSK = (DK + 31) / 32, KSS = (JS + 31) / 32;
    constexpr int OK = L::OK, OS = L::OS;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    u16 *sKt = (u16 *)(smem + L::o_kt), *sQt = (u16 *)(smem + L::o_qt);
    u16 *sdO = (u16 *)(smem + L::o_do), *sVp = (u16 *)(smem + L::o_vp);
    u16 *sAt = (u16 *)(smem + L::o_at), *sdAt = (u16 *)(smem + L::o_dat);
    float *sF = (float *)(smem + L::o_f);
    float *sOutK = (float *)smem, *sOutV = (float *)(smem + L::o_do);
    typedef typename chunk_detail::InRaw<TIn>::type Raw;

    // work item: workgroups are dealt to the 8 XCDs round-robin; give each XCD
    // a contiguous range of (b, h, chunk), so neighbouring chunks of a head
    // share an L2
    const int per_xcd = (a.n_work + 7) / 8;
    const int wi = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
    if (wi >= a.n_work) return;
    const int bh = wi / a.n_chunks, c = wi % a.n_chunks;
    const int b = bh / a.H, h = bh % a.H;
    const int tid = threadIdx.x, lane = tid & 63, lc = lane & 15, lg = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const long long T = a.T, H = a.H, c0 = (long long)c * C;
    const long long row0 = (long long)b * T * H + h;
    const TIn *gq = (const TIn *)a.q, *gk = (const TIn *)a.k, *gg = (const TIn *)a.g;
    const TIn *gt = (const TIn *)a.tau, *gv = (const TIn *)a.v, *gb = (const TIn *)a.beta;
    constexpr size_t SD = (size_t)DK * DV;
    const float *Sin = a.s_chunks + ((size_t)bh * a.n_chunks + c) * SD;
    const float *Dout = a.d_chunks + ((size_t)bh * a.n_chunks + c) * SD;
    // token rows of head h from the chunk start to the sequence end
    const long long lim = (T - c0) * H - h;
    const size_t bk = (size_t)(row0 + c0 * H) * DK, bv = (size_t)(row0 + c0 * H) * DV;
    constexpr long long ESZ = sizeof(TIn);
    const unsigned HK = (unsigned)(H * DK), HV = (unsigned)(H * DV);
    const bool rwave = wave < NRB;
    const int r = 16 * wave + lc;
    const rsrc_t Rq = make_rsrc(gq + bk, lim * DK * ESZ), Rk = make_rsrc(gk + bk, lim * DK * ESZ);
    const rsrc_t Rg = make_rsrc(gg + bk, lim * DK * ESZ), Rt = make_rsrc(gt + bk, lim * DK * ESZ);
    auto gate = [&](const rsrc_t &R, int t, int i) { return ld_tok<TIn>(R, (16 * t + 4 * lg + i) * HK + r); };

    // ---- phase A: gates of this wave's dk block, Qt and Kt into LDS (split);
    //      then A^T[s][u] = sum_r Kt[s][r] Qt[u][r] by token tiles, over Qt
    constexpr bool kStageGates = !std::is_same<TIn, float>::value;
    const rsrc_t Rgates[4] = {Rq, Rk, Rg, Rt};
    GateStage<DK, C, NT> gs;                // kept in registers for phase C
    if constexpr (kStageGates) {
        gs.load(Rgates, HK, tid);
        gs.store((__bf16 *)(smem + L::o_gsa), tid);
        __syncthreads();
    }
    float d_[NU][4];                       // b - b_m (log2 units) at (token, r)
    float ebm = 0.f, fl = 0.f, ebl = 0.f;
    if (rwave) {
        float q_[NU][4], k_[NU][4], g_[NU][4], t_[NU][4];
        if constexpr (kStageGates) {
            read_gates<DK, C>((const __bf16 *)(smem + L::o_gsa), wave, lc, lg, q_, k_, g_, t_);
        } else {
#pragma unroll
            for (int t = 0; t < NU; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    q_[t][i] = gate(Rq, t, i); k_[t][i] = gate(Rk, t, i);
                    g_[t][i] = gate(Rg, t, i); t_[t][i] = gate(Rt, t, i);
                }
        }
        // b = inclusive cumulative sum of -g tau (log2 units): within the
        // lane's 4 tokens, across the 4 lane groups, then across token tiles
        float run = 0.f;
#pragma unroll
        for (int t = 0; t < NU; ++t) {
            float p[4], s = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) { s = __builtin_fmaf(g_[t][i], t_[t][i], s); p[i] = s; }
            float incl = s, y;
            y = __shfl_up(incl, 16); if (lg >= 1) incl += y;
            y = __shfl_up(incl, 32); if (lg >= 2) incl += y;
            const float excl = incl - s, tot = __shfl(incl, 48 + lc);
#pragma unroll
            for (int i = 0; i < 4; ++i) d_[t][i] = -kLog2e * (run + excl + p[i]);
            run += tot;
        }
        // reference token C/2 - 1: lane group 3, i = 3 of its tile
        const float bm = __shfl(d_[(C / 2 - 1) / 16][3], 48 + lc);
        const float bL = -kLog2e * run;
#pragma unroll
        for (int t = 0; t < NU; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int u = 16 * t + 4 * lg + i;
                d_[t][i] -= bm;
                u16 tq[NS], tk[NS];
                split1<NS>(q_[t][i] * __builtin_amdgcn_exp2f(d_[t][i]), tq);
                split1<NS>(gate_pow(g_[t][i], t_[t][i]) * k_[t][i] * __builtin_amdgcn_exp2f(-d_[t][i]), tk);
#pragma unroll
                for (int n = 0; n < NS; ++n) {
                    sQt[n * LK + u * PK + r] = tq[n];
                    sKt[n * LK + u * PK + r] = tk[n];
                }
            }
        ebm = __builtin_amdgcn_exp2f(bm);
        fl = __builtin_amdgcn_exp2f(bL - bm);
        ebl = __builtin_amdgcn_exp2f(bL);
        if (lg == 0) sF[r] = fl;
    }
    __syncthreads();
    {
        f32x4 at[NU];
        const int st = wave;
        if (st < NU) {
#pragma unroll
            for (int ut = 0; ut < NU; ++ut) at[ut] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k0 = 0; k0 < DK; k0 += 32) {
                bf16x8 A[NS];
                sop_rows<NS, DK>(sKt, LK, PK, 16 * st + lc, k0, lg, A);
#pragma unroll
                for (int ut = 0; ut < NU; ++ut)
                    if (ut >= st) {
                        bf16x8 Bv[NS];
                        sop_rows<NS, DK>(sQt, LK, PK, 16 * ut + lc, k0, lg, Bv);
                        at[ut] = mma_split<NS>(A, Bv, at[ut]);
                    }
            }
        }
        __syncthreads();                   // Qt no longer read
        // A^T (causal: u >= s) over Qt; the tile left of an odd diagonal tile
        // is read by the 32-deep steps and is zero
        if (st < NU) {
#pragma unroll
            for (int ut = 0; ut < NU; ++ut)
                if (ut >= st || ut + 1 == st)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int s_ = 16 * st + 4 * lg + i, u = 16 * ut + lc;
                        u16 ta[NS];
                        split1<NS>(ut >= st && u >= s_ ? at[ut][i] : 0.f, ta);
#pragma unroll
                        for (int n = 0; n < NS; ++n) sAt[n * LC + s_ * PC + u] = ta[n];
                    }
        }
    }

    // ---- phase B, one dv slab at a time: dA^T += V' dO^T (token tiles),
    //      dQt += e^{b_m} dO S_in^T and dKt += f V' D^T (dk blocks), and the
    //      slab's dV' = A^T dO + Kt diag(f) D, dv, dbeta_hat (dv tiles)
    f32x4 dat[NU], dqt[NU], dkt[NU];
    float sd = 0.f;                        // sum_j S_in[r][j] D[r][j]
#pragma unroll
    for (int t = 0; t < NU; ++t) {
        dat[t] = f32x4{0.f, 0.f, 0.f, 0.f}; dqt[t] = dat[t]; dkt[t] = dat[t];
    }
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl) {
        const int j0 = sl * JS;
        // dO and V' = beta_hat v of the slab into LDS, split (16-byte pieces)
        {
            const rsrc_t Rd = make_rsrc(a.dout + bv, lim * DV * 4);
            const rsrc_t Rv = make_rsrc(gv + bv, lim * DV * ESZ);
            const rsrc_t Rb = make_rsrc(gb + bv, lim * DV * ESZ);
            constexpr int NPD = C * JS / 4, LPD = (NPD + NT - 1) / NT;
            typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
            constexpr int EPV = 16 / (int)sizeof(TIn);
            constexpr int NPV = C * JS / EPV, LPV = (NPV + NT - 1) / NT;
            u32x4v xd[LPD], xv[LPV], xb[LPV];
#pragma unroll
            for (int m = 0; m < LPD; ++m) {
                const int p = tid + m * NT, u = p / (JS / 4), j = (p % (JS / 4)) * 4;
                xd[m] = __builtin_amdgcn_raw_buffer_load_b128(Rd, p < NPD ? (u * HV + j0 + j) * 4u : 0x80000000u, 0, 0);
            }
#pragma unroll
            for (int m = 0; m < LPV; ++m) {
                const int p = tid + m * NT, u = p / (JS / EPV), j = (p % (JS / EPV)) * EPV;
                const unsigned o = p < NPV ? (u * HV + j0 + j) * (unsigned)ESZ : 0x80000000u;
                xv[m] = __builtin_amdgcn_raw_buffer_load_b128(Rv, o, 0, 0);
                xb[m] = __builtin_amdgcn_raw_buffer_load_b128(Rb, o, 0, 0);
            }
#pragma unroll
            for (int m = 0; m < LPD; ++m) {
                const int p = tid + m * NT, u = p / (JS / 4), j = (p % (JS / 4)) * 4;
                if (p < NPD) {
                    unsigned w0[NS], w1[NS];
                    chunk_detail::split_pair<NS>(__uint_as_float(xd[m][0]), __uint_as_float(xd[m][1]), w0);
                    chunk_detail::split_pair<NS>(__uint_as_float(xd[m][2]), __uint_as_float(xd[m][3]), w1);
#pragma unroll
                    for (int n = 0; n < NS; ++n) *(uint2 *)(sdO + n * LS + u * PS + j) = uint2{w0[n], w1[n]};
                }
            }
#pragma unroll
            for (int m = 0; m < LPV; ++m) {
                const int p = tid + m * NT, u = p / (JS / EPV), j = (p % (JS / EPV)) * EPV;
                if (p < NPV) {
                    unsigned w[EPV / 2][NS];
#pragma unroll
                    for (int q2 = 0; q2 < EPV / 2; ++q2) {
                        float x0, x1;
                        if constexpr (EPV == 8) {
                            x0 = __uint_as_float(xv[m][q2] << 16) * __uint_as_float(xb[m][q2] << 16);
                            x1 = __uint_as_float(xv[m][q2] & 0xffff0000u) * __uint_as_float(xb[m][q2] & 0xffff0000u);
                        } else {
                            x0 = __uint_as_float(xv[m][2 * q2]) * __uint_as_float(xb[m][2 * q2]);
                            x1 = __uint_as_float(xv[m][2 * q2 + 1]) * __uint_as_float(xb[m][2 * q2 + 1]);
                        }
                        chunk_detail::split_pair<NS>(x0, x1, w[q2]);
                    }
#pragma unroll
                    for (int n = 0; n < NS; ++n) {
                        if constexpr (EPV == 8)
                            *(uint4 *)(sVp + n * LS + u * PS + j) = uint4{w[0][n], w[1][n], w[2][n], w[3][n]};
                        else
                            *(uint2 *)(sVp + n * LS + u * PS + j) = uint2{w[0][n], w[1][n]};
                    }
                }
            }
        }
        __syncthreads();
        // dA^T[s][u] += sum_j V'[s][j] dO[u][j], s tile of this wave, u tiles >= it
        if (wave < NU) {
            const int st = wave;
#pragma unroll
            for (int k0 = 0; k0 < JS; k0 += 32) {
                bf16x8 A[NS];
                sop_rows<NS, JS>(sVp, LS, PS, 16 * st + lc, k0, lg, A);
#pragma unroll
                for (int ut = 0; ut < NU; ++ut)
                    if (ut >= st) {
                        bf16x8 Bv[NS];
                        sop_rows<NS, JS>(sdO, LS, PS, 16 * ut + lc, k0, lg, Bv);
                        dat[ut] = mma_split<NS>(A, Bv, dat[ut]);
                    }
            }
        }
        // state terms of the dk block (B operands: S_in and D rows r of the slab)
        if (rwave) {
#pragma unroll
            for (int ks = 0; ks < KSS; ++ks) {
                float s_[8], d[8];
                op_rows<JS>(Sin, DV, r, j0 + 32 * ks, lg, s_);
                op_rows<JS>(Dout, DV, r, j0 + 32 * ks, lg, d);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    sd = __builtin_fmaf(s_[e], d[e], sd);
                    s_[e] *= ebm;
                    d[e] *= fl;
                }
                bf16x8 Bs[NS], Bd[NS];
                split8<NS>(s_, Bs);
                split8<NS>(d, Bd);
#pragma unroll
                for (int t = 0; t < NU; ++t) {
                    bf16x8 A[NS];
                    sop_rows<NS, JS>(sdO, LS, PS, 16 * t + lc, 32 * ks, lg, A);
                    dqt[t] = mma_split<NS>(A, Bs, dqt[t]);
                    sop_rows<NS, JS>(sVp, LS, PS, 16 * t + lc, 32 * ks, lg, A);
                    dkt[t] = mma_split<NS>(A, Bd, dkt[t]);
                }
            }
        }
        // v and beta_hat for dv = beta_hat dV' and dbeta_hat = v dV', read along
        // rows 4 elements a lane for the row-store pass below (issued here so
        // their latency passes under the dV' products)
        constexpr int PRV = JS / 4, NPR = C * PRV, LPR = (NPR + NT - 1) / NT;
        typedef typename std::conditional<std::is_same<TIn, float>::value, chunk_detail::u32x4,
                                          unsigned __attribute__((ext_vector_type(2)))>::type Raw4;
        Raw4 v4[LPR], b4[LPR];
        {
            const rsrc_t Rv = make_rsrc(gv + bv, lim * DV * ESZ), Rb = make_rsrc(gb + bv, lim * DV * ESZ);
#pragma unroll
            for (int m = 0; m < LPR; ++m) {
                const int p = tid + m * NT, u = p / PRV, j = (p % PRV) * 4;
                const unsigned o = p < NPR ? (u * HV + j0 + j) * (unsigned)ESZ : 0x80000000u;
                if constexpr (std::is_same<TIn, float>::value) {
                    v4[m] = __builtin_amdgcn_raw_buffer_load_b128(Rv, o, 0, 0);
                    b4[m] = __builtin_amdgcn_raw_buffer_load_b128(Rb, o, 0, 0);
                } else {
                    v4[m] = __builtin_amdgcn_raw_buffer_load_b64(Rv, o, 0, 0);
                    b4[m] = __builtin_amdgcn_raw_buffer_load_b64(Rb, o, 0, 0);
                }
            }
        }
        // dV' of this wave's dv tile of the slab
        f32x4 dvp[NU];
        const int jt = wave;                           // tile within the slab
        const int jg = j0 + 16 * jt + lc;              // this lane's dv column
        if (jt < NJS) {
#pragma unroll
            for (int t = 0; t < NU; ++t) dvp[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KSC; ++ks) {
                bf16x8 Bv[NS];
                sop_cols<NS, C>(sdO, LS, PS, 16 * jt + lc, 32 * ks, lg, Bv);
#pragma unroll
                for (int t = 0; t < NU; ++t)
                    if (2 * ks + 1 >= t) {
                        bf16x8 A[NS];
                        sop_rows<NS, C>(sAt, LC, PC, 16 * t + lc, 32 * ks, lg, A);
                        dvp[t] = mma_split<NS>(A, Bv, dvp[t]);
                    }
            }
#pragma unroll
            for (int ks = 0; ks < KSK; ++ks) {
                float y[8];
                bf16x8 Bv[NS];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int kk = 32 * ks + kslot(lg, e);
                    y[e] = kk < DK ? Dout[(size_t)kk * DV + jg] * sF[kk] : 0.f;
                }
                split8<NS>(y, Bv);
#pragma unroll
                for (int t = 0; t < NU; ++t) {
                    bf16x8 A[NS];
                    sop_rows<NS, DK>(sKt, LK, PK, 16 * t + lc, 32 * ks, lg, A);
                    dvp[t] = mma_split<NS>(A, Bv, dvp[t]);
                }
            }
        }
        __syncthreads();                   // the slab's dO and V' no longer read
        if (jt < NJS)
#pragma unroll
            for (int t = 0; t < NU; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) sOutV[(16 * t + 4 * lg + i) * OS + 16 * jt + lc] = dvp[t][i];
        __syncthreads();
        {
            const rsrc_t Rdv = make_rsrc(a.dv + bv, lim * DV * 4), Rdb = make_rsrc(a.dbeta + bv, lim * DV * 4);
#pragma unroll
            for (int m = 0; m < LPR; ++m) {
                const int p = tid + m * NT;
                if (p < NPR) {
                    const int u = p / PRV, j = (p % PRV) * 4;
                    const f32x4 x = *(const f32x4 *)(sOutV + u * OS + j);
                    f32x4 dvo, dbo;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        float ve, be;
                        if constexpr (std::is_same<TIn, float>::value) {
                            ve = __uint_as_float(v4[m][e]);
                            be = __uint_as_float(b4[m][e]);
                        } else {
                            ve = __uint_as_float((e & 1) ? (v4[m][e >> 1] & 0xffff0000u) : (v4[m][e >> 1] << 16));
                            be = __uint_as_float((e & 1) ? (b4[m][e >> 1] & 0xffff0000u) : (b4[m][e >> 1] << 16));
                        }
                        dvo[e] = be * x[e];
                        dbo[e] = ve * x[e];
                    }
                    const unsigned o = (u * HV + j0 + j) * 4u;
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(chunk_detail::u32x4, dvo), Rdv, o, 0, 2);
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(chunk_detail::u32x4, dbo), Rdb, o, 0, 2);
                }
            }
        }
        __syncthreads();                   // staging read before the next slab's planes
    }

    // ---- phase C: dA^T into LDS (over dO), then dQt += dA Kt (s <= u) and
    //      dKt += dA^T Qt (u >= s) with Kt and Qt of the dk block as B operands
    //      (gates again: bf16 from the words loaded in phase A, still in
    //      registers, through LDS over the block's Kt and Qt planes, which are
    //      free by now; fp32 read again directly, from L2)
    GateStage<DK, C, NT> &gsc = gs;         // the words loaded in phase A
    if (wave < NU) {
        const int st = wave;
#pragma unroll
        for (int ut = 0; ut < NU; ++ut)
            if (ut >= st || ut + 1 == st)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int s_ = 16 * st + 4 * lg + i, u = 16 * ut + lc;
                    u16 td[NS];
                    split1<NS>(ut >= st && u >= s_ ? dat[ut][i] : 0.f, td);
#pragma unroll
                    for (int n = 0; n < NS; ++n) sdAt[n * LC + s_ * PC + u] = td[n];
                }
    }
    float q_[NU][4], k_[NU][4], g_[NU][4], t_[NU][4], ah_[NU][4];
    float rs = 0.f;
    if constexpr (kStageGates) {
        gsc.store((__bf16 *)(smem + L::o_gsc), tid);
        __syncthreads();
    }
    if (rwave) {
        if constexpr (kStageGates) {
            read_gates<DK, C>((const __bf16 *)(smem + L::o_gsc), wave, lc, lg, q_, k_, g_, t_);
        } else {
#pragma unroll
            for (int t = 0; t < NU; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    q_[t][i] = gate(Rq, t, i); k_[t][i] = gate(Rk, t, i);
                    g_[t][i] = gate(Rg, t, i); t_[t][i] = gate(Rt, t, i);
                }
        }
        // rowsum(S_o * D)_r = e^{b_L} sum_j S_in[r][j] D[r][j] + sum_s Kt[s][r] (f V' D^T)[s][r]
        // (S_o = diag(e^{b_L}) S_in + diag(f) Kt^T V'; dKt holds only its state term here)
        rs = ebl * sd;
#pragma unroll
        for (int t = 0; t < NU; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                ah_[t][i] = gate_pow(g_[t][i], t_[t][i]);
                rs = __builtin_fmaf(ah_[t][i] * k_[t][i] * __builtin_amdgcn_exp2f(-d_[t][i]), dkt[t][i], rs);
            }
        rs += __shfl_xor(rs, 16);
        rs += __shfl_xor(rs, 32);
    }
    if constexpr (!kStageGates) __syncthreads();       // dA^T planes complete (else above)
    if (rwave) {
#pragma unroll
        for (int ks = 0; ks < KSC; ++ks) {
            float kx[8], qx[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int t = 2 * ks + (e >> 2), i = e & 3;
                kx[e] = ah_[t][i] * k_[t][i] * __builtin_amdgcn_exp2f(-d_[t][i]);
                qx[e] = q_[t][i] * __builtin_amdgcn_exp2f(d_[t][i]);
            }
            bf16x8 BK[NS], BQ[NS];
            split8<NS>(kx, BK);
            split8<NS>(qx, BQ);
#pragma unroll
            for (int t = 0; t < NU; ++t) {
                bf16x8 A[NS];
                if (2 * ks <= t) {                         // dA[u][s] = dA^T[s][u], u in tile t
                    sop_cols<NS, C>(sdAt, LC, PC, 16 * t + lc, 32 * ks, lg, A);
                    dqt[t] = mma_split<NS>(A, BK, dqt[t]);
                }
                if (2 * ks + 1 >= t) {                     // dA^T rows s in tile t
                    sop_rows<NS, C>(sdAt, LC, PC, 16 * t + lc, 32 * ks, lg, A);
                    dkt[t] = mma_split<NS>(A, BQ, dkt[t]);
                }
            }
        }
    }
    __syncthreads();                       // the LDS now stages dq, dk, dg, dtau

    // ---- elementwise tail of the dk block: dq, dk, then dlambda as a suffix
    //      sum over the chunk's tokens (+ rowsum(S_o D)), dg and dtau
    if (rwave) {
        float carry = rs;
#pragma unroll
        for (int t = NU - 1; t >= 0; --t) {
            float x[4], dah[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int u = 16 * t + 4 * lg + i;
                const float dqv = __builtin_amdgcn_exp2f(d_[t][i]) * dqt[t][i];
                const float dkp = __builtin_amdgcn_exp2f(-d_[t][i]) * dkt[t][i];     // dL/dk'
                x[i] = q_[t][i] * dqv - ah_[t][i] * k_[t][i] * dkp;
                dah[i] = k_[t][i] * dkp;                                        // dL/d(g^tau)
                sOutK[(0 * C + u) * OK + r] = dqv;
                sOutK[(1 * C + u) * OK + r] = ah_[t][i] * dkp;
            }
            float sfx[4];
            sfx[3] = x[3];
#pragma unroll
            for (int i = 2; i >= 0; --i) sfx[i] = x[i] + sfx[i + 1];
            float incl = sfx[0], y;
            y = __shfl_down(incl, 16); if (lg <= 2) incl += y;
            y = __shfl_down(incl, 32); if (lg <= 1) incl += y;
            const float excl = incl - sfx[0], tot = __shfl(incl, lc);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int u = 16 * t + 4 * lg + i;
                const float dl = carry + excl + sfx[i];
                const float gv_ = g_[t][i], tv = t_[t][i];
                float dgv = -tv * dl, dtv = -gv_ * dl;
                if (gv_ > 0.f) {
                    dgv += tv * ah_[t][i] * __builtin_amdgcn_rcpf(gv_) * dah[i];
                    dtv += ah_[t][i] * (__builtin_amdgcn_logf(gv_) * (1.f / kLog2e)) * dah[i];
                }
                sOutK[(2 * C + u) * OK + r] = dgv;
                sOutK[(3 * C + u) * OK + r] = dtv;
            }
            carry += tot;
        }
    }
    __syncthreads();
    // whole rows to HBM (16-byte non-temporal stores; rows past T dropped by the range)
    {
        constexpr int PR = DK / 4, NP = 4 * C * PR, LP = (NP + NT - 1) / NT;
#pragma unroll
        for (int m = 0; m < LP; ++m) {
            const int p = tid + m * NT;
            if (p < NP) {
                const int o = p / (C * PR), u = (p / PR) % C, j = (p % PR) * 4;
                float *d = o == 0 ? a.dq : o == 1 ? a.dk : o == 2 ? a.dg : a.dtau;    // wave-uniform
                const rsrc_t R = make_rsrc(d + bk, lim * DK * 4);
                const chunk_detail::u32x4 x = *(const chunk_detail::u32x4 *)(sOutK + (o * C + u) * OK + j);
                __builtin_amdgcn_raw_buffer_store_b128(x, R, (u * HK + j) * 4u, 0, 2);
            }
        }
    }
}

template <int DK, int DV, typename TIn>
hipError_t launch_typed(const ChunkBwdLaunch &Lc, hipStream_t stream)
{
    typedef GradCfg<DK, DV, std::is_same<TIn, float>::value ? 3 : 2> L;
    constexpr int C = L::C;
    const int n_chunks = (Lc.T + C - 1) / C, BH = Lc.B * Lc.H;
    constexpr int NS = std::is_same<TIn, float>::value ? 3 : 2;
    constexpr int JT = SweepTile<DK, DV, NS>::JT;     // one workgroup per (b, h, JT columns) and direction
    typedef SweepCfg<DK, JT, NS> SL;
    constexpr size_t sweep_lds = SL::bytes;
    static std::atomic<bool> sweep_lds_set[kMaxDevices];
    hipError_t e0 = set_lds_limit_once((const void *)state_sweeps_kernel<DK, JT, TIn>, sweep_lds,
                                       sweep_lds_set);
    if (e0 != hipSuccess) return e0;
    SweepArgs sa;
    sa.T = Lc.T; sa.H = Lc.H; sa.dv = DV; sa.n_chunks = n_chunks;
    sa.q = Lc.in.q; sa.k = Lc.in.k; sa.g = Lc.in.g; sa.tau = Lc.in.tau; sa.v = Lc.in.v; sa.beta = Lc.in.beta;
    sa.s0 = Lc.s0; sa.dout = Lc.dout; sa.dsf = Lc.dsf;
    sa.s_chunks = Lc.s_chunks; sa.s_final = Lc.s_final; sa.d_chunks = Lc.d_chunks; sa.ds0 = Lc.ds0;
    hipLaunchKernelGGL((state_sweeps_kernel<DK, JT, TIn>), dim3(BH, DV / JT, 2), dim3(SL::NT),
                       sweep_lds, stream, sa);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;

    static std::atomic<bool> grad_lds_set[kMaxDevices];
    e = set_lds_limit_once((const void *)chunk_grad_kernel<DK, DV, TIn>, L::bytes, grad_lds_set);
    if (e != hipSuccess) return e;
    GradArgs ga;
    ga.T = Lc.T; ga.H = Lc.H; ga.n_chunks = n_chunks; ga.n_work = BH * n_chunks;
    ga.q = Lc.in.q; ga.k = Lc.in.k; ga.g = Lc.in.g; ga.tau = Lc.in.tau; ga.v = Lc.in.v;
    ga.beta = Lc.in.beta; ga.dout = Lc.dout;
    ga.s_chunks = Lc.s_chunks; ga.d_chunks = Lc.d_chunks;
    ga.dq = Lc.dq; ga.dk = Lc.dk_; ga.dg = Lc.dg; ga.dtau = Lc.dtau; ga.dv = Lc.dv_; ga.dbeta = Lc.dbeta;
    const int grid = 8 * ((ga.n_work + 7) / 8);
    hipLaunchKernelGGL((chunk_grad_kernel<DK, DV, TIn>), dim3(grid), dim3(L::NT), L::bytes, stream, ga);
    return hipGetLastError();
}

}  // namespace bwd_detail

#define RODIMUS_BWD_SHAPES(X)                                                            \
    X(16, 16) X(16, 32) X(16, 64) X(16, 128) X(32, 16) X(32, 32) X(32, 64) X(32, 128)    \
    X(64, 16) X(64, 32) X(64, 64) X(64, 128) X(128, 16) X(128, 32) X(128, 64) X(128, 128)

size_t chunk_bwd_lds_bytes(int dk, int dv, bool f32_inputs)
{
#define RODIMUS_BWD_LDS(XK, XV)                                                                  \
    if (dk == XK && dv == XV)                                                                     \
        return f32_inputs ? bwd_detail::GradCfg<XK, XV, 3>::bytes : bwd_detail::GradCfg<XK, XV, 2>::bytes;
    RODIMUS_BWD_SHAPES(RODIMUS_BWD_LDS)
#undef RODIMUS_BWD_LDS
    return 0;
}

int chunk_bwd_chunk(int dk) { return dk == 128 ? 32 : 64; }

hipError_t launch_chunk_bwd(const ChunkBwdLaunch &Lc, hipStream_t stream)
{
#define RODIMUS_BWD_CASE(XK, XV)                                                          \
    if (Lc.dk == XK && Lc.dv == XV)                                                       \
        return Lc.f32_inputs ? bwd_detail::launch_typed<XK, XV, float>(Lc, stream)        \
                             : bwd_detail::launch_typed<XK, XV, __bf16>(Lc, stream);
    RODIMUS_BWD_SHAPES(RODIMUS_BWD_CASE)
#undef RODIMUS_BWD_CASE
    return hipErrorInvalidValue;
}

}  // namespace rodimus
