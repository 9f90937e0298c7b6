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
//   dL/dS_in = diag(e^{b_L}) D + diag(e^{b_m}) Qt^T dO     (carried to the previous chunk)
//   dq = e^{b - b_m} dQt,  dk' = e^{b_m - b} dKt,  dk = g^tau dk',  d(g^tau) = k dk',
//   dv = beta_hat dV',  dbeta_hat = v dV'
//   dlambda_r = sum_{u >= r} (q_u dq_u - k'_u dk'_u) + rowsum(S_o * D)   (per dk column;
//               the sum runs over the chunk's tokens u >= r)
//   dg = -tau dlambda + tau g^(tau-1) d(g^tau),  dtau = -g dlambda + ln(g) g^tau d(g^tau)
// (the g^tau terms taken as 0 at g = 0).  The last identity replaces the per-token
// state products of a token-level backward: every output and the chunk-end state
// depend on lambda_r only through e^{b_u - b_s} with s < r <= u and through e^{b_u},
// e^{b_L}, which is what the two sums count.
//
// The chunk-start states come from a state-only sweep of the forward chunk
// kernel at the same 16-token chunk length (in the workspace); this kernel then
// runs the backward sweep, one workgroup of 8 waves per (b, h), with the state
// adjoint D (dk x dv fp32) in LDS.  Every product is a 16x16-tile MFMA
// (v_mfma_f32_16x16x32_bf16, or v_mfma_f32_16x16x16_bf16 where the contraction
// runs over the chunk's 16 tokens; fp32 accumulate) whose fp32 LDS operands are
// split into NS bf16 terms as they are read (NS = 2 for bf16 inputs, 3 for fp32),
// as in the forward.  The next chunk's inputs and state are loaded into
// registers (16-byte loads) while the current one is processed.  Tail tokens
// read as zero (inert) and their gradients are not stored.
#include "chunk_kernel.h"

namespace rodimus {
namespace bwd_detail {

using chunk_detail::bf16x8;
using chunk_detail::f32x4;
using chunk_detail::kLog2e;

constexpr int kC = 16;                 // tokens per chunk
constexpr int kThreads = 512;          // 8 waves
constexpr int kWaves = kThreads / 64;

struct BwdArgs {
    int T, H, n_chunks;
    const void *q, *k, *g, *tau, *v, *beta;
    const float *dout, *dsf;
    const float *s_chunks;             // [B*H][n_chunks][DK][DV] chunk-start states
    const float *s_final;              // [B*H][DK][DV]
    float *dq, *dk, *dg, *dtau, *dv, *dbeta, *ds0;
};

// LDS layout in floats; rows padded by one float so row- and column-wise
// operand reads both spread over the banks.
template <int DK, int DV>
struct Cfg {
    static constexpr int C = kC;
    static constexpr int SK = DK + 1, SV = DV + 1, SC = C + 1;
    // [C][SK] arrays: q, k, g, tau, Qt, Kt, e^{b-b_m}, e^{b_m-b}, g^tau, q dq, k' dk', d(g^tau)
    static constexpr int o_q = 0, o_k = o_q + C * SK, o_g = o_k + C * SK, o_t = o_g + C * SK;
    static constexpr int o_qt = o_t + C * SK, o_kt = o_qt + C * SK, o_eb = o_kt + C * SK;
    static constexpr int o_ei = o_eb + C * SK, o_ah = o_ei + C * SK;
    static constexpr int o_xq = o_ah + C * SK, o_xk = o_xq + C * SK, o_ya = o_xk + C * SK;
    // [C][SV] arrays: v, beta_hat, V', dO
    static constexpr int o_v = o_ya + C * SK, o_b = o_v + C * SV, o_vp = o_b + C * SV;
    static constexpr int o_do = o_vp + C * SV;
    static constexpr int o_a = o_do + C * SV, o_da = o_a + C * SC;
    static constexpr int o_s = o_da + C * SC, o_d = o_s + DK * SV;
    static constexpr int o_bm = o_d + DK * SV, o_fl = o_bm + DK, o_el = o_fl + DK, o_rs = o_el + DK;
    static constexpr int floats = o_rs + DK;
    static constexpr size_t bytes = (size_t)floats * 4;
};

__device__ __forceinline__ float ld_in(const __bf16 *p, size_t i) { return (float)p[i]; }
__device__ __forceinline__ float ld_in(const float *p, size_t i) { return p[i]; }

// g^tau with pow semantics at g = 0, and its two partial derivatives' factors:
// d(g^tau)/dg = tau g^(tau-1) = tau ah / g,  d(g^tau)/dtau = ah ln g (0 at g = 0).
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

// acc (16 x 16 tile, MFMA C-layout: row 4*(lane/16) + r, column lane % 16) +=
// sum over k < K of A(r, k) B(k, c), with A(r, k) = pa[r*sar + k*sak] (times
// ka[k] when ka is given) and B(k, c) = pb[k*sbk + c*sbc], fp32 LDS operands.
// k-slots of a 32-deep step: lane group g takes k = 4g..4g+3 and 16+4g..16+4g+3
// for both operands.
template <int NS>
__device__ __forceinline__ f32x4 tile_mm(f32x4 acc, const float *pa, int sar, int sak,
                                         const float *ka, const float *pb, int sbk, int sbc,
                                         int K, int lane) {
    const int rc = lane & 15, g = lane >> 4;
    for (int k0 = 0; k0 < K; k0 += 32) {
        float av[8], bv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int kk = k0 + (e < 4 ? 4 * g + e : 12 + 4 * g + e);
            const bool ok = kk < K;
            const float s = (ka && ok) ? ka[kk] : 1.f;
            av[e] = ok ? pa[rc * sar + kk * sak] * s : 0.f;
            bv[e] = ok ? pb[kk * sbk + rc * sbc] : 0.f;
        }
        bf16x8 A[NS], B[NS];
        split8<NS>(av, A);
        split8<NS>(bv, B);
        acc = chunk_detail::mma_split<NS>(A, B, acc);
    }
    return acc;
}

// The same for K = 16 exactly (the chunk length) on v_mfma_f32_16x16x16_bf16:
// lane group g takes k = 4g..4g+3 for both operands.
template <int NS>
__device__ __forceinline__ f32x4 tile_mm16(f32x4 acc, const float *pa, int sar, int sak,
                                           const float *pb, int sbk, int sbc, int lane) {
    typedef short s4 __attribute__((ext_vector_type(4)));
    const int rc = lane & 15, g = lane >> 4;
    float av[4], bv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        av[e] = pa[rc * sar + (4 * g + e) * sak];
        bv[e] = pb[(4 * g + e) * sbk + rc * sbc];
    }
    unsigned wa[2][NS], wb[2][NS];
    chunk_detail::split_pair<NS>(av[0], av[1], wa[0]);
    chunk_detail::split_pair<NS>(av[2], av[3], wa[1]);
    chunk_detail::split_pair<NS>(bv[0], bv[1], wb[0]);
    chunk_detail::split_pair<NS>(bv[2], bv[3], wb[1]);
    s4 A[NS], B[NS];
#pragma unroll
    for (int n = 0; n < NS; ++n) {
        A[n] = __builtin_bit_cast(s4, uint2{wa[0][n], wa[1][n]});
        B[n] = __builtin_bit_cast(s4, uint2{wb[0][n], wb[1][n]});
    }
    // term products of total order < NS, smallest first
    if constexpr (NS == 3) {
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(A[1], B[1], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(A[0], B[2], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(A[2], B[0], acc, 0, 0, 0);
    }
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(A[0], B[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(A[1], B[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(A[0], B[0], acc, 0, 0, 0);
    return acc;
}

template <int DK, int DV, typename TIn>
__global__ __launch_bounds__(kThreads, 1) void chunk_bwd_kernel(BwdArgs a)
{
    constexpr int NS = std::is_same<TIn, float>::value ? 3 : 2;
    constexpr int C = kC;
    typedef Cfg<DK, DV> L;
    constexpr int SK = L::SK, SV = L::SV, SC = L::SC;
    extern __shared__ __attribute__((aligned(16))) float sm[];
    float *sq = sm + L::o_q, *sk = sm + L::o_k, *sg = sm + L::o_g, *st = sm + L::o_t;
    float *sQt = sm + L::o_qt, *sKt = sm + L::o_kt, *sEb = sm + L::o_eb, *sEi = sm + L::o_ei;
    float *sAh = sm + L::o_ah, *sXq = sm + L::o_xq, *sXk = sm + L::o_xk, *sYa = sm + L::o_ya;
    float *sv = sm + L::o_v, *sb = sm + L::o_b, *sVp = sm + L::o_vp, *sdO = sm + L::o_do;
    float *sA = sm + L::o_a, *sdA = sm + L::o_da, *sS = sm + L::o_s, *sD = sm + L::o_d;
    float *sbm = sm + L::o_bm, *sfl = sm + L::o_fl, *sel = sm + L::o_el, *srs = sm + L::o_rs;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int bh = blockIdx.x;
    const int b = bh / a.H, h = bh % a.H;
    const long long T = a.T, H = a.H;
    const long long head0 = (long long)b * T * H + h;
    const TIn *gq = (const TIn *)a.q, *gk = (const TIn *)a.k, *gg = (const TIn *)a.g;
    const TIn *gt = (const TIn *)a.tau, *gv = (const TIn *)a.v, *gb = (const TIn *)a.beta;
    const float *ws = a.s_chunks + (size_t)bh * a.n_chunks * DK * DV;
    const int lc = lane & 15, lg = lane >> 4;
    auto gidx_k = [&](long long t, int i) { return (size_t)((head0 + t * H) * DK + i); };
    auto gidx_v = [&](long long t, int j) { return (size_t)((head0 + t * H) * DV + j); };

    // one chunk's inputs and chunk-start state, prefetched into registers a
    // chunk ahead with 16-byte loads (tokens past T read as zero): per-token
    // tensors as 16-byte pieces of token rows, the state as float4s
    typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
    constexpr int EPV = 16 / (int)sizeof(TIn);                  // elements per piece
    constexpr int NPK = C * DK / EPV, NPV = C * DV / EPV, NPD = C * DV / 4, NPS = DK * DV / 4;
    constexpr int LK = (NPK + kThreads - 1) / kThreads, LV = (NPV + kThreads - 1) / kThreads;
    constexpr int LD = (NPD + kThreads - 1) / kThreads, LS = (NPS + kThreads - 1) / kThreads;
    u32x4v rq[LK], rk[LK], rg[LK], rt[LK], rv[LV], rb[LV], rd[LD], rs_[LS];
    auto ld16 = [&](const void *base, size_t elem, bool ok, size_t esz) {
        return ok ? *(const u32x4v *)((const char *)base + elem * esz) : u32x4v{0u, 0u, 0u, 0u};
    };
    auto prefetch = [&](int c) {
        const long long t0 = (long long)c * C;
#pragma unroll
        for (int m = 0; m < LK; ++m) {
            const int pidx = tid + m * kThreads, u = pidx / (DK / EPV), i = (pidx % (DK / EPV)) * EPV;
            const bool ok = pidx < NPK && t0 + u < T;
            rq[m] = ld16(gq, gidx_k(t0 + u, i), ok, sizeof(TIn));
            rk[m] = ld16(gk, gidx_k(t0 + u, i), ok, sizeof(TIn));
            rg[m] = ld16(gg, gidx_k(t0 + u, i), ok, sizeof(TIn));
            rt[m] = ld16(gt, gidx_k(t0 + u, i), ok, sizeof(TIn));
        }
#pragma unroll
        for (int m = 0; m < LV; ++m) {
            const int pidx = tid + m * kThreads, u = pidx / (DV / EPV), j = (pidx % (DV / EPV)) * EPV;
            const bool ok = pidx < NPV && t0 + u < T;
            rv[m] = ld16(gv, gidx_v(t0 + u, j), ok, sizeof(TIn));
            rb[m] = ld16(gb, gidx_v(t0 + u, j), ok, sizeof(TIn));
        }
#pragma unroll
        for (int m = 0; m < LD; ++m) {
            const int pidx = tid + m * kThreads, u = pidx / (DV / 4), j = (pidx % (DV / 4)) * 4;
            rd[m] = ld16(a.dout, gidx_v(t0 + u, j), pidx < NPD && t0 + u < T, 4);
        }
#pragma unroll
        for (int m = 0; m < LS; ++m) {
            const int pidx = tid + m * kThreads;
            rs_[m] = ld16(ws, (size_t)c * DK * DV + (size_t)pidx * 4, pidx < NPS, 4);
        }
    };
    // element n of a piece as fp32
    auto elem = [&](const u32x4v &x, int n) -> float {
        if constexpr (EPV == 8)
            return __uint_as_float((n & 1) ? (x[n >> 1] & 0xffff0000u) : (x[n >> 1] << 16));
        else
            return __uint_as_float(x[n]);
    };
    auto stage = [&]() {
#pragma unroll
        for (int m = 0; m < LK; ++m) {
            const int pidx = tid + m * kThreads, u = pidx / (DK / EPV), i = (pidx % (DK / EPV)) * EPV;
            if (pidx < NPK)
#pragma unroll
                for (int n = 0; n < EPV; ++n) {
                    sq[u * SK + i + n] = elem(rq[m], n); sk[u * SK + i + n] = elem(rk[m], n);
                    sg[u * SK + i + n] = elem(rg[m], n); st[u * SK + i + n] = elem(rt[m], n);
                }
        }
#pragma unroll
        for (int m = 0; m < LV; ++m) {
            const int pidx = tid + m * kThreads, u = pidx / (DV / EPV), j = (pidx % (DV / EPV)) * EPV;
            if (pidx < NPV)
#pragma unroll
                for (int n = 0; n < EPV; ++n) {
                    const float vv = elem(rv[m], n), bb = elem(rb[m], n);
                    sv[u * SV + j + n] = vv; sb[u * SV + j + n] = bb; sVp[u * SV + j + n] = vv * bb;
                }
        }
#pragma unroll
        for (int m = 0; m < LD; ++m) {
            const int pidx = tid + m * kThreads, u = pidx / (DV / 4), j = (pidx % (DV / 4)) * 4;
            if (pidx < NPD)
#pragma unroll
                for (int n = 0; n < 4; ++n) sdO[u * SV + j + n] = __uint_as_float(rd[m][n]);
        }
#pragma unroll
        for (int m = 0; m < LS; ++m) {
            const int pidx = tid + m * kThreads, i = (pidx * 4) / DV, j = (pidx * 4) % DV;
            if (pidx < NPS)
#pragma unroll
                for (int n = 0; n < 4; ++n) sS[i * SV + j + n] = __uint_as_float(rs_[m][n]);
        }
    };
    // rowsum(S_o * D) per dk row, S_o and D as they are in LDS
    auto rowsum = [&]() {
        for (int i = tid / 8; i < DK; i += kThreads / 8) {
            float acc = 0.f;
            for (int j = tid % 8; j < DV; j += 8) acc += sS[i * SV + j] * sD[i * SV + j];
            acc += __shfl_xor(acc, 1, 8);
            acc += __shfl_xor(acc, 2, 8);
            acc += __shfl_xor(acc, 4, 8);
            if (tid % 8 == 0) srs[i] = acc;
        }
    };

    // S_T and D = dL/dS_T, and the last chunk's rowsum
    for (int e = tid; e < DK * DV; e += kThreads) {
        const int i = e / DV, j = e % DV;
        sS[i * SV + j] = a.s_final[(size_t)bh * DK * DV + e];
        sD[i * SV + j] = a.dsf ? a.dsf[(size_t)bh * DK * DV + e] : 0.f;
    }
    if (a.n_chunks > 0) prefetch(a.n_chunks - 1);
    __syncthreads();
    rowsum();

    for (int c = a.n_chunks - 1; c >= 0; --c) {
        const long long t0 = (long long)c * C;
        __syncthreads();
        stage();                                   // S_in(c) and the inputs of chunk c
        if (c > 0) prefetch(c - 1);
        __syncthreads();
        // gates: the 16 tokens of a dk column sit on 16 consecutive lanes
        // (element e -> column e / C, token e % C), so the chunk-local
        // cumulative sum of lambda (log2 units) is a 16-lane scan; then
        // e^{b-b_m}, e^{b_m-b}, g^tau, Qt, Kt per element, and e^{b_m},
        // e^{b_L - b_m}, e^{b_L} per column
        for (int e = tid; e < C * DK; e += kThreads) {
            const int i = e / C, u = e % C;
            const float gv_ = sg[u * SK + i], tv = st[u * SK + i];
            float b_ = -kLog2e * gv_ * tv;
#pragma unroll
            for (int o = 1; o < C; o <<= 1) {
                const float y = __shfl_up(b_, o, C);
                if (u >= o) b_ += y;
            }
            const float bm = __shfl(b_, C / 2 - 1, C), bL = __shfl(b_, C - 1, C);
            const float d = b_ - bm;
            const float eb = __builtin_amdgcn_exp2f(d), ei = __builtin_amdgcn_exp2f(-d);
            const float ah = gate_pow(gv_, tv);
            sEb[u * SK + i] = eb;
            sEi[u * SK + i] = ei;
            sAh[u * SK + i] = ah;
            sQt[u * SK + i] = sq[u * SK + i] * eb;
            sKt[u * SK + i] = ah * sk[u * SK + i] * ei;
            if (u == 0) {
                sbm[i] = __builtin_amdgcn_exp2f(bm);
                sfl[i] = __builtin_amdgcn_exp2f(bL - bm);
                sel[i] = __builtin_amdgcn_exp2f(bL);
            }
        }
        __syncthreads();
        // A = tril(Qt Kt^T) and dA = tril(dO V'^T), [u][s]
        if (wave < 2) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            float *dst = wave == 0 ? sA : sdA;
            if (wave == 0) acc = tile_mm<NS>(acc, sQt, SK, 1, nullptr, sKt, 1, SK, DK, lane);
            else acc = tile_mm<NS>(acc, sdO, SV, 1, nullptr, sVp, 1, SV, DV, lane);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int u = 4 * lg + r, s_ = lc;
                dst[u * SC + s_] = s_ <= u ? acc[r] : 0.f;
            }
        }
        __syncthreads();
        // dQt, dKt (C x dk) and dV' (C x dv) tiles
        constexpr int NQ = DK / 16, NV = DV / 16;
        for (int tile = wave; tile < 2 * NQ + NV; tile += kWaves) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            if (tile < NQ) {                       // dQt columns I
                const int I = tile;
                acc = tile_mm<NS>(acc, sdO, SV, 1, nullptr, sS + I * 16 * SV, 1, SV, DV, lane);
                const float sc = sbm[I * 16 + lc];
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[r] *= sc;
                acc = tile_mm16<NS>(acc, sdA, SC, 1, sKt + I * 16, SK, 1, lane);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int u = 4 * lg + r, i = I * 16 + lc;
                    const float dqv = sEb[u * SK + i] * acc[r];
                    sXq[u * SK + i] = sq[u * SK + i] * dqv;
                    if (t0 + u < T) a.dq[gidx_k(t0 + u, i)] = dqv;
                }
            } else if (tile < 2 * NQ) {            // dKt columns I
                const int I = tile - NQ;
                acc = tile_mm<NS>(acc, sVp, SV, 1, nullptr, sD + I * 16 * SV, 1, SV, DV, lane);
                const float sc = sfl[I * 16 + lc];
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[r] *= sc;
                acc = tile_mm16<NS>(acc, sdA, 1, SC, sQt + I * 16, SK, 1, lane);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int u = 4 * lg + r, i = I * 16 + lc;
                    const float ah = sAh[u * SK + i];
                    const float dkp = acc[r] * sEi[u * SK + i];          // dL/dk'
                    sXk[u * SK + i] = ah * sk[u * SK + i] * dkp;
                    sYa[u * SK + i] = sk[u * SK + i] * dkp;             // dL/d(g^tau)
                    if (t0 + u < T) a.dk[gidx_k(t0 + u, i)] = ah * dkp;
                }
            } else {                               // dV' columns J
                const int J = tile - 2 * NQ;
                acc = tile_mm16<NS>(acc, sA, 1, SC, sdO + J * 16, SV, 1, lane);
                acc = tile_mm<NS>(acc, sKt, SK, 1, sfl, sD + J * 16, SV, 1, DK, lane);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int u = 4 * lg + r, j = J * 16 + lc;
                    if (t0 + u < T) {
                        a.dv[gidx_v(t0 + u, j)] = sb[u * SV + j] * acc[r];
                        a.dbeta[gidx_v(t0 + u, j)] = sv[u * SV + j] * acc[r];
                    }
                }
            }
        }
        __syncthreads();
        // dL/dS_in = diag(e^{b_L}) D + diag(e^{b_m}) Qt^T dO, into D
        for (int tile = wave; tile < (DK / 16) * (DV / 16); tile += kWaves) {
            const int I = tile / (DV / 16), J = tile % (DV / 16);
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = tile_mm16<NS>(acc, sQt + I * 16, 1, SK, sdO + J * 16, SV, 1, lane);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = I * 16 + 4 * lg + r, j = J * 16 + lc;
                sD[i * SV + j] = __builtin_fmaf(sbm[i], acc[r], sel[i] * sD[i * SV + j]);
            }
        }
        // meanwhile dlambda = rowsum(S_o D) + reverse cumulative sum over the
        // chunk's tokens of q dq - k' dk' (a 16-lane scan per dk column), then
        // dg, dtau; after the barrier the previous chunk's rowsum (S_o(c-1) =
        // S_in(c) in LDS, D now dL/dS_in(c))
        for (int e = tid; e < C * DK; e += kThreads) {
            const int i = e / C, u = e % C;
            float dl = sXq[u * SK + i] - sXk[u * SK + i];
#pragma unroll
            for (int o = 1; o < C; o <<= 1) {
                const float y = __shfl_down(dl, o, C);
                if (u + o < C) dl += y;
            }
            dl += srs[i];
            if (t0 + u < T) {
                const float gv_ = sg[u * SK + i], tv = st[u * SK + i];
                const float ah = sAh[u * SK + i], dah = sYa[u * SK + i];
                float dgv = -tv * dl, dtv = -gv_ * dl;
                if (gv_ > 0.f) {
                    dgv += tv * ah * __builtin_amdgcn_rcpf(gv_) * dah;
                    dtv += ah * (__builtin_amdgcn_logf(gv_) * (1.f / kLog2e)) * dah;
                }
                a.dg[gidx_k(t0 + u, i)] = dgv;
                a.dtau[gidx_k(t0 + u, i)] = dtv;
            }
        }
        __syncthreads();
        rowsum();
    }
    __syncthreads();
    if (a.ds0)
        for (int e = tid; e < DK * DV; e += kThreads)
            a.ds0[(size_t)bh * DK * DV + e] = sD[(e / DV) * SV + e % DV];
}

template <int DK, int DV, typename TIn>
hipError_t launch_typed(int BH, const BwdArgs &args, hipStream_t stream)
{
    typedef Cfg<DK, DV> L;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void *)chunk_bwd_kernel<DK, DV, TIn>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)L::bytes);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    hipLaunchKernelGGL((chunk_bwd_kernel<DK, DV, TIn>), dim3(BH), dim3(kThreads), L::bytes, stream, args);
    return hipGetLastError();
}

}  // namespace bwd_detail

size_t chunk_bwd_lds_bytes(int dk, int dv)
{
#define RODIMUS_BWD_LDS(XK, XV) if (dk == XK && dv == XV) return bwd_detail::Cfg<XK, XV>::bytes;
    RODIMUS_BWD_LDS(16, 16) RODIMUS_BWD_LDS(16, 32) RODIMUS_BWD_LDS(16, 64) RODIMUS_BWD_LDS(16, 128)
    RODIMUS_BWD_LDS(32, 16) RODIMUS_BWD_LDS(32, 32) RODIMUS_BWD_LDS(32, 64) RODIMUS_BWD_LDS(32, 128)
    RODIMUS_BWD_LDS(64, 16) RODIMUS_BWD_LDS(64, 32) RODIMUS_BWD_LDS(64, 64) RODIMUS_BWD_LDS(64, 128)
    RODIMUS_BWD_LDS(128, 16) RODIMUS_BWD_LDS(128, 32)
#undef RODIMUS_BWD_LDS
    return 0;
}

int chunk_bwd_chunk() { return bwd_detail::kC; }

hipError_t launch_chunk_bwd(const ChunkBwdLaunch &Lc, hipStream_t stream)
{
    bwd_detail::BwdArgs a;
    a.T = Lc.T; a.H = Lc.H; a.n_chunks = (Lc.T + bwd_detail::kC - 1) / bwd_detail::kC;
    a.q = Lc.in.q; a.k = Lc.in.k; a.g = Lc.in.g; a.tau = Lc.in.tau; a.v = Lc.in.v; a.beta = Lc.in.beta;
    a.dout = Lc.dout; a.dsf = Lc.dsf; a.s_chunks = Lc.s_chunks; a.s_final = Lc.s_final;
    a.dq = Lc.dq; a.dk = Lc.dk_; a.dg = Lc.dg; a.dtau = Lc.dtau; a.dv = Lc.dv_; a.dbeta = Lc.dbeta;
    a.ds0 = Lc.ds0;
    const int BH = Lc.B * Lc.H;
#define RODIMUS_BWD_CASE(XK, XV)                                                              \
    if (Lc.dk == XK && Lc.dv == XV)                                                           \
        return Lc.f32_inputs ? bwd_detail::launch_typed<XK, XV, float>(BH, a, stream)         \
                             : bwd_detail::launch_typed<XK, XV, __bf16>(BH, a, stream);
    RODIMUS_BWD_CASE(16, 16) RODIMUS_BWD_CASE(16, 32) RODIMUS_BWD_CASE(16, 64) RODIMUS_BWD_CASE(16, 128)
    RODIMUS_BWD_CASE(32, 16) RODIMUS_BWD_CASE(32, 32) RODIMUS_BWD_CASE(32, 64) RODIMUS_BWD_CASE(32, 128)
    RODIMUS_BWD_CASE(64, 16) RODIMUS_BWD_CASE(64, 32) RODIMUS_BWD_CASE(64, 64) RODIMUS_BWD_CASE(64, 128)
    RODIMUS_BWD_CASE(128, 16) RODIMUS_BWD_CASE(128, 32)
#undef RODIMUS_BWD_CASE
    return hipErrorInvalidValue;
}

}  // namespace rodimus
