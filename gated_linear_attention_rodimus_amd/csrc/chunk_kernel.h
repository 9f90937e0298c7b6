// chunk_kernel.h -- chunkwise-parallel DDTS forward on gfx950 MFMA (kernel
// template; instantiated per dk in chunk_dk*.hip).
//
// Why a chunk form exists: the authors state that DDTS selects only along n
// (the dk rows of the state), which is what makes chunkwise-parallel training
// possible (Rodimus* rebuttal page, paperhub.cn, bullet "Efficient
// Parallelization"; also the answer on sequential processing bottlenecks).
// The pages only name the algorithm (their Section 3.1.3 and Appendix B3 are
// not reproduced), so the chunk form below is derived from the recurrence:
//
// Inside a chunk of L <= C tokens (local index u), with lambda_u = -g_u*tau_u
// and the chunk-local inclusive cumulative sum b_u = sum_{r<=u} lambda_r (per
// column i of dk), the recurrence unrolls exactly into
//   O   = tril(Qt Kt^T) V' + Qt' S_in            (diagonal kept)
//   S_o = diag(exp(b_L)) S_in + Kh^T V'
// with V' = beta_hat*v, k' = g^tau * k and
//   Qt[u,i] = q[u,i] exp(b_u - b_m),  Kt[s,i] = k'[s,i] exp(b_m - b_s),
//   Qt'     = Qt with S_in's rows pre-scaled by exp(b_m),
//   Kh[s,i] = k'[s,i] exp(b_L - b_s).
// b_m is the cumulative sum at the middle of the chunk: referencing the
// exponentials there halves their range (all exponents stay within half a
// chunk's total decay), and Qt Kt^T reproduces exp(b_u - b_s) for s <= u.
//
// Precision: all four products run on bf16 MFMA (v_mfma_f32_16x16x32_bf16)
// with fp32 accumulation.  Every fp32 operand is split into NS bf16 terms
// (x = x0 + x1 [+ x2]) and the product keeps the cross terms of total order
// < NS: 3 MFMAs for bf16 inputs (NS = 2, ~16 mantissa bits per operand) and
// 6 MFMAs for fp32 inputs (NS = 3, ~24 bits).  The state is carried in fp32
// registers across chunks.
//
// Workgroup = 4 waves, owns one (b, h, dv tile of DVT columns, segment).  Per
// chunk:
//  1. prep: every thread owns one column (i of dk, or j of the dv tile) and a
//     run of consecutive tokens; it loads the inputs, forms the local
//     cumulative sum (cross-thread offsets through LDS), the gates and the
//     scaled operands, and writes them to LDS as bf16 planes: Qt and Kt in
//     row form [u][i], Kh^T and V'^T in column form [i][s] / [j][s] (the
//     token dimension is the contraction for the last two products);
//  2. each wave writes bf16 images of its state tiles (rows scaled by
//     exp(b_m)) and computes its share of the 16x16 tiles of A^T = Kt Qt^T
//     (upper triangle incl. diagonal), stored as register images;
//  3. each wave computes dS = Kh^T V' for its state tiles and updates
//     S = diag(exp(b_L)) S + dS in registers;
//  4. each wave computes its output tiles O = A V' + Qt S' and stores fp32.
// The MFMA operand k-slots are assigned so that a C-layout tile (rows 4g..4g+3
// of lane group g) is directly a B operand of the next product: a 32-deep
// k-step takes rows {4g..4g+3} of one 16-row tile and {16+4g..16+4g+3} of the
// next, and the other operand is read from LDS with the same slot mapping.
//
// Inputs for chunk c+1 are loaded into registers while chunk c's MFMA phases
// run.
#pragma once
#include "internal.h"

#include <type_traits>

namespace rodimus {
namespace chunk_detail {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr float kLog2e = 1.4426950408889634f;

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16;

__device__ __forceinline__ float in_to_f32(u16 x) { return __uint_as_float((unsigned)x << 16); }
__device__ __forceinline__ float in_to_f32(float x) { return x; }

template <typename TIn> struct InRaw;
template <> struct InRaw<__bf16> { typedef u16 type; };
template <> struct InRaw<float> { typedef float type; };

// Split x into NS bf16 terms, x ~= p[0] + p[1] (+ p[2]); each residual is exact in fp32.
template <int NS>
__device__ __forceinline__ void split(float x, __bf16 *p) {
    const __bf16 h = (__bf16)x;
    p[0] = h;
    if constexpr (NS > 1) {
        const float r = x - (float)h;
        const __bf16 m = (__bf16)r;
        p[1] = m;
        if constexpr (NS > 2) p[2] = (__bf16)(r - (float)m);
    }
}

__device__ __forceinline__ bf16x8 cat(bf16x4 lo, bf16x4 hi) {
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ bf16x4 zero4() {
    bf16x4 z;
    z[0] = z[1] = z[2] = z[3] = (__bf16)0.f;
    return z;
}

// acc += sum over split-term pairs (a, b) with a + b < NS of A[a] * B[b].
template <int NS>
__device__ __forceinline__ f32x4 mma_split(const bf16x8 *A, const bf16x8 *Bv, f32x4 acc) {
    if constexpr (NS == 3) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[1], Bv[1], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[0], Bv[2], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[2], Bv[0], acc, 0, 0, 0);
    }
    if constexpr (NS >= 2) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[0], Bv[1], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[1], Bv[0], acc, 0, 0, 0);
    }
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[0], Bv[0], acc, 0, 0, 0);
    return acc;
}

struct Args {
    int B, T, H, dv;
    int n_seg, chunks_per_seg, n_chunks, n_jt;
    int mode;                    // 0: outputs, 1: segment transfer
    const void *q, *k, *g, *tau, *v, *beta;
    const float *s_in; long long s_in_bh, s_in_seg;
    float *out;
    float *s_out; long long s_out_bh, s_out_seg; int s_out_last_only;
    float *gam_out;
    int remap;                   // XCD-aware block mapping on/off
};

// LDS layout (bytes), shared by the host-side size query.
template <int DK, int DVT, int C, int NS>
struct Lds {
    static constexpr int NU = C / 16, NI = DK / 16, NJ = DVT / 16;
    static constexpr int NA = NU * (NU + 1) / 2;
    static constexpr int NG = kThreads / DK;          // token groups for dk columns
    static constexpr int RS = DK + 8;                 // row-form stride (bf16)
    static constexpr int CS = C + 8;                  // column-form stride (bf16)
    static constexpr size_t q_off = 0;
    static constexpr size_t k_off = q_off + (size_t)NS * C * RS * 2;
    static constexpr size_t kh_off = k_off + (size_t)NS * C * RS * 2;
    static constexpr size_t v_off = kh_off + (size_t)NS * DK * CS * 2;
    static constexpr size_t a_off = v_off + (size_t)NS * DVT * CS * 2;
    static constexpr size_t s_off = a_off + (size_t)NA * NS * 64 * 4 * 2;
    static constexpr size_t tot_off = s_off + (size_t)NI * NJ * NS * 64 * 4 * 2;
    static constexpr size_t gam_off = tot_off + (size_t)NG * DK * 4;
    static constexpr size_t em_off = gam_off + (size_t)DK * 4;
    static constexpr size_t bytes = em_off + (size_t)DK * 4;
};

template <int DK, int DVT, int C, typename TIn>
__global__ __launch_bounds__(kThreads, 1) void chunk_fwd_kernel(Args a)
{
    constexpr int NS = std::is_same<TIn, float>::value ? 3 : 2;
    typedef Lds<DK, DVT, C, NS> L;
    typedef typename InRaw<TIn>::type Raw;
    constexpr int NU = L::NU, NI = L::NI, NJ = L::NJ, NA = L::NA;
    constexpr int RS = L::RS, CS = L::CS;
    // column-owner layout for the dk tensors and for the dv tile
    constexpr int NG = kThreads / DK, TPG = C / NG;
    constexpr int NGV = kThreads / DVT, TPGV = C / NGV;
    static_assert(TPG >= 1 && TPGV >= 1, "chunk too small for the tile");
    constexpr int SPW = (NI * NJ + kWaves - 1) / kWaves;      // state tiles per wave

    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    __bf16 *sQ = (__bf16 *)(smem + L::q_off);
    __bf16 *sK = (__bf16 *)(smem + L::k_off);
    __bf16 *sKh = (__bf16 *)(smem + L::kh_off);
    __bf16 *sV = (__bf16 *)(smem + L::v_off);
    __bf16 *sA = (__bf16 *)(smem + L::a_off);
    __bf16 *sS = (__bf16 *)(smem + L::s_off);
    float *sTot = (float *)(smem + L::tot_off);
    float *sGam = (float *)(smem + L::gam_off);
    float *sEm = (float *)(smem + L::em_off);

    // ---- block -> (b, h, dv tile, segment); XCD-aware: consecutive logical ids
    // (the dv tiles of one head first) land on the same XCD, which shares L2.
    const int nblk = gridDim.x;
    int id = blockIdx.x;
    if (a.remap) id = (id % 8) * (nblk / 8) + id / 8;
    const int jt = id % a.n_jt;
    const int rest = id / a.n_jt;
    const int seg = rest % a.n_seg;
    const int bh = rest / a.n_seg;
    const int b = bh / a.H, h = bh % a.H;
    const int j0 = jt * DVT;
    const int c_begin = seg * a.chunks_per_seg;
    const int c_end = min(a.n_chunks, c_begin + a.chunks_per_seg);
    const bool outputs = a.mode == 0;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int lc = lane & 15, lg = lane >> 4;          // MFMA lane column / group
    const int ci = tid % DK, cgp = tid / DK;           // dk column owner
    const int cj = tid % DVT, cgv = tid / DVT;         // dv column owner

    const Raw *gq = (const Raw *)a.q, *gk = (const Raw *)a.k, *gg = (const Raw *)a.g;
    const Raw *gt = (const Raw *)a.tau, *gv = (const Raw *)a.v, *gb = (const Raw *)a.beta;

    // ---- state tiles owned by this wave, fp32 C-layout: S[slot][r] holds
    // row I*16 + 4*lg + r, column J*16 + lc of the dv tile.
    float S[SPW][4];
    {
        const float *sin = a.s_in ? a.s_in + bh * a.s_in_bh + seg * a.s_in_seg : nullptr;
#pragma unroll
        for (int slot = 0; slot < SPW; ++slot) {
            const int idx = slot * kWaves + wave;
            const int I = idx / NJ, J = idx % NJ;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float x = 0.f;
                if (idx < NI * NJ && sin)
                    x = sin[(size_t)(I * 16 + 4 * lg + r) * a.dv + j0 + J * 16 + lc];
                S[slot][r] = x;
            }
        }
    }
    float gam_acc = 1.f;                                // product of chunk decays (mode 1)

    // ---- raw input registers for one chunk
    Raw rq[TPG], rk[TPG], rg[TPG], rt[TPG], rv[TPGV], rb[TPGV];
    auto load_chunk = [&](int ch) {
        const int t0 = ch * C;
#pragma unroll
        for (int m = 0; m < TPG; ++m) {
            const int tok = t0 + cgp * TPG + m;
            const bool ok = tok < a.T;
            const size_t idx = (((size_t)b * a.T + (ok ? tok : 0)) * a.H + h) * DK + ci;
            rq[m] = (ok && outputs) ? gq[idx] : Raw(0);
            rk[m] = ok ? gk[idx] : Raw(0);
            rg[m] = ok ? gg[idx] : Raw(0);
            rt[m] = ok ? gt[idx] : Raw(0);
        }
#pragma unroll
        for (int m = 0; m < TPGV; ++m) {
            const int tok = t0 + cgv * TPGV + m;
            const bool ok = tok < a.T;
            const size_t idx = (((size_t)b * a.T + (ok ? tok : 0)) * a.H + h) * a.dv + j0 + cj;
            rv[m] = ok ? gv[idx] : Raw(0);
            rb[m] = ok ? gb[idx] : Raw(0);
        }
    };

    if (c_begin < c_end) load_chunk(c_begin);

    for (int ch = c_begin; ch < c_end; ++ch) {
        const int t0 = ch * C;

        // ================= 1. prep: cumulative decay, gates, operands -> LDS
        float cum[TPG];
        {
            float run = 0.f;
#pragma unroll
            for (int m = 0; m < TPG; ++m) {
                run += -(in_to_f32(rg[m]) * in_to_f32(rt[m]));
                cum[m] = run;
            }
            sTot[cgp * DK + ci] = run;
        }
        __syncthreads();
        float off = 0.f, bm = 0.f, bL = 0.f;
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
            const float x = sTot[gi * DK + ci];
            if (gi < cgp) off += x;
            if (gi < NG / 2) bm += x;
            bL += x;
        }
        {
            __bf16 kh_pl[NS][TPG];
#pragma unroll
            for (int m = 0; m < TPG; ++m) {
                const int u = cgp * TPG + m;
                const float bu = off + cum[m];
                const float gv_ = in_to_f32(rg[m]), tv_ = in_to_f32(rt[m]);
                const float kv_ = in_to_f32(rk[m]);
                // log2 of alpha_hat = tau*log2(g), with pow semantics at g = 0
                const float la = gv_ > 0.f ? tv_ * __builtin_amdgcn_logf(gv_)
                                           : (tv_ == 0.f ? 0.f : -INFINITY);
                __bf16 p[NS];
                if (outputs) {
                    const float qt = in_to_f32(rq[m]) * __builtin_amdgcn_exp2f((bu - bm) * kLog2e);
                    split<NS>(qt, p);
#pragma unroll
                    for (int n = 0; n < NS; ++n) sQ[(n * C + u) * RS + ci] = p[n];
                    const float kt = kv_ * __builtin_amdgcn_exp2f(la + (bm - bu) * kLog2e);
                    split<NS>(kt, p);
#pragma unroll
                    for (int n = 0; n < NS; ++n) sK[(n * C + u) * RS + ci] = p[n];
                }
                const float kh = kv_ * __builtin_amdgcn_exp2f(la + (bL - bu) * kLog2e);
                split<NS>(kh, p);
#pragma unroll
                for (int n = 0; n < NS; ++n) kh_pl[n][m] = p[n];
            }
#pragma unroll
            for (int n = 0; n < NS; ++n) {
                __bf16 *dst = sKh + (n * DK + ci) * CS + cgp * TPG;
#pragma unroll
                for (int m = 0; m < TPG; ++m) dst[m] = kh_pl[n][m];
            }
        }
        if (cgp == 0) {
            sGam[ci] = __builtin_amdgcn_exp2f(bL * kLog2e);
            sEm[ci] = __builtin_amdgcn_exp2f(bm * kLog2e);
        }
        {
            __bf16 v_pl[NS][TPGV];
#pragma unroll
            for (int m = 0; m < TPGV; ++m) {
                __bf16 p[NS];
                split<NS>(in_to_f32(rb[m]) * in_to_f32(rv[m]), p);
#pragma unroll
                for (int n = 0; n < NS; ++n) v_pl[n][m] = p[n];
            }
#pragma unroll
            for (int n = 0; n < NS; ++n) {
                __bf16 *dst = sV + (n * DVT + cj) * CS + cgv * TPGV;
#pragma unroll
                for (int m = 0; m < TPGV; ++m) dst[m] = v_pl[n][m];
            }
        }
        __syncthreads();

        // prefetch the next chunk's inputs while the MFMA phases run
        if (ch + 1 < c_end) load_chunk(ch + 1);

        // ================= 2. state images (rows scaled by exp(b_m)) and A^T tiles
        if (outputs) {
#pragma unroll
            for (int slot = 0; slot < SPW; ++slot) {
                const int idx = slot * kWaves + wave;
                if (idx < NI * NJ) {
                    const int I = idx / NJ;
                    __bf16 pl[NS][4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        __bf16 p[NS];
                        split<NS>(S[slot][r] * sEm[I * 16 + 4 * lg + r], p);
#pragma unroll
                        for (int n = 0; n < NS; ++n) pl[n][r] = p[n];
                    }
#pragma unroll
                    for (int n = 0; n < NS; ++n) {
                        bf16x4 w;
                        w[0] = pl[n][0]; w[1] = pl[n][1]; w[2] = pl[n][2]; w[3] = pl[n][3];
                        *(bf16x4 *)(sS + ((idx * NS + n) * 64 + lane) * 4) = w;
                    }
                }
            }
            // A^T tile (Sb, Ub), Sb <= Ub: rows s of Kt, columns u of Qt, k = i
#pragma unroll
            for (int Ub = 0; Ub < NU; ++Ub) {
#pragma unroll
                for (int Sb = 0; Sb <= Ub; ++Sb) {
                    const int tix = Ub * (Ub + 1) / 2 + Sb;
                    if (tix % kWaves != wave) continue;
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < (DK + 31) / 32; ++ks) {
                        const int i_lo = ks * 32 + 4 * lg, i_hi = i_lo + 16;
                        bf16x8 A[NS], Bv[NS];
#pragma unroll
                        for (int n = 0; n < NS; ++n) {
                            const __bf16 *kr = sK + (n * C + Sb * 16 + lc) * RS;
                            const __bf16 *qr = sQ + (n * C + Ub * 16 + lc) * RS;
                            const bf16x4 klo = *(const bf16x4 *)(kr + i_lo);
                            const bf16x4 qlo = *(const bf16x4 *)(qr + i_lo);
                            const bf16x4 khi = i_hi < DK ? *(const bf16x4 *)(kr + i_hi) : zero4();
                            const bf16x4 qhi = i_hi < DK ? *(const bf16x4 *)(qr + i_hi) : zero4();
                            A[n] = cat(klo, khi);
                            Bv[n] = cat(qlo, qhi);
                        }
                        acc = mma_split<NS>(A, Bv, acc);
                    }
                    __bf16 pl[NS][4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        float x = acc[r];
                        if (Sb == Ub && 4 * lg + r > lc) x = 0.f;     // causal: keep s <= u
                        __bf16 p[NS];
                        split<NS>(x, p);
#pragma unroll
                        for (int n = 0; n < NS; ++n) pl[n][r] = p[n];
                    }
#pragma unroll
                    for (int n = 0; n < NS; ++n) {
                        bf16x4 w;
                        w[0] = pl[n][0]; w[1] = pl[n][1]; w[2] = pl[n][2]; w[3] = pl[n][3];
                        *(bf16x4 *)(sA + ((tix * NS + n) * 64 + lane) * 4) = w;
                    }
                }
            }
        }

        // ================= 3. dS = Kh^T V' and S = diag(exp(b_L)) S + dS
#pragma unroll
        for (int slot = 0; slot < SPW; ++slot) {
            const int idx = slot * kWaves + wave;
            if (idx < NI * NJ) {
                const int I = idx / NJ, J = idx % NJ;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < (C + 31) / 32; ++ks) {
                    const int s_lo = ks * 32 + 4 * lg, s_hi = s_lo + 16;
                    bf16x8 A[NS], Bv[NS];
#pragma unroll
                    for (int n = 0; n < NS; ++n) {
                        const __bf16 *kr = sKh + (n * DK + I * 16 + lc) * CS;
                        const __bf16 *vr = sV + (n * DVT + J * 16 + lc) * CS;
                        const bf16x4 klo = *(const bf16x4 *)(kr + s_lo);
                        const bf16x4 vlo = *(const bf16x4 *)(vr + s_lo);
                        const bf16x4 khi = s_hi < C ? *(const bf16x4 *)(kr + s_hi) : zero4();
                        const bf16x4 vhi = s_hi < C ? *(const bf16x4 *)(vr + s_hi) : zero4();
                        A[n] = cat(klo, khi);
                        Bv[n] = cat(vlo, vhi);
                    }
                    acc = mma_split<NS>(A, Bv, acc);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    S[slot][r] = sGam[I * 16 + 4 * lg + r] * S[slot][r] + acc[r];
            }
        }
        if (!outputs) {
            gam_acc *= sGam[ci];
            __syncthreads();           // LDS is rewritten by the next chunk's prep
            continue;
        }
        __syncthreads();

        // ================= 4. O = A V' + Qt S'  (output tiles (Ub, J))
#pragma unroll
        for (int ot = 0; ot < NU * NJ; ++ot) {
            if (ot % kWaves != wave) continue;
            const int Ub = ot / NJ, J = ot % NJ;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            // intra-chunk: k = s over token blocks 0..Ub, two 16-blocks per step
#pragma unroll
            for (int p = 0; p <= Ub / 2; ++p) {
                const int S0 = 2 * p, S1 = 2 * p + 1;
                const int s_lo = p * 32 + 4 * lg, s_hi = s_lo + 16;
                bf16x8 A[NS], Bv[NS];
#pragma unroll
                for (int n = 0; n < NS; ++n) {
                    const int t0x = Ub * (Ub + 1) / 2 + S0;
                    const bf16x4 alo = *(const bf16x4 *)(sA + ((t0x * NS + n) * 64 + lane) * 4);
                    const bf16x4 ahi = S1 <= Ub
                        ? *(const bf16x4 *)(sA + (((t0x + 1) * NS + n) * 64 + lane) * 4) : zero4();
                    const __bf16 *vr = sV + (n * DVT + J * 16 + lc) * CS;
                    const bf16x4 vlo = *(const bf16x4 *)(vr + s_lo);
                    const bf16x4 vhi = (S1 <= Ub) ? *(const bf16x4 *)(vr + s_hi) : zero4();
                    A[n] = cat(alo, ahi);
                    Bv[n] = cat(vlo, vhi);
                }
                acc = mma_split<NS>(A, Bv, acc);
            }
            // inter-chunk: k = i, A = Qt rows, B = state images of tiles (2ks, J), (2ks+1, J)
#pragma unroll
            for (int ks = 0; ks < (DK + 31) / 32; ++ks) {
                const int i_lo = ks * 32 + 4 * lg, i_hi = i_lo + 16;
                const int I0 = 2 * ks, I1 = 2 * ks + 1;
                bf16x8 A[NS], Bv[NS];
#pragma unroll
                for (int n = 0; n < NS; ++n) {
                    const __bf16 *qr = sQ + (n * C + Ub * 16 + lc) * RS;
                    const bf16x4 qlo = *(const bf16x4 *)(qr + i_lo);
                    const bf16x4 qhi = i_hi < DK ? *(const bf16x4 *)(qr + i_hi) : zero4();
                    const bf16x4 slo = *(const bf16x4 *)(sS + (((I0 * NJ + J) * NS + n) * 64 + lane) * 4);
                    const bf16x4 shi = I1 < NI
                        ? *(const bf16x4 *)(sS + (((I1 * NJ + J) * NS + n) * 64 + lane) * 4) : zero4();
                    A[n] = cat(qlo, qhi);
                    Bv[n] = cat(slo, shi);
                }
                acc = mma_split<NS>(A, Bv, acc);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tok = t0 + Ub * 16 + 4 * lg + r;
                if (tok < a.T)
                    a.out[(((size_t)b * a.T + tok) * a.H + h) * a.dv + j0 + J * 16 + lc] = acc[r];
            }
        }
        __syncthreads();               // LDS is rewritten by the next chunk's prep
    }

    // ---- state out
    if (a.s_out && (!a.s_out_last_only || seg == a.n_seg - 1)) {
        float *so = a.s_out + bh * a.s_out_bh + seg * a.s_out_seg;
#pragma unroll
        for (int slot = 0; slot < SPW; ++slot) {
            const int idx = slot * kWaves + wave;
            if (idx < NI * NJ) {
                const int I = idx / NJ, J = idx % NJ;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    so[(size_t)(I * 16 + 4 * lg + r) * a.dv + j0 + J * 16 + lc] = S[slot][r];
            }
        }
    }
    if (!outputs && a.gam_out && jt == 0 && cgp == 0)
        a.gam_out[((size_t)bh * a.n_seg + seg) * DK + ci] = gam_acc;
}

template <int DK, int DVT, int C, typename TIn>
hipError_t launch_t(const ChunkLaunch &Lc, hipStream_t stream)
{
    constexpr int NS = std::is_same<TIn, float>::value ? 3 : 2;
    const size_t lds = Lds<DK, DVT, C, NS>::bytes;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void *)chunk_fwd_kernel<DK, DVT, C, TIn>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    Args a;
    a.B = Lc.B; a.T = Lc.T; a.H = Lc.H; a.dv = Lc.dv;
    a.n_seg = Lc.n_seg; a.chunks_per_seg = Lc.chunks_per_seg;
    a.n_chunks = (Lc.T + C - 1) / C;
    a.n_jt = Lc.dv / DVT;
    a.mode = Lc.mode;
    a.q = Lc.in.q; a.k = Lc.in.k; a.g = Lc.in.g; a.tau = Lc.in.tau; a.v = Lc.in.v; a.beta = Lc.in.beta;
    a.s_in = Lc.s_in; a.s_in_bh = Lc.s_in_bh_stride; a.s_in_seg = Lc.s_in_seg_stride;
    a.out = Lc.out;
    a.s_out = Lc.s_out; a.s_out_bh = Lc.s_out_bh_stride; a.s_out_seg = Lc.s_out_seg_stride;
    a.s_out_last_only = Lc.s_out_last_only;
    a.gam_out = Lc.gam_out;
    const long long blocks = (long long)Lc.B * Lc.H * Lc.n_seg * a.n_jt;
    a.remap = (blocks % 8 == 0) ? 1 : 0;
    hipLaunchKernelGGL((chunk_fwd_kernel<DK, DVT, C, TIn>), dim3((unsigned)blocks), dim3(kThreads),
                       lds, stream, a);
    return hipGetLastError();
}

// Instantiates every (DVT, C) tile shape for one dk and defines its size
// query and launcher.
#define RODIMUS_DEFINE_CHUNK_DK(XK)                                                   \
    size_t chunk_lds_bytes_dk##XK(int dvt, int C, bool f32)                           \
    {                                                                                 \
        using chunk_detail::Lds;                                                      \
        if (dvt == 16 && C == 16) return f32 ? Lds<XK, 16, 16, 3>::bytes : Lds<XK, 16, 16, 2>::bytes; \
        if (dvt == 16 && C == 32) return f32 ? Lds<XK, 16, 32, 3>::bytes : Lds<XK, 16, 32, 2>::bytes; \
        if (dvt == 16 && C == 64) return f32 ? Lds<XK, 16, 64, 3>::bytes : Lds<XK, 16, 64, 2>::bytes; \
        if (dvt == 32 && C == 16) return f32 ? Lds<XK, 32, 16, 3>::bytes : Lds<XK, 32, 16, 2>::bytes; \
        if (dvt == 32 && C == 32) return f32 ? Lds<XK, 32, 32, 3>::bytes : Lds<XK, 32, 32, 2>::bytes; \
        if (dvt == 32 && C == 64) return f32 ? Lds<XK, 32, 64, 3>::bytes : Lds<XK, 32, 64, 2>::bytes; \
        if (dvt == 64 && C == 16) return f32 ? Lds<XK, 64, 16, 3>::bytes : Lds<XK, 64, 16, 2>::bytes; \
        if (dvt == 64 && C == 32) return f32 ? Lds<XK, 64, 32, 3>::bytes : Lds<XK, 64, 32, 2>::bytes; \
        if (dvt == 64 && C == 64) return f32 ? Lds<XK, 64, 64, 3>::bytes : Lds<XK, 64, 64, 2>::bytes; \
        return 0;                                                                     \
    }                                                                                 \
    hipError_t launch_chunk_dk##XK(const ChunkLaunch &Lc, hipStream_t stream)         \
    {                                                                                 \
        using chunk_detail::launch_t;                                                 \
        if (Lc.DVT == 16 && Lc.C == 16) return Lc.f32_inputs ? launch_t<XK, 16, 16, float>(Lc, stream) : launch_t<XK, 16, 16, __bf16>(Lc, stream); \
        if (Lc.DVT == 16 && Lc.C == 32) return Lc.f32_inputs ? launch_t<XK, 16, 32, float>(Lc, stream) : launch_t<XK, 16, 32, __bf16>(Lc, stream); \
        if (Lc.DVT == 16 && Lc.C == 64) return Lc.f32_inputs ? launch_t<XK, 16, 64, float>(Lc, stream) : launch_t<XK, 16, 64, __bf16>(Lc, stream); \
        if (Lc.DVT == 32 && Lc.C == 16) return Lc.f32_inputs ? launch_t<XK, 32, 16, float>(Lc, stream) : launch_t<XK, 32, 16, __bf16>(Lc, stream); \
        if (Lc.DVT == 32 && Lc.C == 32) return Lc.f32_inputs ? launch_t<XK, 32, 32, float>(Lc, stream) : launch_t<XK, 32, 32, __bf16>(Lc, stream); \
        if (Lc.DVT == 32 && Lc.C == 64) return Lc.f32_inputs ? launch_t<XK, 32, 64, float>(Lc, stream) : launch_t<XK, 32, 64, __bf16>(Lc, stream); \
        if (Lc.DVT == 64 && Lc.C == 16) return Lc.f32_inputs ? launch_t<XK, 64, 16, float>(Lc, stream) : launch_t<XK, 64, 16, __bf16>(Lc, stream); \
        if (Lc.DVT == 64 && Lc.C == 32) return Lc.f32_inputs ? launch_t<XK, 64, 32, float>(Lc, stream) : launch_t<XK, 64, 32, __bf16>(Lc, stream); \
        if (Lc.DVT == 64 && Lc.C == 64) return Lc.f32_inputs ? launch_t<XK, 64, 64, float>(Lc, stream) : launch_t<XK, 64, 64, __bf16>(Lc, stream); \
        return hipErrorInvalidValue;                                                  \
    }

}  // namespace chunk_detail
}  // namespace rodimus
