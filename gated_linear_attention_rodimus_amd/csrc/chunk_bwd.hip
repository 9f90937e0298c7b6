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
//   (1) the forward chunk kernel in state-only mode, which writes S_in of every
//       chunk and S_T to the workspace;
//   (2) adjoint_sweep_kernel: D backwards over the chunks by the dL/dS_in line
//       above, one workgroup per (b, h, 64 dv columns), writing D of every
//       chunk to the workspace and dL/dS_0;
//   (3) chunk_grad_kernel: one workgroup per (b, h, chunk), every chunk in
//       parallel, forming all of the chunk's gradients from S_in, S_o and D.
// Every product is a 16x16-tile MFMA (v_mfma_f32_16x16x32_bf16, fp32
// accumulate) whose fp32 operands are split into NS bf16 terms as they are
// read (NS = 2 for bf16 inputs, 3 for fp32), as in the forward.  Tail tokens
// read as zero (inert) and their gradients are not stored.
#include "chunk_kernel.h"

namespace rodimus {
namespace bwd_detail {

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
__device__ __forceinline__ void st_tok(rsrc_t r, unsigned off_elems, float v) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off_elems * 4u, 0, 2);   // non-temporal
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

// ... from an array whose columns run along k: x[e] = p[(k0 + kslot(lg, e)) * pitch + col].
template <int K>
__device__ __forceinline__ void op_cols(const float *p, int pitch, int col, int k0, int lg, float *x) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
        x[e] = (K >= 32 || e < 4) ? p[(size_t)(k0 + kslot(lg, e)) * pitch + col] : 0.f;
}

// ------------------------------------------------------------------ (2) adjoint sweep

struct SweepArgs {
    int T, H, dv, n_chunks;
    const void *q, *g, *tau;
    const float *dout, *dsf;
    float *d_chunks;           // [B*H][n_chunks][DK][dv]: D = dL/dS leaving every chunk
    float *ds0;                // [B*H][DK][dv] or null
};

// One workgroup per (b, h, JT columns of dv); wave w owns dk rows 16w..16w+15.
// D lives in registers in the MFMA C-layout (row 16 w + 4 lg + i, column
// 16 jt + lc).  Per chunk, last to first: store D (= dL/dS leaving the chunk),
// then D <- diag(e^{b_L}) D + (q e^{b})^T dO, with q e^{b} (b <= 0, from the
// chunk start) formed in the A-operand layout directly: lane (lc, lg) holds
// column r = 16 w + lc at tokens 16 t + 4 lg + i, which for t = 2 ks, 2 ks + 1
// are the k-slots of step ks.  dO of the chunk is staged in LDS (two buffers)
// and the next chunk's gates and dO are loaded into registers meanwhile.
template <int DK, int JT, typename TIn>
__global__ __launch_bounds__(64 * (DK / 16)) void adjoint_sweep_kernel(SweepArgs a)
{
    constexpr int NS = std::is_same<TIn, float>::value ? 3 : 2;
    constexpr int C = ChunkOf<DK>::C, NU = C / 16, NW = DK / 16, NT = 64 * NW;
    constexpr int NJ = JT / 16, PJ = JT + 4;
    constexpr int NPD = C * JT / 4, LD = (NPD + NT - 1) / NT;
    __shared__ __attribute__((aligned(16))) float sdo[2][C * PJ];

    const int tid = threadIdx.x, lane = tid & 63, lc = lane & 15, lg = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int bh = blockIdx.x, j0 = blockIdx.y * JT;
    const int b = bh / a.H, h = bh % a.H, dv = a.dv;
    const long long T = a.T, H = a.H, row0 = (long long)b * T * H + h;
    const int r = 16 * wave + lc;
    const TIn *gq = (const TIn *)a.q, *gg = (const TIn *)a.g, *gt = (const TIn *)a.tau;

    f32x4 D[NJ];
#pragma unroll
    for (int jt = 0; jt < NJ; ++jt) D[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (a.dsf)
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                D[jt][i] = a.dsf[((size_t)bh * DK + 16 * wave + 4 * lg + i) * dv + j0 + 16 * jt + lc];

    // next chunk's gates, kept raw (converted where used, so the loads stay in
    // flight across the chunk in between)
    typedef typename chunk_detail::InRaw<TIn>::type Raw;
    Raw pq[NU][4], pg[NU][4], pt[NU][4];
    f32x4 pd[LD];
    auto prefetch = [&](int c) {
        const long long c0 = (long long)c * C;
        const long long lim = (T - c0) * H - h;                // token rows left from here
        const size_t bk = (size_t)(row0 + c0 * H) * DK, bv = (size_t)(row0 + c0 * H) * dv;
        const rsrc_t Rq = make_rsrc(gq + bk, lim * DK * (long long)sizeof(TIn));
        const rsrc_t Rg = make_rsrc(gg + bk, lim * DK * (long long)sizeof(TIn));
        const rsrc_t Rt = make_rsrc(gt + bk, lim * DK * (long long)sizeof(TIn));
        const rsrc_t Rd = make_rsrc(a.dout + bv, lim * dv * 4);
#pragma unroll
        for (int t = 0; t < NU; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const unsigned o = (unsigned)((16 * t + 4 * lg + i) * H * DK + r);
                pq[t][i] = ld_raw<TIn>(Rq, o);
                pg[t][i] = ld_raw<TIn>(Rg, o);
                pt[t][i] = ld_raw<TIn>(Rt, o);
            }
#pragma unroll
        for (int m = 0; m < LD; ++m) {
            const int p = tid + m * NT, u = p / (JT / 4), j = (p % (JT / 4)) * 4;
            const unsigned o = (unsigned)((u * H * dv + j0 + j) * 4);
            pd[m] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(Rd, p < NPD ? o : 0x80000000u, 0, 0));
        }
    };

    if (a.n_chunks > 0) prefetch(a.n_chunks - 1);
    for (int c = a.n_chunks - 1; c >= 0; --c) {
        // q e^{b} over the chunk (b from the chunk start, log2 units) and e^{b_L}
        float qd[NU][4];
        float run = 0.f;
#pragma unroll
        for (int t = 0; t < NU; ++t) {
            float p[4], s = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                s = __builtin_fmaf(chunk_detail::in_to_f32(pg[t][i]), chunk_detail::in_to_f32(pt[t][i]), s);
                p[i] = s;
            }
            float incl = s, y;
            y = __shfl_up(incl, 16); if (lg >= 1) incl += y;
            y = __shfl_up(incl, 32); if (lg >= 2) incl += y;
            const float excl = incl - s, tot = __shfl(incl, 48 + lc);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                qd[t][i] = chunk_detail::in_to_f32(pq[t][i]) *
                           __builtin_amdgcn_exp2f(-kLog2e * (run + excl + p[i]));
            run += tot;
        }
        const float ebl = __builtin_amdgcn_exp2f(-kLog2e * run);
        float *buf = sdo[c & 1];
#pragma unroll
        for (int m = 0; m < LD; ++m) {
            const int p = tid + m * NT, u = p / (JT / 4), j = (p % (JT / 4)) * 4;
            if (p < NPD) *(f32x4 *)(buf + u * PJ + j) = pd[m];
        }
        if (c > 0) prefetch(c - 1);
        __syncthreads();
        float *wd = a.d_chunks + ((size_t)bh * a.n_chunks + c) * DK * dv;
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                __builtin_nontemporal_store(D[jt][i], wd + (size_t)(16 * wave + 4 * lg + i) * dv + j0 + 16 * jt + lc);
        float el[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) el[i] = __shfl(ebl, 4 * lg + i);
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
            for (int i = 0; i < 4; ++i) D[jt][i] *= el[i];
#pragma unroll
        for (int ks = 0; ks < C / 32; ++ks) {
            float ax[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) ax[e] = qd[2 * ks + (e >> 2)][e & 3];
            bf16x8 A[NS];
            split8<NS>(ax, A);
#pragma unroll
            for (int jt = 0; jt < NJ; ++jt) {
                float bx[8];
                op_cols<C>(buf, PJ, 16 * jt + lc, 32 * ks, lg, bx);
                bf16x8 Bv[NS];
                split8<NS>(bx, Bv);
                D[jt] = mma_split<NS>(A, Bv, D[jt]);
            }
        }
    }
    if (a.ds0)
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                a.ds0[((size_t)bh * DK + 16 * wave + 4 * lg + i) * dv + j0 + 16 * jt + lc] = D[jt][i];
}

// ------------------------------------------------------------------ (3) chunk gradients

struct GradArgs {
    int T, H, n_chunks, n_work;
    const void *q, *k, *g, *tau, *v, *beta;
    const float *dout;
    const float *s_chunks;     // [B*H][n_chunks][DK][DV] S entering every chunk
    const float *s_final;      // [B*H][DK][DV]
    const float *d_chunks;     // [B*H][n_chunks][DK][DV] D leaving every chunk
    float *dq, *dk, *dg, *dtau, *dv, *dbeta;
};

// LDS in floats, rows padded by 4 floats (16-byte aligned rows; the four k-slot
// groups of a column-wise operand read land in distinct banks).
template <int DK, int DV>
struct GradCfg {
    static constexpr int C = ChunkOf<DK>::C, NU = C / 16, NRB = DK / 16, NJT = DV / 16;
    static constexpr int NW = NRB > 4 ? NRB : 4, NT = 64 * NW;
    static constexpr int PK = DK + 4, PV = DV + 4, PC = C + 4;
    static constexpr int o_qt = 0, o_kt = o_qt + C * PK, o_do = o_kt + C * PK, o_vp = o_do + C * PV;
    static constexpr int end0 = o_vp + C * PV;
    // A^T and dA^T are written once Qt and V' are no longer read: over them
    // where the rows fit, else past the end
    static constexpr int o_at = PC <= PK ? o_qt : end0;
    static constexpr int end1 = PC <= PK ? end0 : end0 + C * PC;
    static constexpr int o_dat = PC <= PV ? o_vp : end1;
    static constexpr int end2 = PC <= PV ? end1 : end1 + C * PC;
    static constexpr int o_f = end2;
    static constexpr int floats = o_f + DK;
    static constexpr size_t bytes = (size_t)floats * 4;
};

// One workgroup per (b, h, chunk).  Roles of wave w:
//   dk block w (w < DK/16): the gates of columns 16w..16w+15 over the chunk's
//     tokens (lane (lc, lg): column 16 w + lc, tokens 16 t + 4 lg + i, which is
//     also the MFMA C-layout of a [token tile t] x [dk block w] tile and, for
//     t = 2 ks, 2 ks + 1, the k-slots of step ks), then dQt and dKt of the block
//     and the elementwise tail (dq, dk, dlambda, dg, dtau);
//   token tile w (w < C/16): rows w of A^T and dA^T;
//   dv tiles w, w + NW, ...: dV' of those 16 columns, then dv and dbeta_hat.
template <int DK, int DV, typename TIn>
__global__ __launch_bounds__((GradCfg<DK, DV>::NT), 1) void chunk_grad_kernel(GradArgs a)
{
    typedef GradCfg<DK, DV> L;
    constexpr int NS = std::is_same<TIn, float>::value ? 3 : 2;
    constexpr int C = L::C, NU = L::NU, NRB = L::NRB, NJT = L::NJT, NW = L::NW, NT = L::NT;
    constexpr int PK = L::PK, PV = L::PV, PC = L::PC;
    constexpr int KSC = C / 32, JPW = (NJT + NW - 1) / NW;
    extern __shared__ __attribute__((aligned(16))) float sm[];
    float *sQt = sm + L::o_qt, *sKt = sm + L::o_kt, *sdO = sm + L::o_do, *sVp = sm + L::o_vp;
    float *sAt = sm + L::o_at, *sdAt = sm + L::o_dat, *sF = sm + L::o_f;

    // work item: workgroups are dealt to the 8 XCDs round-robin; give each XCD
    // a contiguous range of (b, h, chunk), so the state a chunk reads as S_o is
    // read as S_in by its neighbour on the same L2
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
    const float *Sout = c + 1 < a.n_chunks ? Sin + SD : a.s_final + (size_t)bh * SD;
    const float *Dout = a.d_chunks + ((size_t)bh * a.n_chunks + c) * SD;
    // token rows of head h from the chunk start to the sequence end
    const long long lim = (T - c0) * H - h;
    const size_t bk = (size_t)(row0 + c0 * H) * DK, bv = (size_t)(row0 + c0 * H) * DV;
    constexpr long long ESZ = sizeof(TIn);
    const unsigned HK = (unsigned)(H * DK), HV = (unsigned)(H * DV);

    // ---- dO and V' = beta_hat v of the chunk into LDS (16-byte pieces)
    {
        const rsrc_t Rd = make_rsrc(a.dout + bv, lim * DV * 4);
        const rsrc_t Rv = make_rsrc(gv + bv, lim * DV * ESZ);
        const rsrc_t Rb = make_rsrc(gb + bv, lim * DV * ESZ);
        constexpr int NPD = C * DV / 4, LPD = (NPD + NT - 1) / NT;
        typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
        constexpr int EPV = 16 / (int)sizeof(TIn);
        constexpr int NPV = C * DV / EPV, LPV = (NPV + NT - 1) / NT;
        u32x4v xd[LPD], xv[LPV], xb[LPV];
#pragma unroll
        for (int m = 0; m < LPD; ++m) {
            const int p = tid + m * NT, u = p / (DV / 4), j = (p % (DV / 4)) * 4;
            xd[m] = __builtin_amdgcn_raw_buffer_load_b128(Rd, p < NPD ? (u * HV + j) * 4u : 0x80000000u, 0, 0);
        }
#pragma unroll
        for (int m = 0; m < LPV; ++m) {
            const int p = tid + m * NT, u = p / (DV / EPV), j = (p % (DV / EPV)) * EPV;
            const unsigned o = p < NPV ? (u * HV + j) * (unsigned)ESZ : 0x80000000u;
            xv[m] = __builtin_amdgcn_raw_buffer_load_b128(Rv, o, 0, 0);
            xb[m] = __builtin_amdgcn_raw_buffer_load_b128(Rb, o, 0, 0);
        }
#pragma unroll
        for (int m = 0; m < LPD; ++m) {
            const int p = tid + m * NT, u = p / (DV / 4), j = (p % (DV / 4)) * 4;
            if (p < NPD) *(f32x4 *)(sdO + u * PV + j) = __builtin_bit_cast(f32x4, xd[m]);
        }
#pragma unroll
        for (int m = 0; m < LPV; ++m) {
            const int p = tid + m * NT, u = p / (DV / EPV), j = (p % (DV / EPV)) * EPV;
            if (p < NPV)
#pragma unroll
                for (int n4 = 0; n4 < EPV / 4; ++n4) {
                    f32x4 o;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int n = 4 * n4 + e;
                        float vv, bb;
                        if constexpr (EPV == 8) {
                            vv = __uint_as_float((n & 1) ? (xv[m][n >> 1] & 0xffff0000u) : (xv[m][n >> 1] << 16));
                            bb = __uint_as_float((n & 1) ? (xb[m][n >> 1] & 0xffff0000u) : (xb[m][n >> 1] << 16));
                        } else {
                            vv = __uint_as_float(xv[m][n]);
                            bb = __uint_as_float(xb[m][n]);
                        }
                        o[e] = vv * bb;
                    }
                    *(f32x4 *)(sVp + u * PV + j + 4 * n4) = o;
                }
        }
    }

    // ---- gates of this wave's dk block
    const bool rwave = wave < NRB;
    const int r = 16 * wave + lc;
    float q_[NU][4], k_[NU][4], g_[NU][4], t_[NU][4], d_[NU][4], ah_[NU][4];
    float ebm = 0.f, fl = 0.f;
    if (rwave) {
        const rsrc_t Rq = make_rsrc(gq + bk, lim * DK * ESZ), Rk = make_rsrc(gk + bk, lim * DK * ESZ);
        const rsrc_t Rg = make_rsrc(gg + bk, lim * DK * ESZ), Rt = make_rsrc(gt + bk, lim * DK * ESZ);
#pragma unroll
        for (int t = 0; t < NU; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const unsigned o = (16 * t + 4 * lg + i) * HK + r;
                q_[t][i] = ld_tok<TIn>(Rq, o);
                k_[t][i] = ld_tok<TIn>(Rk, o);
                g_[t][i] = ld_tok<TIn>(Rg, o);
                t_[t][i] = ld_tok<TIn>(Rt, o);
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
                d_[t][i] -= bm;                                    // b - b_m
                ah_[t][i] = gate_pow(g_[t][i], t_[t][i]);
                sQt[u * PK + r] = q_[t][i] * __builtin_amdgcn_exp2f(d_[t][i]);
                sKt[u * PK + r] = ah_[t][i] * k_[t][i] * __builtin_amdgcn_exp2f(-d_[t][i]);
            }
        ebm = __builtin_amdgcn_exp2f(bm);
        fl = __builtin_amdgcn_exp2f(bL - bm);
        if (lg == 0) sF[r] = fl;
    }
    __syncthreads();

    // ---- score tiles: A^T[s][u] = sum_r Kt[s][r] Qt[u][r], dA^T[s][u] =
    //      sum_j V'[s][j] dO[u][j], for the s tile of this wave and u tiles >= it
    f32x4 at[NU], dat[NU];
    if (wave < NU) {
        const int st = wave;
#pragma unroll
        for (int ut = 0; ut < NU; ++ut) { at[ut] = f32x4{0.f, 0.f, 0.f, 0.f}; dat[ut] = at[ut]; }
#pragma unroll
        for (int k0 = 0; k0 < DK; k0 += 32) {
            float x[8];
            bf16x8 A[NS];
            op_rows<DK>(sKt, PK, 16 * st + lc, k0, lg, x);
            split8<NS>(x, A);
#pragma unroll
            for (int ut = 0; ut < NU; ++ut)
                if (ut >= st) {
                    bf16x8 Bv[NS];
                    op_rows<DK>(sQt, PK, 16 * ut + lc, k0, lg, x);
                    split8<NS>(x, Bv);
                    at[ut] = mma_split<NS>(A, Bv, at[ut]);
                }
        }
#pragma unroll
        for (int k0 = 0; k0 < DV; k0 += 32) {
            float x[8];
            bf16x8 A[NS];
            op_rows<DV>(sVp, PV, 16 * st + lc, k0, lg, x);
            split8<NS>(x, A);
#pragma unroll
            for (int ut = 0; ut < NU; ++ut)
                if (ut >= st) {
                    bf16x8 Bv[NS];
                    op_rows<DV>(sdO, PV, 16 * ut + lc, k0, lg, x);
                    split8<NS>(x, Bv);
                    dat[ut] = mma_split<NS>(A, Bv, dat[ut]);
                }
        }
    }

    // ---- state terms of dQt and dKt for this wave's dk block, and rowsum(S_o * D):
    //      dQt += e^{b_m} dO S_in^T, dKt += f V' D^T (B operands straight from
    //      the workspace rows r = 16 w + lc)
    f32x4 dqt[NU], dkt[NU];
    float rs = 0.f;
    if (rwave) {
#pragma unroll
        for (int t = 0; t < NU; ++t) { dqt[t] = f32x4{0.f, 0.f, 0.f, 0.f}; dkt[t] = dqt[t]; }
#pragma unroll
        for (int k0 = 0; k0 < DV; k0 += 32) {
            float s[8], d[8], so[8];
            op_rows<DV>(Sin, DV, r, k0, lg, s);
            op_rows<DV>(Dout, DV, r, k0, lg, d);
            op_rows<DV>(Sout, DV, r, k0, lg, so);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                rs = __builtin_fmaf(so[e], d[e], rs);
                s[e] *= ebm;
                d[e] *= fl;
            }
            bf16x8 Bs[NS], Bd[NS];
            split8<NS>(s, Bs);
            split8<NS>(d, Bd);
#pragma unroll
            for (int t = 0; t < NU; ++t) {
                float x[8];
                bf16x8 A[NS];
                op_rows<DV>(sdO, PV, 16 * t + lc, k0, lg, x);
                split8<NS>(x, A);
                dqt[t] = mma_split<NS>(A, Bs, dqt[t]);
                op_rows<DV>(sVp, PV, 16 * t + lc, k0, lg, x);
                split8<NS>(x, A);
                dkt[t] = mma_split<NS>(A, Bd, dkt[t]);
            }
        }
        rs += __shfl_xor(rs, 16);
        rs += __shfl_xor(rs, 32);
    }
    __syncthreads();                       // Qt and V' no longer read

    // ---- A^T and dA^T (causal: u >= s) into LDS; the tile left of an odd
    //      diagonal tile is read by the 32-deep steps and is zero
    if (wave < NU) {
        const int st = wave;
#pragma unroll
        for (int ut = 0; ut < NU; ++ut)
            if (ut >= st)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int s_ = 16 * st + 4 * lg + i, u = 16 * ut + lc;
                    const bool keep = u >= s_;
                    sAt[s_ * PC + u] = keep ? at[ut][i] : 0.f;
                    sdAt[s_ * PC + u] = keep ? dat[ut][i] : 0.f;
                }
        if (st & 1)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int s_ = 16 * st + 4 * lg + i, u = 16 * (st - 1) + lc;
                sAt[s_ * PC + u] = 0.f;
                sdAt[s_ * PC + u] = 0.f;
            }
    }
    __syncthreads();

    // ---- dQt += dA Kt (s <= u), dKt += dA^T Qt (u >= s); Kt and Qt of the
    //      block as B operands from the gate registers
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
                float x[8];
                bf16x8 A[NS];
                if (2 * ks <= t) {                         // dA[u][s] = dA^T[s][u], u in tile t
                    op_cols<C>(sdAt, PC, 16 * t + lc, 32 * ks, lg, x);
                    split8<NS>(x, A);
                    dqt[t] = mma_split<NS>(A, BK, dqt[t]);
                }
                if (2 * ks + 1 >= t) {                     // dA^T rows s in tile t
                    op_rows<C>(sdAt, PC, 16 * t + lc, 32 * ks, lg, x);
                    split8<NS>(x, A);
                    dkt[t] = mma_split<NS>(A, BQ, dkt[t]);
                }
            }
        }
    }

    // ---- dV' = A^T dO + Kt diag(f) D for this wave's dv tiles
    f32x4 dvp[JPW][NU];
#pragma unroll
    for (int jj = 0; jj < JPW; ++jj) {
        const int jt = wave + jj * NW;
        if (jt < NJT) {
#pragma unroll
            for (int t = 0; t < NU; ++t) dvp[jj][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KSC; ++ks) {
                float y[8];
                bf16x8 Bv[NS];
                op_cols<C>(sdO, PV, 16 * jt + lc, 32 * ks, lg, y);
                split8<NS>(y, Bv);
#pragma unroll
                for (int t = 0; t < NU; ++t)
                    if (2 * ks + 1 >= t) {
                        float x[8];
                        bf16x8 A[NS];
                        op_rows<C>(sAt, PC, 16 * t + lc, 32 * ks, lg, x);
                        split8<NS>(x, A);
                        dvp[jj][t] = mma_split<NS>(A, Bv, dvp[jj][t]);
                    }
            }
#pragma unroll
            for (int k0 = 0; k0 < DK; k0 += 32) {
                float y[8];
                bf16x8 Bv[NS];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int kk = k0 + kslot(lg, e);
                    y[e] = kk < DK ? Dout[(size_t)kk * DV + 16 * jt + lc] * sF[kk] : 0.f;
                }
                split8<NS>(y, Bv);
#pragma unroll
                for (int t = 0; t < NU; ++t) {
                    float x[8];
                    bf16x8 A[NS];
                    op_rows<DK>(sKt, PK, 16 * t + lc, k0, lg, x);
                    split8<NS>(x, A);
                    dvp[jj][t] = mma_split<NS>(A, Bv, dvp[jj][t]);
                }
            }
        }
    }

    // ---- elementwise tail of the dk block: dq, dk, then dlambda as a suffix
    //      sum over the chunk's tokens (+ rowsum(S_o D)), dg and dtau
    if (rwave) {
        const rsrc_t Rq = make_rsrc(a.dq + bk, lim * DK * 4), Rk = make_rsrc(a.dk + bk, lim * DK * 4);
        const rsrc_t Rg = make_rsrc(a.dg + bk, lim * DK * 4), Rt = make_rsrc(a.dtau + bk, lim * DK * 4);
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
                st_tok(Rq, u * HK + r, dqv);
                st_tok(Rk, u * HK + r, ah_[t][i] * dkp);
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
                st_tok(Rg, u * HK + r, dgv);
                st_tok(Rt, u * HK + r, dtv);
            }
            carry += tot;
        }
    }

    // ---- dv = beta_hat dV', dbeta_hat = v dV'
    {
        const rsrc_t Rv = make_rsrc(gv + bv, lim * DV * ESZ), Rb = make_rsrc(gb + bv, lim * DV * ESZ);
        const rsrc_t Rdv = make_rsrc(a.dv + bv, lim * DV * 4), Rdb = make_rsrc(a.dbeta + bv, lim * DV * 4);
#pragma unroll
        for (int jj = 0; jj < JPW; ++jj) {
            const int jt = wave + jj * NW;
            if (jt < NJT) {
                float vv[NU][4], bb[NU][4];
#pragma unroll
                for (int t = 0; t < NU; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const unsigned o = (16 * t + 4 * lg + i) * HV + 16 * jt + lc;
                        vv[t][i] = ld_tok<TIn>(Rv, o);
                        bb[t][i] = ld_tok<TIn>(Rb, o);
                    }
#pragma unroll
                for (int t = 0; t < NU; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const unsigned o = (16 * t + 4 * lg + i) * HV + 16 * jt + lc;
                        st_tok(Rdv, o, bb[t][i] * dvp[jj][t][i]);
                        st_tok(Rdb, o, vv[t][i] * dvp[jj][t][i]);
                    }
            }
        }
    }
}

template <int DK, int DV, typename TIn>
hipError_t launch_typed(const ChunkBwdLaunch &Lc, hipStream_t stream)
{
    typedef GradCfg<DK, DV> L;
    constexpr int C = L::C;
    const int n_chunks = (Lc.T + C - 1) / C, BH = Lc.B * Lc.H;
    constexpr int JT = DV < 64 ? DV : 64;
    SweepArgs sa;
    sa.T = Lc.T; sa.H = Lc.H; sa.dv = DV; sa.n_chunks = n_chunks;
    sa.q = Lc.in.q; sa.g = Lc.in.g; sa.tau = Lc.in.tau;
    sa.dout = Lc.dout; sa.dsf = Lc.dsf; sa.d_chunks = Lc.d_chunks; sa.ds0 = Lc.ds0;
    hipLaunchKernelGGL((adjoint_sweep_kernel<DK, JT, TIn>), dim3(BH, DV / JT), dim3(64 * (DK / 16)), 0,
                       stream, sa);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;

    static bool attr_set = false;
    if (!attr_set) {
        e = hipFuncSetAttribute((const void *)chunk_grad_kernel<DK, DV, TIn>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)L::bytes);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    GradArgs ga;
    ga.T = Lc.T; ga.H = Lc.H; ga.n_chunks = n_chunks; ga.n_work = BH * n_chunks;
    ga.q = Lc.in.q; ga.k = Lc.in.k; ga.g = Lc.in.g; ga.tau = Lc.in.tau; ga.v = Lc.in.v;
    ga.beta = Lc.in.beta; ga.dout = Lc.dout;
    ga.s_chunks = Lc.s_chunks; ga.s_final = Lc.s_final; ga.d_chunks = Lc.d_chunks;
    ga.dq = Lc.dq; ga.dk = Lc.dk_; ga.dg = Lc.dg; ga.dtau = Lc.dtau; ga.dv = Lc.dv_; ga.dbeta = Lc.dbeta;
    const int grid = 8 * ((ga.n_work + 7) / 8);
    hipLaunchKernelGGL((chunk_grad_kernel<DK, DV, TIn>), dim3(grid), dim3(L::NT), L::bytes, stream, ga);
    return hipGetLastError();
}

}  // namespace bwd_detail

#define RODIMUS_BWD_SHAPES(X)                                                            \
    X(16, 16) X(16, 32) X(16, 64) X(16, 128) X(32, 16) X(32, 32) X(32, 64) X(32, 128)    \
    X(64, 16) X(64, 32) X(64, 64) X(64, 128) X(128, 16) X(128, 32) X(128, 64) X(128, 128)

size_t chunk_bwd_lds_bytes(int dk, int dv)
{
#define RODIMUS_BWD_LDS(XK, XV) if (dk == XK && dv == XV) return bwd_detail::GradCfg<XK, XV>::bytes;
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
