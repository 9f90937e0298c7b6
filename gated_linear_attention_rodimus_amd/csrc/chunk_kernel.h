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
//   O   = tril(Qt Kt^T) V' + Qt S'                (diagonal kept)
//   S_o = diag(exp(b_L)) S_in + Kh^T V'
// with V' = beta_hat*v, k' = g^tau * k and
//   Qt[u,i] = q[u,i] exp(b_u - b_m),  Kt[s,i] = k'[s,i] exp(b_m - b_s),
//   S'[i,:] = exp(b_m[i]) S_in[i,:],    Kh[s,i] = Kt[s,i] exp(b_L - b_m),
// and Kh^T V' = diag(exp(b_L - b_m)) Kt^T V', so Kt serves both products.
// b_m is the cumulative sum at the middle of the chunk: referencing the
// exponentials there halves their range (all exponents stay within half a
// chunk's total decay), and Qt Kt^T reproduces exp(b_u - b_s) for s <= u.
// Cumulative sums are kept in log2 units so every exponential is one v_exp_f32;
// alpha_hat = g^tau is folded into Kt's exponent (tau*log2 g), which leaves
// three transcendentals per (token, dk column).
//
// Precision: all four products run on bf16 MFMA (v_mfma_f32_16x16x32_bf16)
// with fp32 accumulation.  Every fp32 operand is split into NS bf16 terms
// (x = x0 + x1 [+ x2]) and the product keeps the cross terms of total order
// < NS: 3 MFMAs for bf16 inputs (NS = 2, ~16 mantissa bits per operand) and
// 6 MFMAs for fp32 inputs (NS = 3, ~24 bits).  The state stays in fp32
// registers across chunks.
//
// Workgroup: one (b, h, dv tile of DVT columns, segment), warp-specialised.
//  - 4 producer waves prepare chunk c+1 while the consumers compute chunk c.
//    Each producer thread owns a pair of adjacent dk columns and a run of
//    consecutive tokens: it forms the local cumulative sum (cross-thread
//    offsets through LDS), the gates and Qt, Kt (row form [u][i], bf16 planes)
//    in one of two LDS pipeline buffers, plus exp(b_m), exp(b_L) and
//    exp(b_L - b_m) per column.
//  - DVT/16 consumer waves; consumer w owns dv columns 16w..16w+15 of the
//    tile for the whole sweep: its state block S[:, w] (fp32 MFMA C-layout,
//    dk x 16), its V' columns (loaded straight into MFMA B-operand order) and
//    its output columns.  Per chunk it builds the B operands S' from its state
//    registers, computes its share of the 16x16 tiles of A^T = Kt Qt^T (stored
//    as register images in LDS), then dS = diag(exp(b_L - b_m)) Kt^T V' (Kt^T
//    through the transposing LDS read) with S = diag(exp(b_L)) S + dS, and
//    finally its output columns O = A V' + Qt S'.
//  Two workgroup barriers per chunk separate the phases; the consumers read
//  the buffer the producers wrote one iteration earlier.
// MFMA k-slots: a 32-deep k-step takes rows {4g..4g+3} of one 16-row tile and
// {16+4g..16+4g+3} of the next (g = lane/16), so a C-layout tile (rows
// 4g..4g+3 of lane group g) is directly a B operand of the next product; LDS
// operands are read with the same slot mapping.
//
// Global traffic goes through buffer resources whose size ends at the last
// valid token of the sequence: tail-chunk loads beyond it return zero (which
// makes those tokens inert: lambda = 0, k' = 0, v' = 0) and stores beyond it
// are dropped, so the loop has no per-element bounds branches.  Each role
// loads the next chunk's inputs into registers one iteration ahead.
#pragma once
#include "internal.h"

#include <type_traits>

namespace rodimus {
namespace chunk_detail {

constexpr float kLog2e = 1.4426950408889634f;
// s_waitcnt immediate (gfx9 encoding): vmcnt(0), expcnt and lgkmcnt unlimited
constexpr int kWaitVmcnt0 = 0x0f70;
constexpr int kBufFlags = 0x00020000;          // raw buffer, 32-bit data format (gfx9)

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16;

__device__ __forceinline__ float in_to_f32(u16 x) { return __uint_as_float((unsigned)x << 16); }
__device__ __forceinline__ float in_to_f32(float x) { return x; }

template <typename TIn> struct InRaw;
template <> struct InRaw<__bf16> { typedef u16 type; };
template <> struct InRaw<float> { typedef float type; };

__device__ __forceinline__ u16 buf_load(__amdgpu_buffer_rsrc_t r, unsigned off, u16) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}
__device__ __forceinline__ float buf_load(__amdgpu_buffer_rsrc_t r, unsigned off, float) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

// Dot product of two packed bf16 pairs accumulated into an fp32 value,
// a.lo * b.lo + a.hi * b.hi + c (v_dot2c_f32_bf16); the products are exact.
__device__ __forceinline__ float dot2_bf16(unsigned a, unsigned b, float c) {
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, a), __builtin_bit_cast(bf2, b), c,
                                          false);
}

// Two adjacent elements of a per-token input: one 32-bit word for bf16, two
// for fp32.
template <typename TIn> struct Pair;
template <> struct Pair<__bf16> {
    typedef unsigned type;
    static __device__ __forceinline__ type load(__amdgpu_buffer_rsrc_t r, unsigned off) {
        return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
    }
    static __device__ __forceinline__ float lo(type x) { return __uint_as_float(x << 16); }
    static __device__ __forceinline__ float hi(type x) { return __uint_as_float(x & 0xffff0000u); }
    // run + g * t of the low / high elements (one packed dot product each; the
    // operands are the unpacked words, i.e. pairs (0, x))
    static __device__ __forceinline__ float gt_lo(type g, type t, float run) {
        return dot2_bf16(g << 16, t << 16, run);
    }
    static __device__ __forceinline__ float gt_hi(type g, type t, float run) {
        return dot2_bf16(g & 0xffff0000u, t & 0xffff0000u, run);
    }
};
template <> struct Pair<float> {
    typedef unsigned type __attribute__((ext_vector_type(2)));
    static __device__ __forceinline__ type load(__amdgpu_buffer_rsrc_t r, unsigned off) {
        return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    }
    static __device__ __forceinline__ float lo(type x) { return __uint_as_float(x[0]); }
    static __device__ __forceinline__ float hi(type x) { return __uint_as_float(x[1]); }
    static __device__ __forceinline__ float gt_lo(type g, type t, float run) {
        return __builtin_fmaf(lo(g), lo(t), run);
    }
    static __device__ __forceinline__ float gt_hi(type g, type t, float run) {
        return __builtin_fmaf(hi(g), hi(t), run);
    }
};

// Buffer resource over [p, p + bytes); bytes is clamped to 31 bits.  The
// arguments are wave-uniform; readfirstlane states that to the compiler so the
// descriptor lives in SGPRs (a descriptor it cannot prove uniform turns every
// load into a readfirstlane loop).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, long long bytes) {
    if (bytes < 0) bytes = 0;
    if (bytes > 0x7fffffffLL) bytes = 0x7fffffffLL;
    const unsigned long long a = (unsigned long long)p;
    const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)a);
    const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(a >> 32));
    const int n = __builtin_amdgcn_readfirstlane((int)bytes);
    void *base = (void *)(((unsigned long long)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, n, kBufFlags);
}

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// A constant materialised in an SGPR by an instruction the optimiser does not
// look through (so a dot product with it is not rewritten into other forms).
template <unsigned V>
__device__ __forceinline__ unsigned sgpr_const() {
    unsigned r;
    asm("s_mov_b32 %0, %1" : "=s"(r) : "i"(V));
    return r;
}

// Split two fp32 values into NS packed bf16 pairs: out[n] holds term n of x0
// (low half) and of x1 (high half); x ~= sum of the terms.  Each term is the
// round-to-nearest-even bf16 of the remaining residual (v_cvt_pk_bf16_f32); the
// residual x - term is exact in fp32 and is formed by one packed dot product
// with the constant pair (-1, 0) or (0, -1).
template <int NS>
__device__ __forceinline__ void split_pair(float x0, float x1, unsigned *out) {
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
    typedef float f2 __attribute__((ext_vector_type(2)));
    f2 x = {x0, x1};
#pragma unroll
    for (int n = 0; n < NS; ++n) {
        const unsigned hu = __builtin_bit_cast(unsigned, __builtin_convertvector(x, bf2));
        out[n] = hu;
        if (n + 1 < NS) {
            x[0] = dot2_bf16(hu, sgpr_const<0x0000bf80u>(), x[0]);   // x0 - term (low half)
            x[1] = dot2_bf16(hu, sgpr_const<0xbf800000u>(), x[1]);   // x1 - term (high half)
        }
    }
}

__device__ __forceinline__ bf16x8 pack8(unsigned a, unsigned b, unsigned c, unsigned d) {
    return __builtin_bit_cast(bf16x8, u32x4{a, b, c, d});
}

__device__ __forceinline__ bf16x8 cat(bf16x4 lo, bf16x4 hi) {
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ bf16x4 zero4() {
    bf16x4 z;
    z[0] = z[1] = z[2] = z[3] = (__bf16)0.f;
    return z;
}

// acc += sum over split-term pairs (a, b) with a + b < NS of A[a] * B[b]
// (smallest terms first).
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

// Same as mma_split for NT independent tiles, issued term-major so that
// consecutive MFMAs never depend on each other.
template <int NS, int NT>
__device__ __forceinline__ void mma_split_n(const bf16x8 (*A)[NS], const bf16x8 (*Bv)[NS],
                                            f32x4 *acc) {
    if constexpr (NS == 3) {
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[t][1], Bv[t][1], acc[t], 0, 0, 0);
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[t][0], Bv[t][2], acc[t], 0, 0, 0);
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[t][2], Bv[t][0], acc[t], 0, 0, 0);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[t][0], Bv[t][1], acc[t], 0, 0, 0);
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[t][1], Bv[t][0], acc[t], 0, 0, 0);
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[t][0], Bv[t][0], acc[t], 0, 0, 0);
}

struct Args {
    int B, T, H, dv;
    int n_seg, chunks_per_seg, n_chunks, n_jt;
    int mode;                    // 0: outputs, 1: segment transfer
    const void *q, *k, *g, *tau, *v, *beta;
    const float *s_in; long long s_in_bh, s_in_seg;
    float *out;
    float *s_out; long long s_out_bh, s_out_seg; int s_out_last_only;
    float *gam_out; long long gam_bh;   // segment decays (mode 1): head bh, segment p at bh * gam_bh + p * DK
    int remap;                   // XCD-aware block mapping on/off
    // fused steps (kernels instantiated with FU only)
    const void *u, *w; int rank; // beta_hat = sigmoid(u w) when u is set: u [B][T][H][rank], w [H][rank][dv]
    const float *dfeed;          // feedthrough o += d * v, d [H][dv], or null
    int conv_w;                  // ShortConv taps (1: none); q, k, v carry conv_w - 1 history rows
    const float *cq, *ck, *cv;   // taps [H][D][conv_w]
};

// v_mul_legacy_f32: an IEEE product, except that 0 times anything (infinities
// included) is 0.
__device__ float fmul_legacy(float, float) __asm("llvm.amdgcn.fmul.legacy");

// log2 of alpha_hat = g^tau: tau * log2(g), and exactly 0 when tau == 0 (g^0 = 1,
// also at g = 0 where log2(g) = -inf); -inf for g = 0 < tau.
__device__ __forceinline__ float log2_gate_pow(float g, float tau) {
    return fmul_legacy(tau, __builtin_amdgcn_logf(g));
}

// Transposed LDS read of a 16-bit operand (gfx950 ds_read_b64_tr_b16).  Within
// each 16-lane group, lane m passes the address of 4 consecutive 16-bit values
// (row m/4, columns 4*(m%4)..+3 of a 4 x 16 block); lane i receives column i
// of the block, rows 0..3.
__device__ __forceinline__ bf16x4 lds_read_tr(const __bf16 *p) {
    typedef short v4s __attribute__((ext_vector_type(4)));
    v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4s *)(const_cast<__bf16 *>(p)));
    return __builtin_bit_cast(bf16x4, r);
}

// Compile-time shape of one instantiation, and its LDS layout (bytes).  The
// segment-transfer mode (OUT_ false) keeps no Qt planes, score tiles or
// output tile.
template <int DK, int DVT, int C, int NS_, bool OUT_ = true, int FU_ = 0>
struct Cfg {
    static constexpr int NS = NS_;
    static constexpr bool OUT = OUT_;
    static constexpr bool FU = FU_ != 0;                      // fused steps compiled in
    static constexpr bool CONV = FU_ == 1;                    // ... with the ShortConv (2: without)
    static constexpr int HALO = CONV ? 3 : 0;                 // ShortConv history rows (4 taps)
    static constexpr int NP = 4;                              // producer waves
    static constexpr int NJ = DVT / 16;                       // consumer waves
    static constexpr int NW = NP + NJ;
    static constexpr int NT = 64 * NW;                        // threads
    static constexpr int NU = C / 16, NI = DK / 16;
    static constexpr int NA = NU * (NU + 1) / 2;              // A^T tiles (upper triangle)
    static constexpr int PP = DK / 2;                         // dk column pairs
    static constexpr int NG0 = 64 * NP / PP;                  // token groups per column pair
    static constexpr int NG = NG0 < C ? NG0 : C;              // groups actually used
    static constexpr int TPG = C / NG;                        // tokens per group
    static constexpr int KSI = (DK + 31) / 32;                // k-steps over dk
    static constexpr int KSC = (C + 31) / 32;                 // k-steps over tokens
    static constexpr int RS = DK + 4;                         // row stride (bf16)
    static constexpr int MID = C / 2 - 1;                     // reference token b_m
    // one pipeline buffer: Qt and Kt planes, exp(b_m), exp(b_L), exp(b_L - b_m)
    static constexpr size_t bq_off = 0;
    static constexpr size_t bk_off = bq_off + (OUT ? (size_t)NS * C * RS * 2 : 0);
    static constexpr size_t bem_off = bk_off + (size_t)NS * C * RS * 2;
    static constexpr size_t bgam_off = bem_off + (size_t)DK * 4;
    static constexpr size_t bgm_off = bgam_off + (size_t)DK * 4;
    static constexpr size_t buf_bytes = (bgm_off + (size_t)DK * 4 + 15) / 16 * 16;
    static constexpr size_t a_off = 2 * buf_bytes;
    static constexpr size_t tot_off = a_off + (OUT ? (size_t)NA * NS * 64 * 4 * 2 : 0);
    static constexpr size_t mid_off = tot_off + (size_t)NG * DK * 4;
    // per consumer wave: raw v rows of one chunk (with the convolution's
    // history rows and one row of padding in ShortConv kernels), [SV][16] bf16, then
    // beta_hat, [C][16]
    static constexpr size_t stg_off = mid_off + (size_t)DK * 4;
    static constexpr int SV = C + (CONV ? HALO + 1 : 0);
    static constexpr size_t stg_wave = (size_t)(SV + C) * 16 * 2;
    // output tile of one chunk, [C][OS] fp32 (row stride DVT + 16 floats: the
    // four row groups of an MFMA C-layout write land in distinct banks)
    static constexpr int OS = DVT + 16;
    static constexpr size_t out_off = stg_off + (NS == 2 ? (size_t)NJ * stg_wave : 0);
    static constexpr size_t bytes = out_off + (OUT ? (size_t)C * OS * 4 : 0);
    // workgroups per CU the kernel is compiled for: two for bf16 inputs at
    // dk <= 64 and C <= 32, and in the transfer mode also at C = 64 on tiles
    // narrower than 64 x 64, where two fit the CU's LDS and the waves per SIMD
    // that brings leave each wave enough registers (128) without spilling;
    // one otherwise, and always one for the 12-wave 128-column tile
    static constexpr int per_cu =
        ((C <= 32 || (!OUT && (DK < 64 || DVT < 64))) && NS == 2 && 2 * bytes <= 160 * 1024 &&
         DK <= 64 && !FU && (NW <= 8 || (!OUT && C <= 32))) ? 2 : 1;
    static constexpr int waves_per_eu = (per_cu * NW + 3) / 4;
    static_assert(NG >= 1 && TPG * NG == C, "token groups");
    static_assert(C % 16 == 0 && DK % 16 == 0 && DVT % 16 == 0, "tile multiples");
};

template <int DK, int DVT, int C, typename TIn, bool OUT, int FU>
__global__ __launch_bounds__((Cfg<DK, DVT, C, 2>::NT),
                             (Cfg<DK, DVT, C, std::is_same<TIn, float>::value ? 3 : 2, OUT, FU>::waves_per_eu))
void chunk_fwd_kernel(Args a)
{
    constexpr int NS = std::is_same<TIn, float>::value ? 3 : 2;
    typedef Cfg<DK, DVT, C, NS, OUT, FU> L;
    constexpr int HALO = L::HALO;
    typedef typename InRaw<TIn>::type Raw;
    typedef Pair<TIn> PR;
    typedef typename PR::type Raw2;
    constexpr int NU = L::NU, NI = L::NI, NJ = L::NJ, NA = L::NA, NP = L::NP, PP = L::PP;
    constexpr int NG = L::NG, TPG = L::TPG, KSI = L::KSI, KSC = L::KSC;
    constexpr int RS = L::RS, MID = L::MID;
    constexpr int esz = sizeof(Raw);

    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    __bf16 *sA = (__bf16 *)(smem + L::a_off);
    float *sTot = (float *)(smem + L::tot_off);
    float *sMid = (float *)(smem + L::mid_off);
    auto bQ = [&](int buf) { return (__bf16 *)(smem + buf * L::buf_bytes + L::bq_off); };
    auto bK = [&](int buf) { return (__bf16 *)(smem + buf * L::buf_bytes + L::bk_off); };
    auto bEm = [&](int buf) { return (float *)(smem + buf * L::buf_bytes + L::bem_off); };
    auto bGam = [&](int buf) { return (float *)(smem + buf * L::buf_bytes + L::bgam_off); };
    auto bGm = [&](int buf) { return (float *)(smem + buf * L::buf_bytes + L::bgm_off); };

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
    const int c_begin = seg * a.chunks_per_seg;
    const int c_end = min(a.n_chunks, c_begin + a.chunks_per_seg);
    constexpr bool outputs = OUT;           // mode 0: outputs; mode 1: segment transfer

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lc = lane & 15, lg = lane >> 4;          // MFMA lane column / group
    const bool producer = wave < NP;
    const int cw = wave - NP;                          // consumer index (dv block)
    const int jcol = jt * DVT + (producer ? 0 : cw) * 16;
    const int cp = tid % PP, cgp = tid / PP;           // producer: dk column pair owner
    const int c0 = 2 * cp;                             // its columns c0, c0 + 1
    const bool prep = producer && cgp < NG;

    const long long T = a.T, H = a.H, dv = a.dv;
    const long long row_k = H * DK, row_v = H * dv;    // elements between tokens
    const long long head0 = (long long)b * T * H + h;
    // q, k, v of FU kernels: [B][T + conv_w - 1][H][D], the convolution's
    // history rows first; row X of a chunk's window is raw token t0 + X - HALO,
    // stored at row t0 + X - HALO + conv_w - 1 (rows before 0 read as zero)
    const int conv_w = L::CONV ? a.conv_w : 1;
    const long long Tx = T + conv_w - 1;
    const long long head0x = (long long)b * Tx * H + h;
    const long long xshift = (long long)conv_w - 1;            // stored row - raw token
    const Raw *gq = (const Raw *)a.q + head0x * DK;
    const Raw *gk = (const Raw *)a.k + head0x * DK;
    const Raw *gg = (const Raw *)a.g + head0 * DK;
    const Raw *gt = (const Raw *)a.tau + head0 * DK;
    const Raw *gv = (const Raw *)a.v + head0x * dv + jcol;
    const Raw *gb = (const Raw *)a.beta + head0 * dv + jcol;
    float *go = a.out ? a.out + head0 * dv + jt * DVT : nullptr;   // this dv tile

    // byte offsets of this thread's elements inside one chunk
    const unsigned off_k = (unsigned)(((long long)cgp * TPG * row_k + c0) * esz);
    const unsigned off_v = (unsigned)(((long long)4 * lg * row_v + lc) * esz);
    const unsigned step_k = (unsigned)(row_k * esz), step_v = (unsigned)(row_v * esz);

    // ---- consumer state block: S[I][r] = row I*16 + 4*lg + r, column jcol + lc
    float S[NI][4];
    {
        const float *sin = a.s_in ? a.s_in + bh * a.s_in_bh + seg * a.s_in_seg : nullptr;
#pragma unroll
        for (int I = 0; I < NI; ++I)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                S[I][r] = (sin && !producer) ? sin[(size_t)(I * 16 + 4 * lg + r) * a.dv + jcol + lc] : 0.f;
        // complete these loads here: a wait for them placed inside the chunk
        // loop would also wait for every output store still in flight
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    }
    // A^T tiles (Sb, Ub), Sb <= Ub, of the chunk in LDS buffer cb (rows s of Kt,
    // columns u of Qt, k = i), causally masked and stored split in sA as MFMA
    // A-operand register images.  Producer wave wi takes tiles wi, wi + NP, ...,
    // in interleaved groups.
    auto score_tiles = [&](int wi, int cb) {
        constexpr int TPW = (NA + NP - 1) / NP;            // tiles per wave
        // interleave group; one tile at a time in the 12-wave 128-column tile,
        // whose waves have 168 registers each, and two for fp32 inputs (three
        // split terms: four tiles' operands spill)
        constexpr int G = L::NW > 8 ? 1 : NS == 3 ? (TPW < 2 ? TPW : 2) : TPW < 4 ? TPW : 4;
        const __bf16 *qb = bQ(cb), *kb = bK(cb);
#pragma unroll
        for (int j0 = 0; j0 < TPW; j0 += G) {
            int sbv[G], ubv[G];
            bool live[G];
#pragma unroll
            for (int j = 0; j < G; ++j) {
                int tix = wi + NP * (j0 + j);
                live[j] = j0 + j < TPW && tix < NA;
                if (!live[j]) tix = 0;
                // tile index -> (Sb, Ub): tix = Ub (Ub + 1) / 2 + Sb
                int ub = 0;
#pragma unroll
                for (int q = 1; q < NU; ++q) ub += tix >= q * (q + 1) / 2 ? 1 : 0;
                ubv[j] = ub;
                sbv[j] = tix - ub * (ub + 1) / 2;
            }
            f32x4 acc[G];
#pragma unroll
            for (int j = 0; j < G; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
            bf16x8 A[KSI][G][NS], Bq[KSI][G][NS];
#pragma unroll
            for (int ks = 0; ks < KSI; ++ks) {
                const int i_lo = ks * 32 + 4 * lg, i_hi = i_lo + 16;
#pragma unroll
                for (int j = 0; j < G; ++j)
#pragma unroll
                    for (int n = 0; n < NS; ++n) {
                        const __bf16 *kr = kb + (n * C + sbv[j] * 16 + lc) * RS;
                        const __bf16 *qr = qb + (n * C + ubv[j] * 16 + lc) * RS;
                        const bf16x4 klo = *(const bf16x4 *)(kr + i_lo);
                        const bf16x4 qlo = *(const bf16x4 *)(qr + i_lo);
                        const bf16x4 khi = i_hi < DK ? *(const bf16x4 *)(kr + i_hi) : zero4();
                        const bf16x4 qhi = i_hi < DK ? *(const bf16x4 *)(qr + i_hi) : zero4();
                        A[ks][j][n] = cat(klo, khi);
                        Bq[ks][j][n] = cat(qlo, qhi);
                    }
            }
#pragma unroll
            for (int ks = 0; ks < KSI; ++ks) mma_split_n<NS, G>(A[ks], Bq[ks], acc);
#pragma unroll
            for (int j = 0; j < G; ++j) {
                if (!live[j]) continue;
                const int tix = ubv[j] * (ubv[j] + 1) / 2 + sbv[j];
                const bool diag = sbv[j] == ubv[j];
                float x[4];
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    x[r] = (diag && 4 * lg + r > lc) ? 0.f : acc[j][r];   // causal: s <= u
                unsigned w0[NS], w1[NS];
                split_pair<NS>(x[0], x[1], w0);
                split_pair<NS>(x[2], x[3], w1);
#pragma unroll
                for (int n = 0; n < NS; ++n)
                    *(uint2 *)(sA + ((tix * NS + n) * 64 + lane) * 4) = make_uint2(w0[n], w1[n]);
            }
        }
    };

    // Pipeline: in iteration it the producers prepare chunk it (LDS buffer
    // it & 1) while the consumers compute chunk it - 1 (LDS buffer
    // (it - 1) & 1).  Phase 1 (up to barrier A): producers issue the loads of
    // chunk it + 1, take the cumulative decay sums of chunk it and compute the
    // A^T tiles of chunk it - 1; consumers form S' and V' of chunk it - 1 and
    // update the state.  Phase 2 (up to barrier B): producers write the scaled
    // operands of chunk it; consumers compute and store the outputs of chunk
    // it - 1.  The two roles run separate loops with the same barrier sequence,
    // so each is register-allocated on its own.
    if (producer) {
        // the producers' operand preparation is the longer role of each chunk:
        // let their instructions issue first on the SIMDs they share with
        // consumers (measured ~2.5 % on the 130M layer)
        __builtin_amdgcn_s_setprio(2);
        // raw inputs of two chunks (the current one and the next, in flight):
        // a dk column pair, TPG consecutive tokens
        // (FU: q, k with HALO more rows before the group's first token)
        Raw2 rq[2][TPG + HALO], rk[2][TPG + HALO], rg[2][TPG], rt[2][TPG];
        auto load_dk = [&](int ch, auto rsel, bool valid) {
            constexpr int R = decltype(rsel)::value;
            const long long t0 = (long long)ch * C;
            const long long base = t0 * row_k;
            const long long lim = valid ? ((T - t0) * H - h) * DK * esz : 0;
            const __amdgpu_buffer_rsrc_t Rg = make_rsrc(gg + base, lim);
            const __amdgpu_buffer_rsrc_t Rt = make_rsrc(gt + base, lim);
            if constexpr (FU) {
                // window rows of the group: raw tokens t0 + cgp*TPG - HALO + i;
                // the resource starts at the chunk's first stored row, so rows
                // before the tensor's start have offsets that wrap to beyond its
                // range and read as zero
                const long long lx = valid ? ((Tx - t0) * H - h) * DK * esz : 0;
                const __amdgpu_buffer_rsrc_t Rk = make_rsrc(gk + base, lx);
                const __amdgpu_buffer_rsrc_t Rq = make_rsrc(gq + base, lx);
#pragma unroll
                for (int i = 0; i < TPG + HALO; ++i) {
                    const long long row = (long long)cgp * TPG + i - HALO + xshift;
                    const unsigned o = (unsigned)((row * row_k + c0) * esz);
                    rk[R][i] = PR::load(Rk, o);
                    if (outputs) rq[R][i] = PR::load(Rq, o);
                }
#pragma unroll
                for (int m = 0; m < TPG; ++m) {
                    const unsigned o = off_k + m * step_k;
                    rg[R][m] = PR::load(Rg, o);
                    rt[R][m] = PR::load(Rt, o);
                }
            } else {
                const __amdgpu_buffer_rsrc_t Rk = make_rsrc(gk + base, lim);
                const __amdgpu_buffer_rsrc_t Rq = make_rsrc(gq + base, lim);
#pragma unroll
                for (int m = 0; m < TPG; ++m) {
                    const unsigned o = off_k + m * step_k;
                    rg[R][m] = PR::load(Rg, o);
                    rt[R][m] = PR::load(Rt, o);
                    rk[R][m] = PR::load(Rk, o);
                    if (outputs) rq[R][m] = PR::load(Rq, o);
                }
            }
        };
        // FU: ShortConv taps of this thread's two columns, zero beyond conv_w
        float tq0[4], tq1[4], tk0[4], tk1[4];
        if constexpr (FU) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bool on = prep && j < conv_w && conv_w > 1;
                const size_t r0 = ((size_t)h * DK + c0) * conv_w + j, r1 = r0 + conv_w;
                tq0[j] = on && outputs ? a.cq[r0] : 0.f;
                tq1[j] = on && outputs ? a.cq[r1] : 0.f;
                tk0[j] = on ? a.ck[r0] : 0.f;
                tk1[j] = on ? a.ck[r1] : 0.f;
            }
        }
        // q and k of token m of the group (chunk ch, set R): the raw values, or
        // (FU, conv_w > 1) their convolution over the window, zero past the
        // sequence end so those tokens stay inert
        auto qk_at = [&](int ch, auto rsel, int m, float &q0, float &q1, float &k0, float &k1) {
            constexpr int R = decltype(rsel)::value;
            if constexpr (FU) {
                if (conv_w > 1) {
                    q0 = q1 = k0 = k1 = 0.f;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int i = m + HALO - j;
                        k0 = __builtin_fmaf(tk0[j], PR::lo(rk[R][i]), k0);
                        k1 = __builtin_fmaf(tk1[j], PR::hi(rk[R][i]), k1);
                        if (outputs) {
                            q0 = __builtin_fmaf(tq0[j], PR::lo(rq[R][i]), q0);
                            q1 = __builtin_fmaf(tq1[j], PR::hi(rq[R][i]), q1);
                        }
                    }
                    if ((long long)ch * C + cgp * TPG + m >= T) q0 = q1 = k0 = k1 = 0.f;
                } else {
                    q0 = PR::lo(rq[R][m + HALO]); q1 = PR::hi(rq[R][m + HALO]);
                    k0 = PR::lo(rk[R][m + HALO]); k1 = PR::hi(rk[R][m + HALO]);
                }
            } else {
                q0 = PR::lo(rq[R][m]); q1 = PR::hi(rq[R][m]);
                k0 = PR::lo(rk[R][m]); k1 = PR::hi(rk[R][m]);
            }
        };
        float gam_acc0 = 1.f, gam_acc1 = 1.f;           // products of chunk decays (mode 1)
        auto iter = [&](int it, auto rsel) {
            constexpr int R = decltype(rsel)::value;
            const bool work = prep && it < c_end;
            const int pb = it & 1;
            // the next chunk's inputs load during this whole iteration (past the
            // last chunk: empty buffer ranges, the loads return zeros)
            if (prep && it + 1 < c_end) load_dk(it + 1, std::integral_constant<int, 1 - R>(), true);
            // ---- phase 1: local cumulative sums of g * tau of both columns (nats)
            float cum0[TPG], cum1[TPG];
            if (work) {
                float run0 = 0.f, run1 = 0.f;
#pragma unroll
                for (int m = 0; m < TPG; ++m) {
                    run0 = PR::gt_lo(rg[R][m], rt[R][m], run0);
                    run1 = PR::gt_hi(rg[R][m], rt[R][m], run1);
                    cum0[m] = run0;
                    cum1[m] = run1;
                }
                *(float2 *)(sTot + cgp * DK + c0) = make_float2(run0, run1);
                if (MID / TPG == cgp)
                    *(float2 *)(sMid + c0) = make_float2(cum0[MID % TPG], cum1[MID % TPG]);
            }
            // A^T tiles of the previous chunk (its operands are complete since
            // the last barrier)
            if (outputs && it > c_begin) score_tiles(wave, (it - 1) & 1);
            __syncthreads();                               // barrier A
            // ---- phase 2: gates and scaled operands -> LDS buffer pb
            if (work) {
                float off0 = 0.f, off1 = 0.f, bm0 = 0.f, bm1 = 0.f, bL0 = 0.f, bL1 = 0.f;
#pragma unroll
                for (int gi = 0; gi < NG; ++gi) {
                    const float2 x = *(const float2 *)(sTot + gi * DK + c0);
                    if (gi < cgp) { off0 += x.x; off1 += x.y; }
                    if (gi < MID / TPG) { bm0 += x.x; bm1 += x.y; }
                    bL0 += x.x; bL1 += x.y;
                }
                const float2 mid = *(const float2 *)(sMid + c0);
                bm0 += mid.x; bm1 += mid.y;
                // to log2 units: b = -log2(e) * (sum of g * tau).  Kt is taken
                // relative to the reference token r: the midpoint m where it
                // also forms the score tiles, the chunk's last token L in the
                // transfer mode (every factor then at most 1, and the state
                // update needs no rescaling of the product)
                const float ref0 = outputs ? bm0 : bL0, ref1 = outputs ? bm1 : bL1;
                const float sh0 = (ref0 - off0) * kLog2e, sh1 = (ref1 - off1) * kLog2e;
                bm0 *= -kLog2e; bm1 *= -kLog2e;
                bL0 *= -kLog2e; bL1 *= -kLog2e;
                __bf16 *qb = bQ(pb), *kb = bK(pb);
#pragma unroll
                for (int m = 0; m < TPG; ++m) {
                    const int u = cgp * TPG + m;
                    const float d0 = __builtin_fmaf(cum0[m], -kLog2e, sh0);      // b_u - b_r
                    const float d1 = __builtin_fmaf(cum1[m], -kLog2e, sh1);
                    const float la0 = log2_gate_pow(PR::lo(rg[R][m]), PR::lo(rt[R][m]));
                    const float la1 = log2_gate_pow(PR::hi(rg[R][m]), PR::hi(rt[R][m]));
                    float qv0, qv1, kv0, kv1;
                    qk_at(it, rsel, m, qv0, qv1, kv0, kv1);
                    unsigned pk[NS];
                    split_pair<NS>(kv0 * __builtin_amdgcn_exp2f(la0 - d0),
                                   kv1 * __builtin_amdgcn_exp2f(la1 - d1), pk);
#pragma unroll
                    for (int n = 0; n < NS; ++n) *(unsigned *)(kb + (n * C + u) * RS + c0) = pk[n];
                    if (outputs) {
                        split_pair<NS>(qv0 * __builtin_amdgcn_exp2f(d0),
                                       qv1 * __builtin_amdgcn_exp2f(d1), pk);
#pragma unroll
                        for (int n = 0; n < NS; ++n) *(unsigned *)(qb + (n * C + u) * RS + c0) = pk[n];
                    }
                }
                if (cgp == 0) {
                    const float g0 = __builtin_amdgcn_exp2f(bL0), g1 = __builtin_amdgcn_exp2f(bL1);
                    *(float2 *)(bGam(pb) + c0) = make_float2(g0, g1);
                    if (outputs) {
                        *(float2 *)(bEm(pb) + c0) = make_float2(__builtin_amdgcn_exp2f(bm0),
                                                                __builtin_amdgcn_exp2f(bm1));
                        *(float2 *)(bGm(pb) + c0) = make_float2(__builtin_amdgcn_exp2f(bL0 - bm0),
                                                                __builtin_amdgcn_exp2f(bL1 - bm1));
                    }
                    gam_acc0 *= g0;
                    gam_acc1 *= g1;
                }
            }
            __syncthreads();                               // barrier B
        };
        if (prep && c_begin < c_end) load_dk(c_begin, std::integral_constant<int, 0>(), true);
        for (int it = c_begin; it <= c_end; it += 2) {
            iter(it, std::integral_constant<int, 0>());
            if (it + 1 <= c_end) iter(it + 1, std::integral_constant<int, 1>());
        }
        if (!outputs && a.gam_out && jt == 0 && prep && cgp == 0)
            *(float2 *)(a.gam_out + (size_t)bh * a.gam_bh + (size_t)seg * DK + c0) =
                make_float2(gam_acc0, gam_acc1);
        return;
    }

    // ================= consumers
    // this wave's v, beta_hat columns for one chunk, in MFMA B-operand order
    // bf16 inputs: 16-byte loads of whole [token][16 columns] rows (lane l:
    // token l/2 + 32 j, columns 8 (l & 1)..+7), staged per wave in LDS and read
    // back in B-operand order with the transposing read.  fp32 inputs: one
    // element per load, straight into B-operand order.
    constexpr bool kStage = NS == 2;
    constexpr int LV = C >= 32 ? C / 32 : 1;             // 16-byte loads per tensor
    // FU: v window rows X = 0 .. C + HALO - 1 (raw token t0 + X - HALO)
    constexpr int LVX = FU ? (C + HALO + 31) / 32 : LV;
    constexpr int NX = L::CONV && !kStage ? 4 : 1;       // fp32 ShortConv: taps read
    u32x4 rvw[LVX], rbw[LV];
    Raw rv[KSC][8], rb[KSC][8];
    // FU, fp32 inputs: the v rows of each 4-token run of this lane's tokens
    // (k-step p, half hh: tokens tb .. tb + 3, tb = 32 p + 16 hh + 4 lg) with
    // the NX - 1 rows before it; entry x is token tb + x - (NX - 1)
    constexpr int NXW = 4 + NX - 1;
    Raw rvx[FU ? KSC : 1][2][FU ? NXW : 1];
    __bf16 *stg = (__bf16 *)(smem + L::stg_off + (size_t)(producer ? 0 : cw) * L::stg_wave);
    __bf16 *stgb = stg + L::SV * 16;                     // staged beta_hat rows
    // FU: low-rank beta_hat.  The chunk's u rows as MFMA A operands (16-token
    // tile T16: lane row lc = token, k = rank index 4 lg.. and 16 + 4 lg..)
    // and this wave's 16 columns of w as the B operand.
    const bool lowrank = FU && a.u != nullptr;
    typedef typename std::conditional<NS == 2, uint2, u32x4>::type URaw;
    URaw ru[NU][2];
    bf16x8 wB[NS];
    if constexpr (FU) {
        if (lowrank && !producer) {
            float wv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int r = (e < 4 ? 0 : 16) + 4 * lg + (e & 3);
                wv[e] = r < a.rank
                    ? in_to_f32(((const Raw *)a.w)[((size_t)h * a.rank + r) * a.dv + jcol + lc]) : 0.f;
            }
            unsigned w4[4][NS];
#pragma unroll
            for (int e = 0; e < 4; ++e) split_pair<NS>(wv[2 * e], wv[2 * e + 1], w4[e]);
#pragma unroll
            for (int n = 0; n < NS; ++n) wB[n] = pack8(w4[0][n], w4[1][n], w4[2][n], w4[3][n]);
        }
    }
    // FU: the chunk's u rows (issued ahead of the output stores, so that the
    // wait for them in phase 2 does not also wait for those stores)
    auto load_u = [&](int ch) {
        if constexpr (FU) {
            const long long t0 = (long long)ch * C;
            const long long ru_row = H * (long long)a.rank;
            const __amdgpu_buffer_rsrc_t Ru = make_rsrc(
                (const Raw *)a.u + ((long long)b * T * H + h) * a.rank + t0 * ru_row,
                ((T - t0) * H - h) * (long long)a.rank * esz);
#pragma unroll
            for (int t16 = 0; t16 < NU; ++t16)
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const unsigned o = (unsigned)(((16 * t16 + lc) * ru_row + 16 * half + 4 * lg) * esz);
                    if constexpr (NS == 2) {
                        if (half == 0 || a.rank > 16)
                            ru[t16][half] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(Ru, o, 0, 0));
                        else
                            ru[t16][half] = uint2{0u, 0u};
                    } else {
                        if (half == 0 || a.rank > 16)
                            ru[t16][half] = __builtin_amdgcn_raw_buffer_load_b128(Ru, o, 0, 0);
                        else
                            ru[t16][half] = u32x4{0u, 0u, 0u, 0u};
                    }
                }
        }
    };
    auto load_v = [&](int ch, bool valid) {
        const long long t0 = (long long)ch * C;
        const long long base = t0 * row_v;
        const long long lim = valid ? ((T - t0) * H - h) * dv * esz - (long long)jcol * esz : 0;
        const __amdgpu_buffer_rsrc_t Rb = make_rsrc(gb + base, lim);
        if constexpr (FU) {
            const long long lx = valid ? ((Tx - t0) * H - h) * dv * esz - (long long)jcol * esz : 0;
            const __amdgpu_buffer_rsrc_t Rv = make_rsrc(gv + base, lx);
            if constexpr (kStage) {
#pragma unroll
                for (int j = 0; j < LVX; ++j) {
                    const int X = (lane >> 1) + 32 * j;
                    const long long row = (long long)X - HALO + xshift;
                    const unsigned o = (unsigned)((row * row_v + 8 * (lane & 1)) * esz);
                    rvw[j] = X < C + HALO ? __builtin_amdgcn_raw_buffer_load_b128(Rv, o, 0, 0)
                                          : u32x4{0u, 0u, 0u, 0u};
                }
#pragma unroll
                for (int j = 0; j < LV; ++j) {
                    const int u = (lane >> 1) + 32 * j;
                    const unsigned o = (unsigned)(((long long)u * row_v + 8 * (lane & 1)) * esz);
                    rbw[j] = u < C && !lowrank ? __builtin_amdgcn_raw_buffer_load_b128(Rb, o, 0, 0)
                                               : u32x4{0u, 0u, 0u, 0u};
                }
            } else {
#pragma unroll
                for (int p = 0; p < KSC; ++p)
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        const bool live = 32 * p + 16 * hh < C;
                        const int tb = 32 * p + 16 * hh + 4 * lg;
#pragma unroll
                        for (int x = 0; x < NXW; ++x) {
                            const long long row = (long long)tb + x - (NX - 1) + xshift;
                            const unsigned o = (unsigned)((row * row_v + lc) * esz);
                            rvx[p][hh][x] = live && (x >= NX - 1 || conv_w > 1) ? buf_load(Rv, o, Raw()) : Raw(0);
                        }
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const unsigned o = off_v + (p * 32 + 16 * hh + e) * step_v;
                            rb[p][4 * hh + e] = live && !lowrank ? buf_load(Rb, o, Raw()) : Raw(0);
                        }
                    }
            }
            return;
        }
        const __amdgpu_buffer_rsrc_t Rv = make_rsrc(gv + base, lim);
        if constexpr (kStage) {
#pragma unroll
            for (int j = 0; j < LV; ++j) {
                const int u = (lane >> 1) + 32 * j;
                const unsigned o = (unsigned)(((long long)u * row_v + 8 * (lane & 1)) * esz);
                if (u < C) {
                    rvw[j] = __builtin_amdgcn_raw_buffer_load_b128(Rv, o, 0, 0);
                    rbw[j] = __builtin_amdgcn_raw_buffer_load_b128(Rb, o, 0, 0);
                } else {
                    rvw[j] = u32x4{0u, 0u, 0u, 0u};
                    rbw[j] = u32x4{0u, 0u, 0u, 0u};
                }
            }
        } else {
#pragma unroll
            for (int p = 0; p < KSC; ++p)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int u = p * 32 + (e < 4 ? e : 12 + e);            // + 4*lg via off_v
                    if (u < C) {
                        const unsigned o = off_v + u * step_v;
                        rv[p][e] = buf_load(Rv, o, Raw());
                        rb[p][e] = buf_load(Rb, o, Raw());
                    } else {
                        rv[p][e] = Raw(0);
                        rb[p][e] = Raw(0);
                    }
                }
        }
    };
    if (c_begin < c_end) {
        if (lowrank) load_u(c_begin);
        load_v(c_begin, true);
    }

    // the block's output tile of chunk ch (staged in LDS by all consumer waves)
    // to HBM: each wave stores C / NJ whole rows of DVT floats with 16-byte
    // non-temporal stores; rows past the sequence end are dropped by the range
    float *sOut = (float *)(smem + L::out_off);
    auto store_tile = [&](int ch) {
        constexpr int LPR = DVT / 4;                     // lanes per row
        constexpr int RPI = 64 / LPR;                    // rows per store
        constexpr int RPW = C / NJ;                      // rows per consumer wave
        const long long t0 = (long long)ch * C;
        const long long lim = ((T - t0) * H - h) * dv * 4 - (long long)jt * DVT * 4;
        const __amdgpu_buffer_rsrc_t Ro = make_rsrc(go + t0 * row_v, lim);
        const int col = 4 * (lane % LPR);
#pragma unroll
        for (int j = 0; j < RPW / RPI; ++j) {
            const int u = cw * RPW + j * RPI + lane / LPR;
            const u32x4 x = *(const u32x4 *)(sOut + u * L::OS + col);
            __builtin_amdgcn_raw_buffer_store_b128(x, Ro, (unsigned)(((long long)u * row_v + col) * 4), 0, 2);
        }
    };

    // FU: ShortConv taps of this lane's v column (zero beyond conv_w), the
    // feedthrough weight of the column, and the chunk's v values in B-operand
    // order, kept from phase 1 for the feedthrough in phase 2
    float tv[4] = {0.f, 0.f, 0.f, 0.f}, dcol = 0.f;
    float vf[FU ? KSC : 1][8];
    if constexpr (FU) {
        if (conv_w > 1)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                tv[j] = j < conv_w ? a.cv[((size_t)h * a.dv + jcol + lc) * conv_w + j] : 0.f;
        if (a.dfeed) dcol = a.dfeed[(size_t)h * a.dv + jcol + lc];
    }
    // FU: low-rank beta_hat of the chunk whose u rows are in ru, formed in
    // phase 2 of the iteration that loads them (where the consumers would
    // otherwise wait at the barrier) and used in the next phase 1: z = u w,
    // one MFMA per 16-token tile (C-layout: token row 4 lg + e, column lc),
    // all tiles issued before the first sigmoid
    float blr[FU ? 2 * KSC : 1][4];
    auto lowrank_beta = [&]() {
        f32x4 z[2 * KSC];
#pragma unroll
        for (int t16 = 0; t16 < 2 * KSC; ++t16) {
            z[t16] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (t16 < NU) {
                bf16x8 uA[NS];
                if constexpr (NS == 2) {
                    uA[0] = pack8(ru[t16][0].x, ru[t16][0].y, ru[t16][1].x, ru[t16][1].y);
                    z[t16] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(uA[0], wB[0], z[t16], 0, 0, 0);
                } else {
                    unsigned s4[4][NS];
                    const u32x4 lo = ru[t16][0], hi2 = ru[t16][1];
                    split_pair<NS>(__uint_as_float(lo[0]), __uint_as_float(lo[1]), s4[0]);
                    split_pair<NS>(__uint_as_float(lo[2]), __uint_as_float(lo[3]), s4[1]);
                    split_pair<NS>(__uint_as_float(hi2[0]), __uint_as_float(hi2[1]), s4[2]);
                    split_pair<NS>(__uint_as_float(hi2[2]), __uint_as_float(hi2[3]), s4[3]);
#pragma unroll
                    for (int n = 0; n < NS; ++n) uA[n] = pack8(s4[0][n], s4[1][n], s4[2][n], s4[3][n]);
                    z[t16] = mma_split<NS>(uA, wB, z[t16]);
                }
            }
        }
#pragma unroll
        for (int t16 = 0; t16 < 2 * KSC; ++t16)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                blr[t16][e] = __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-kLog2e * z[t16][e]));
    };

    for (int it = c_begin; it <= c_end; ++it) {
        const bool cwork = it > c_begin;
        const int cb = (it - 1) & 1;

        // ================= phase 1: S' and V' operands, state update
        bf16x8 sB[KSI][NS];
        if (cwork && outputs) {
            // B operands S' = diag(exp(b_m)) S_in (k = dk rows)
            const float *em = bEm(cb);
#pragma unroll
            for (int ks = 0; ks < KSI; ++ks) {
                const int I0 = 2 * ks, I1 = 2 * ks + 1 < NI ? 2 * ks + 1 : 2 * ks;
                const f32x4 e0 = *(const f32x4 *)(em + I0 * 16 + 4 * lg);
                const f32x4 e1 = 2 * ks + 1 < NI ? *(const f32x4 *)(em + I1 * 16 + 4 * lg)
                                                 : f32x4{0.f, 0.f, 0.f, 0.f};
                unsigned w0[NS], w1[NS], w2[NS], w3[NS];
                split_pair<NS>(S[I0][0] * e0[0], S[I0][1] * e0[1], w0);
                split_pair<NS>(S[I0][2] * e0[2], S[I0][3] * e0[3], w1);
                split_pair<NS>(S[I1][0] * e1[0], S[I1][1] * e1[1], w2);
                split_pair<NS>(S[I1][2] * e1[2], S[I1][3] * e1[3], w3);
#pragma unroll
                for (int n = 0; n < NS; ++n) sB[ks][n] = pack8(w0[n], w1[n], w2[n], w3[n]);
            }
        }
        bf16x8 vB[KSC][NS];
        if (cwork) {
          if constexpr (FU) {
            // V' = beta_hat * v with the fused steps: v from the convolution
            // window (or raw), beta_hat from u w (or loaded); both in B-operand
            // order: element e of a k-step p is token 32 p + 16 (e / 4) + 4 lg
            // + e % 4 of this lane's column
            const int tcol = 4 * (lc & 3);
            const int tok0 = (it - 1) * C;                   // chunk's first token
            if constexpr (kStage) {
#pragma unroll
                for (int j = 0; j < LVX; ++j) {
                    const int X = (lane >> 1) + 32 * j;
                    if (X < L::SV) *(u32x4 *)(stg + X * 16 + 8 * (lane & 1)) = rvw[j];
                }
                if (!lowrank) {
#pragma unroll
                    for (int j = 0; j < LV; ++j) {
                        const int u = (lane >> 1) + 32 * j;
                        if (u < C) *(u32x4 *)(stgb + u * 16 + 8 * (lane & 1)) = rbw[j];
                    }
                }
            }
#pragma unroll
            for (int p = 0; p < KSC; ++p) {
                float vv[8], bb[8];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const bool live = 32 * p + 16 * hh < C;
                    const int tb = 32 * p + 16 * hh + 4 * lg;    // this lane's first token
                    if constexpr (kStage) {
                        const int rr = tb + (lc >> 2);            // row passed by this lane
                        if (conv_w > 1) {
                            const bf16x4 x0 = live ? lds_read_tr(stg + rr * 16 + tcol) : zero4();
                            const bf16x4 x1 = live ? lds_read_tr(stg + (rr + 4) * 16 + tcol) : zero4();
                            const float xs[8] = {(float)x0[0], (float)x0[1], (float)x0[2], (float)x0[3],
                                                 (float)x1[0], (float)x1[1], (float)x1[2], (float)x1[3]};
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                float acc = 0.f;
#pragma unroll
                                for (int j = 0; j < 4; ++j) acc = __builtin_fmaf(tv[j], xs[e + HALO - j], acc);
                                vv[4 * hh + e] = acc;
                            }
                        } else {
                            const bf16x4 x0 = live ? lds_read_tr(stg + (rr + HALO) * 16 + tcol) : zero4();
#pragma unroll
                            for (int e = 0; e < 4; ++e) vv[4 * hh + e] = (float)x0[e];
                        }
                        if (!lowrank) {
                            const bf16x4 b0 = live ? lds_read_tr(stgb + rr * 16 + tcol) : zero4();
#pragma unroll
                            for (int e = 0; e < 4; ++e) bb[4 * hh + e] = (float)b0[e];
                        }
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int ee = 4 * hh + e;
                            float acc = in_to_f32(rvx[p][hh][e + NX - 1]);
                            if (conv_w > 1) {
                                acc = 0.f;
#pragma unroll
                                for (int j = 0; j < NX; ++j)
                                    acc = __builtin_fmaf(tv[j], in_to_f32(rvx[p][hh][e - j + NX - 1]), acc);
                            }
                            vv[ee] = acc;
                            bb[ee] = in_to_f32(rb[p][ee]);
                        }
                    }
                    if (lowrank) {
                        // tile 2p + hh of this chunk's beta_hat, formed last phase 2
#pragma unroll
                        for (int e = 0; e < 4; ++e) bb[4 * hh + e] = blr[2 * p + hh][e];
                    }
                    // tokens past the sequence end stay inert (without the
                    // convolution their v rows already read as zero)
                    if constexpr (L::CONV) {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (tok0 + tb + e >= T) vv[4 * hh + e] = 0.f;
                    }
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) vf[p][e] = vv[e];
                unsigned w[4][NS];
#pragma unroll
                for (int e = 0; e < 4; ++e) split_pair<NS>(vv[2 * e] * bb[2 * e], vv[2 * e + 1] * bb[2 * e + 1], w[e]);
#pragma unroll
                for (int n = 0; n < NS; ++n) vB[p][n] = pack8(w[0][n], w[1][n], w[2][n], w[3][n]);
            }
          } else {
            // V' = beta_hat * v of this wave's columns, as split B operands (k = tokens)
            if constexpr (kStage) {
                // stage this wave's rows, then read them back token-major
#pragma unroll
                for (int j = 0; j < LV; ++j) {
                    const int u = (lane >> 1) + 32 * j;
                    if (u < C) {
                        *(u32x4 *)(stg + u * 16 + 8 * (lane & 1)) = rvw[j];
                        *(u32x4 *)(stg + C * 16 + u * 16 + 8 * (lane & 1)) = rbw[j];
                    }
                }
                const int trow = 4 * lg + (lc >> 2), tcol = 4 * (lc & 3);
#pragma unroll
                for (int p = 0; p < KSC; ++p) {
                    const int r0 = 32 * p + trow;
                    const bool hi = 32 * p + 16 < C;
                    const bf16x4 v0 = lds_read_tr(stg + r0 * 16 + tcol);
                    const bf16x4 b0 = lds_read_tr(stg + C * 16 + r0 * 16 + tcol);
                    const bf16x4 v1 = hi ? lds_read_tr(stg + (r0 + 16) * 16 + tcol) : zero4();
                    const bf16x4 b1 = hi ? lds_read_tr(stg + C * 16 + (r0 + 16) * 16 + tcol) : zero4();
                    unsigned w[4][NS];
                    split_pair<NS>((float)v0[0] * (float)b0[0], (float)v0[1] * (float)b0[1], w[0]);
                    split_pair<NS>((float)v0[2] * (float)b0[2], (float)v0[3] * (float)b0[3], w[1]);
                    split_pair<NS>((float)v1[0] * (float)b1[0], (float)v1[1] * (float)b1[1], w[2]);
                    split_pair<NS>((float)v1[2] * (float)b1[2], (float)v1[3] * (float)b1[3], w[3]);
#pragma unroll
                    for (int n = 0; n < NS; ++n) vB[p][n] = pack8(w[0][n], w[1][n], w[2][n], w[3][n]);
                }
            } else {
#pragma unroll
                for (int p = 0; p < KSC; ++p) {
                    unsigned w[4][NS];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        split_pair<NS>(in_to_f32(rb[p][2 * e]) * in_to_f32(rv[p][2 * e]),
                                       in_to_f32(rb[p][2 * e + 1]) * in_to_f32(rv[p][2 * e + 1]), w[e]);
#pragma unroll
                    for (int n = 0; n < NS; ++n) vB[p][n] = pack8(w[0][n], w[1][n], w[2][n], w[3][n]);
                }
            }
          }
            // outputs staged last iteration (issued after the wait for this
            // chunk's v loads, so that wait does not include these stores)
            if (lowrank && it < c_end) load_u(it);
            if (outputs && it - 2 >= c_begin) store_tile(it - 2);
            if (it < c_end) load_v(it, true);               // next chunk's v, beta_hat

            // dS = diag(exp(b_L - b_m)) Kt^T V' and S = diag(exp(b_L)) S + dS;
            // in the transfer mode Kt is relative to b_L, so the products
            // accumulate straight onto diag(exp(b_L)) S.  Kt^T is read with the
            // transposing LDS read (k = tokens).  The NI row tiles are
            // independent accumulators, issued interleaved.
            {
                const __bf16 *kb = bK(cb);
                const float *gam = bGam(cb), *gmv = bGm(cb);
                const int trow = 4 * lg + (lc >> 2), tcol = 4 * (lc & 3);
                f32x4 acc[NI];
#pragma unroll
                for (int I = 0; I < NI; ++I) {
                    if constexpr (OUT) {
                        acc[I] = f32x4{0.f, 0.f, 0.f, 0.f};
                    } else {
                        const f32x4 g0 = *(const f32x4 *)(gam + I * 16 + 4 * lg);
#pragma unroll
                        for (int r = 0; r < 4; ++r) acc[I][r] = g0[r] * S[I][r];
                    }
                }
                // row tiles in groups of IG (two groups for fp32 inputs at
                // dk = 128, where all operands at once spill ~36 registers)
                constexpr int IG = NS == 3 && NI > 4 ? NI / 2 : NI;
#pragma unroll
                for (int i0 = 0; i0 < NI; i0 += IG) {
                    bf16x8 A[KSC][IG][NS], Bv[KSC][IG][NS];
#pragma unroll
                    for (int ks = 0; ks < KSC; ++ks) {
                        const int s_lo = ks * 32 + trow, s_hi = s_lo + 16;
#pragma unroll
                        for (int I = 0; I < IG; ++I)
#pragma unroll
                            for (int n = 0; n < NS; ++n) {
                                const __bf16 *base = kb + n * C * RS + (i0 + I) * 16 + tcol;
                                const bf16x4 klo = lds_read_tr(base + s_lo * RS);
                                const bf16x4 khi = ks * 32 + 16 < C ? lds_read_tr(base + s_hi * RS) : zero4();
                                A[ks][I][n] = cat(klo, khi);
                                Bv[ks][I][n] = vB[ks][n];
                            }
                    }
#pragma unroll
                    for (int ks = 0; ks < KSC; ++ks) mma_split_n<NS, IG>(A[ks], Bv[ks], acc + i0);
                }
#pragma unroll
                for (int I = 0; I < NI; ++I) {
                    if constexpr (OUT) {
                        const f32x4 g0 = *(const f32x4 *)(gam + I * 16 + 4 * lg);
                        const f32x4 g1 = *(const f32x4 *)(gmv + I * 16 + 4 * lg);
#pragma unroll
                        for (int r = 0; r < 4; ++r) S[I][r] = __builtin_fmaf(g1[r], acc[I][r], g0[r] * S[I][r]);
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r) S[I][r] = acc[I][r];
                    }
                }
            }
        }
        __syncthreads();                                   // barrier A

        // ================= phase 2: outputs
        if (cwork) {
            if (outputs) {
                // O = A V' + Qt S' for this wave's columns; the NU token tiles
                // are independent accumulators, issued interleaved.
                const __bf16 *qb = bQ(cb);
                f32x4 acc[NU];
#pragma unroll
                for (int U = 0; U < NU; ++U) acc[U] = f32x4{0.f, 0.f, 0.f, 0.f};
                // inter-chunk: k = i, A = Qt rows, B = S'
                {
                    bf16x8 A[KSI][NU][NS], Bv[KSI][NU][NS];
#pragma unroll
                    for (int ks = 0; ks < KSI; ++ks) {
                        const int i_lo = ks * 32 + 4 * lg, i_hi = i_lo + 16;
#pragma unroll
                        for (int U = 0; U < NU; ++U)
#pragma unroll
                            for (int n = 0; n < NS; ++n) {
                                const __bf16 *qr = qb + (n * C + U * 16 + lc) * RS;
                                const bf16x4 qlo = *(const bf16x4 *)(qr + i_lo);
                                const bf16x4 qhi = i_hi < DK ? *(const bf16x4 *)(qr + i_hi) : zero4();
                                A[ks][U][n] = cat(qlo, qhi);
                                Bv[ks][U][n] = sB[ks][n];
                            }
                    }
#pragma unroll
                    for (int ks = 0; ks < KSI; ++ks) mma_split_n<NS, NU>(A[ks], Bv[ks], acc);
                }
                // intra-chunk: k = s over token blocks 2p, 2p+1 for the tiles U >= 2p
#pragma unroll
                for (int p = 0; p < KSC; ++p) {
                    constexpr int NUP = NU;             // tiles with U >= 2p, padded to NU
                    bf16x8 A[NUP][NS], Bv[NUP][NS];
#pragma unroll
                    for (int U = 0; U < NU; ++U) {
                        const bool live = 2 * p <= U;
                        const int t0x = U * (U + 1) / 2 + 2 * p;
                        const bool two = 2 * p + 1 <= U;
#pragma unroll
                        for (int n = 0; n < NS; ++n) {
                            if (live) {
                                const bf16x4 alo = *(const bf16x4 *)(sA + ((t0x * NS + n) * 64 + lane) * 4);
                                const bf16x4 ahi = two
                                    ? *(const bf16x4 *)(sA + (((t0x + 1) * NS + n) * 64 + lane) * 4) : zero4();
                                A[U][n] = cat(alo, ahi);
                                Bv[U][n] = vB[p][n];
                                if (!two)          // keep only the first 16 tokens of this k-step
                                    for (int e = 4; e < 8; ++e) Bv[U][n][e] = (__bf16)0.f;
                            }
                        }
                    }
                    // tiles U < 2p take no part in this k-step
                    if (p == 0) {
                        mma_split_n<NS, NU>(A, Bv, acc);
                    } else {
                        mma_split_n<NS, NU - 2>(A + 2, Bv + 2, acc + 2);
                    }
                }
                // FU: the loaded chunk's beta_hat while these products run
                if constexpr (FU) {
                    if (lowrank && it < c_end) lowrank_beta();
                }
                // FU: feedthrough o += d * v (C-layout rows 4 lg + r of token
                // tile U are elements 4 (U & 1) + r of k-step U / 2)
                if constexpr (FU) {
                    if (a.dfeed) {
#pragma unroll
                        for (int U = 0; U < NU; ++U)
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                acc[U][r] = __builtin_fmaf(dcol, vf[U / 2][4 * (U & 1) + r], acc[U][r]);
                    }
                }
                // into the block's output tile; stored to HBM as whole rows
                // after the next barrier
#pragma unroll
                for (int U = 0; U < NU; ++U)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        sOut[(U * 16 + 4 * lg + r) * L::OS + cw * 16 + lc] = acc[U][r];
            }
        }
        if constexpr (FU) {
            // the same where no outputs were formed this iteration (the first,
            // or the transfer mode)
            if (lowrank && it < c_end && !(cwork && outputs)) lowrank_beta();
        }
        __syncthreads();                                   // barrier B
    }

    if (outputs && c_end > c_begin) store_tile(c_end - 1);

    // ---- state out
    if (a.s_out && (!a.s_out_last_only || seg == a.n_seg - 1)) {
        float *so = a.s_out + bh * a.s_out_bh + seg * a.s_out_seg;
#pragma unroll
        for (int I = 0; I < NI; ++I)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                so[(size_t)(I * 16 + 4 * lg + r) * a.dv + jcol + lc] = S[I][r];
    }
}

template <int DK, int DVT, int C, typename TIn, bool OUT, int FU>
hipError_t launch_mode(const ChunkLaunch &Lc, hipStream_t stream)
{
    constexpr int NS = std::is_same<TIn, float>::value ? 3 : 2;
    typedef Cfg<DK, DVT, C, NS, OUT, FU> L;
    const size_t lds = L::bytes;
    static std::atomic<bool> lds_set[kMaxDevices];
    hipError_t e = set_lds_limit_once((const void *)chunk_fwd_kernel<DK, DVT, C, TIn, OUT, FU>, lds,
                                      lds_set);
    if (e != hipSuccess) return e;
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
    a.gam_out = Lc.gam_out; a.gam_bh = Lc.gam_bh_stride;
    a.u = Lc.fu.u; a.w = Lc.fu.w; a.rank = Lc.fu.rank; a.dfeed = Lc.fu.d;
    a.conv_w = FU ? Lc.fu.conv_w : 1;
    a.cq = Lc.fu.cq; a.ck = Lc.fu.ck; a.cv = Lc.fu.cv;
    const long long blocks = (long long)Lc.B * Lc.H * Lc.n_seg * a.n_jt;
    a.remap = (blocks % 8 == 0) ? 1 : 0;
    hipLaunchKernelGGL((chunk_fwd_kernel<DK, DVT, C, TIn, OUT, FU>), dim3((unsigned)blocks),
                       dim3(L::NT), lds, stream, a);
    return hipGetLastError();
}

// The tile shapes that are compiled (the size queries report 0 LDS bytes for
// the others, so they are never planned): the output-mode layout fits the
// CU's LDS, and the kernel fits its registers without spilling, which rules
// out 64-token chunks at dk = 128 and, with the fused steps on fp32 inputs
// (a load per ShortConv tap kept in registers), chunks beyond 16 tokens.  The
// 128-column tile (a whole head of dv = 128: 4 producer and 8 consumer waves,
// the gates' preparation done once per head) is compiled for bf16 inputs
// without the fused steps, dk <= 64 and chunks of 32 or 64 tokens.
template <int DK, int DVT, int C, int NS, int FU>
constexpr bool compiled_shape()
{
    return Cfg<DK, DVT, C, NS, true, FU>::bytes <= 160 * 1024 && !(DK == 128 && C == 64) &&
           !(FU && NS == 3 && C > 16) && (DVT < 128 || (NS == 2 && !FU && DK <= 64 && C >= 32));
}

template <int DK, int DVT, int C, typename TIn, int FU>
hipError_t launch_t(const ChunkLaunch &Lc, hipStream_t stream)
{
    constexpr int NS = std::is_same<TIn, float>::value ? 3 : 2;
    if constexpr (!compiled_shape<DK, DVT, C, NS, FU>()) {
        return hipErrorInvalidValue;
    } else {
        return Lc.mode == 0 ? launch_mode<DK, DVT, C, TIn, true, FU>(Lc, stream)
                            : launch_mode<DK, DVT, C, TIn, false, FU>(Lc, stream);
    }
}

// Instantiates every (DVT, C) tile shape for one dk, without the fused steps
// (XF 0), with all of them (1) or with those other than the ShortConv (2), and
// defines its size queries and launcher.
#define RODIMUS_CHUNK_CASE_LDS(XK, XV, XC, XF)                                        \
    if (dvt == XV && C == XC)                                                         \
        return f32 ? (chunk_detail::compiled_shape<XK, XV, XC, 3, XF>()               \
                          ? chunk_detail::Cfg<XK, XV, XC, 3, true, XF>::bytes : 0)    \
                   : (chunk_detail::compiled_shape<XK, XV, XC, 2, XF>()               \
                          ? chunk_detail::Cfg<XK, XV, XC, 2, true, XF>::bytes : 0);
#define RODIMUS_CHUNK_CASE_PCU(XK, XV, XC, XF)                                        \
    if (dvt == XV && C == XC)                                                         \
        return outputs ? (f32 ? chunk_detail::Cfg<XK, XV, XC, 3, true, XF>::per_cu    \
                              : chunk_detail::Cfg<XK, XV, XC, 2, true, XF>::per_cu)   \
                       : (f32 ? chunk_detail::Cfg<XK, XV, XC, 3, false, XF>::per_cu   \
                              : chunk_detail::Cfg<XK, XV, XC, 2, false, XF>::per_cu);
#define RODIMUS_CHUNK_CASE_LAUNCH(XK, XV, XC, XF)                                     \
    if (Lc.DVT == XV && Lc.C == XC)                                                   \
        return Lc.f32_inputs ? chunk_detail::launch_t<XK, XV, XC, float, XF>(Lc, stream) \
                             : chunk_detail::launch_t<XK, XV, XC, __bf16, XF>(Lc, stream);
#define RODIMUS_CHUNK_SHAPES(X, XK, XF)                                               \
    X(XK, 16, 16, XF) X(XK, 16, 32, XF) X(XK, 16, 64, XF)                             \
    X(XK, 32, 16, XF) X(XK, 32, 32, XF) X(XK, 32, 64, XF)                             \
    X(XK, 64, 16, XF) X(XK, 64, 32, XF) X(XK, 64, 64, XF)                             \
    X(XK, 128, 32, XF) X(XK, 128, 64, XF)
#define RODIMUS_DEFINE_CHUNK(XK, XF, NAME)                                            \
    size_t chunk_lds_bytes_##NAME(int dvt, int C, bool f32)                           \
    {                                                                                 \
        RODIMUS_CHUNK_SHAPES(RODIMUS_CHUNK_CASE_LDS, XK, XF)                          \
        return 0;                                                                     \
    }                                                                                 \
    int chunk_per_cu_##NAME(int dvt, int C, bool f32, bool outputs)                   \
    {                                                                                 \
        RODIMUS_CHUNK_SHAPES(RODIMUS_CHUNK_CASE_PCU, XK, XF)                          \
        return 1;                                                                     \
    }                                                                                 \
    hipError_t launch_chunk_##NAME(const ChunkLaunch &Lc, hipStream_t stream)         \
    {                                                                                 \
        RODIMUS_CHUNK_SHAPES(RODIMUS_CHUNK_CASE_LAUNCH, XK, XF)                       \
        return hipErrorInvalidValue;                                                  \
    }

}  // namespace chunk_detail
}  // namespace rodimus
