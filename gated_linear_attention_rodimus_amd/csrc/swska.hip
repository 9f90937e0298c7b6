// swska.hip -- sliding-window attention with one key shared by all heads
// (SW-SKA, Rodimus+'s second token mixer) on gfx950 MFMA.
//
// What it computes (summary page, "Approach"; digest page, "Method",
// Rodimus+ bullets: sliding-window attention whose keys are shared across
// heads; the rebuttal counts its projections as multi-head, multi-query and
// output, so q and v have a head each and k one for all): per batch b, head h
// and token t,
//     o[b,t,h] = sum_{t-W < s <= t} softmax_s(scale * q[b,t,h] . k[b,s]) v[b,s,h]
// with scale 1/sqrt(dk) by default.
//
// Workgroup: 4 waves, one (b, 128-query block, h); wave w owns queries
// q0 + 32 w .. + 31 as two 16-query column blocks.  Key tiles of 64 cover
// [q0 - W + 1, q0 + 127]; per tile,
//  - S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (K rows from LDS as A operands,
//    shared by the wave's two query blocks; the queries as B operands held in
//    registers): the C-layout of S^T (lane = query column, 4 consecutive keys
//    per lane) is directly the B operand of the next product, so the
//    probabilities never go through LDS;
//  - an online softmax in fp32 per query, exponentials as exp2; the running
//    maximum is raised only when a tile's maximum exceeds it by more than a
//    factor 2^8, so the outputs are rescaled rarely and every probability
//    stays below 256;
//  - O^T += V^T P^T, V^T read with the transposing LDS read once for both
//    query blocks, P split into two bf16 terms (hi + lo, ~16 bits) so the
//    product keeps fp32-level accuracy.
// The loop is software-pipelined by one tile: the score MFMAs of tile i+1 sit
// in the same block as the softmax of tile i (independent work that the
// scheduler interleaves, so the MFMA and VALU pipes run side by side), then
// come tile i's P V products.  K tiles and V tiles are double-buffered in LDS
// and filled by direct global-to-LDS loads (16 bytes a lane) issued one
// iteration ahead, which takes no registers or VALU work; each row's 16-byte
// pieces are stored XOR-permuted by the row index, which spreads the operand
// reads over all banks.  One workgroup barrier per tile.  Tiles that hold no
// key of a wave's queries' windows are skipped by that wave; the window mask
// runs only on tiles a window edge crosses.  Block ids put the heads of one
// query block on one XCD, so the shared key tile is read from HBM once and
// from that XCD's L2 by the other heads.
#include "chunk_kernel.h"

#include <math.h>

namespace rodimus {
namespace swska_detail {

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int NQ = 2;         // 16-query column blocks per wave
constexpr int QW = 16 * NQ;   // queries per wave
constexpr int NWV = 4;        // waves per workgroup
constexpr int QB = QW * NWV;  // queries per workgroup
constexpr int KB = 64;        // keys per tile
constexpr int NKT = KB / 16;  // 16-key blocks per tile
constexpr int LBW = 2;        // waves per SIMD the registers are sized for
constexpr int NT = 64 * NWV;  // threads per workgroup
constexpr float kLazy = 8.f;  // the running maximum moves when exceeded by more (log2 units)

template <int DK, int DV>
struct Cfg {
    static constexpr int KC = DK / 8;            // 16-byte pieces per K row
    static constexpr int VC = DV / 8;            // per V row
    static constexpr int k_bytes = KB * DK * 2;  // one K tile
    static constexpr int v_bytes = KB * DV * 2;  // one V tile
    static constexpr int bytes = 2 * (k_bytes + v_bytes);
    static constexpr int KLW = k_bytes / 1024 / NWV;   // 1 KB direct loads per wave per K tile
    static constexpr int VLW = v_bytes / 1024 / NWV;
    static_assert(KLW >= 1 && VLW >= 1, "tile too small for the workgroup's loads");
};

struct Args {
    int T, H, window;
    float scale_log2;            // scale * log2(e)
    const __bf16 *q, *k, *v;     // [B][T][H][dk], [B][T][dk], [B][T][H][dv]
    float *out;                  // [B][T][H][dv]
    int remap;                   // XCD-aware block order on/off
};

__device__ __forceinline__ bf16x8 cat(bf16x4 lo, bf16x4 hi) {
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// The chunk kernels' device helpers: the transposing LDS read, buffer
// resources, the packed bf16 dot product and the opaque SGPR constant.
using chunk_detail::dot2_bf16;
using chunk_detail::make_rsrc;
using chunk_detail::sgpr_const;
__device__ __forceinline__ bf16x4 lds_read_tr(const unsigned char *p) {
    return chunk_detail::lds_read_tr((const __bf16 *)p);
}

// Two fp32 values split into hi and lo bf16 pairs (round to nearest even);
// the residual x - hi is exact in fp32 and is formed by one packed dot
// product with (-1, 0) or (0, -1).
__device__ __forceinline__ void split2(float x0, float x1, unsigned &hi, unsigned &lo) {
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
    typedef float f2 __attribute__((ext_vector_type(2)));
    const f2 x = {x0, x1};
    hi = __builtin_bit_cast(unsigned, __builtin_convertvector(x, bf2));
    const f2 r = {dot2_bf16(hi, sgpr_const<0x0000bf80u>(), x0),
                  dot2_bf16(hi, sgpr_const<0xbf800000u>(), x1)};
    lo = __builtin_bit_cast(unsigned, __builtin_convertvector(r, bf2));
}

// Maximum / sum over the four 16-lane rows of the wave (lanes l, l ^ 16,
// l ^ 32, l ^ 48), by the row-swapping permutes.
__device__ __forceinline__ float rows_max(float x) {
    const unsigned u = __float_as_uint(x);
    auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const float y = __builtin_fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const unsigned w = __float_as_uint(y);
    auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
    return __builtin_fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows_sum(float x) {
    const unsigned u = __float_as_uint(x);
    auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const unsigned w = __float_as_uint(y);
    auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// S^T of one tile for the wave's two query blocks: s[j][kt] holds keys
// 16 kt + 4 lg .. +3 (rows) of query 16 j + lc (column).  K piece c of tile
// row r sits at LDS piece c ^ (r % KC); kbo is this lane's offset of row lc
// with the low two bits of its piece, kx = lc % KC.
template <int DK>
__device__ __forceinline__ void tile_scores(f32x4 (&s)[NQ][NKT], const unsigned char *kb,
                                            int kbo, int kx, const bf16x8 (&qB)[NQ][DK / 32])
{
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) {
        // piece 4 ks + lg of row lc at (4 ks + lg) ^ kx: the low two bits are in kbo
        const unsigned char *kp = kb + kbo + 64 * ((ks ^ (kx >> 2)) & (DK / 32 - 1));
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) {
            const bf16x8 A = *(const bf16x8 *)(kp + kt * 16 * DK * 2);
#pragma unroll
            for (int j = 0; j < NQ; ++j)
                s[j][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    A, qB[j][ks], ks == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : s[j][kt], 0, 0, 0);
        }
    }
}

// Online softmax of one tile (in place: scores -> probabilities); the split
// probabilities as the P V B-operands (ph/pl[k2][j]: keys 32 k2 + 4 lg .. +3,
// then 32 k2 + 16 + 4 lg .. +3); the per-lane partial row sums; and corr, the
// factor that rescales what was accumulated before (1 where the maximum did
// not move; resc is set where it moved).  With MASK, scores outside
// t - W < key <= t are dropped first (dq[j] = t minus this lane's first key
// of the tile).
template <bool MASK>
__device__ __forceinline__ void tile_softmax(f32x4 (&s)[NQ][NKT], float (&m)[NQ], float (&l)[NQ],
                                             float (&corr)[NQ], bool &resc,
                                             bf16x8 (&ph)[KB / 32][NQ], bf16x8 (&pl)[KB / 32][NQ],
                                             float c, const int (&dq)[NQ], unsigned W)
{
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
        if (MASK) {
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    s[j][kt][r] = (unsigned)(dq[j] - 16 * kt - r) < W ? s[j][kt][r] : -INFINITY;
        }
        float mloc = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) mloc = __builtin_fmaxf(mloc, s[j][kt][r]);
        const float mt = rows_max(mloc) * c;                 // log2 units
        const bool up = mt > m[j] + kLazy;                    // false while mt = -inf
        const float mnew = up ? mt : m[j];
        corr[j] = up ? __builtin_amdgcn_exp2f(m[j] - mnew) : 1.f;   // exp2(-inf) = 0 at the start
        resc = resc || up;
        m[j] = mnew;
        const float nm = mnew == -INFINITY ? 0.f : -mnew;
        float ps = 0.f;
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[j][kt][r], c, nm));
                s[j][kt][r] = p;
                ps += p;
            }
        l[j] = l[j] * corr[j] + ps;
#pragma unroll
        for (int k2 = 0; k2 < KB / 32; ++k2) {
            unsigned hh[4], ll[4];
            split2(s[j][2 * k2][0], s[j][2 * k2][1], hh[0], ll[0]);
            split2(s[j][2 * k2][2], s[j][2 * k2][3], hh[1], ll[1]);
            split2(s[j][2 * k2 + 1][0], s[j][2 * k2 + 1][1], hh[2], ll[2]);
            split2(s[j][2 * k2 + 1][2], s[j][2 * k2 + 1][3], hh[3], ll[3]);
            ph[k2][j] = __builtin_bit_cast(bf16x8, u32x4{hh[0], hh[1], hh[2], hh[3]});
            pl[k2][j] = __builtin_bit_cast(bf16x8, u32x4{ll[0], ll[1], ll[2], ll[3]});
        }
    }
}

template <int DK, int DV>
__global__ __launch_bounds__(NT, LBW) void swska_fwd_kernel(Args a)
{
    typedef Cfg<DK, DV> L;
    constexpr int KSQ = DK / 32;                 // MFMA k-steps over dk
    constexpr int NDV = DV / 16;                 // output tiles over dv
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    // LDS: K tiles in buffers 0, 1, then V tiles in buffers 0, 1
    auto kbuf = [&](int buf) { return smem + buf * L::k_bytes; };
    auto vbuf = [&](int buf) { return smem + 2 * L::k_bytes + buf * L::v_bytes; };

    // ---- block -> (b, query block, head); consecutive ids (the heads of one
    // query block) on one XCD
    const int nqb = (a.T + QB - 1) / QB;
    const int nblk = gridDim.x;
    int id = blockIdx.x;
    if (a.remap) id = (id % 8) * (nblk / 8) + id / 8;
    const int h = id % a.H;
    const int qb = (id / a.H) % nqb;
    const int b = id / a.H / nqb;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lc = lane & 15, lg = lane >> 4;
    const long long T = a.T, H = a.H;
    const int q0 = qb * QB;
    const int qw0 = q0 + QW * wave;              // the wave's first query
    const unsigned W = (unsigned)a.window;

    // keys of the block: [kstart, kend), in tiles of KB keys from kstart
    const int kstart = q0 - a.window + 1 > 0 ? q0 - a.window + 1 : 0;
    const int kend = q0 + QB < a.T ? q0 + QB : a.T;
    const int ntile = (kend - kstart + KB - 1) / KB;
    const __bf16 *kbase = a.k + (long long)b * T * DK;
    const __bf16 *vbase = a.v + ((long long)b * T * H + h) * DV;

    // Direct loads of a tile into LDS through buffer resources that start at
    // the tile's first row and end after row kend - 1 (loads past it read
    // zeros; those keys are masked).  The wave's j-th 1 KB block covers tile
    // rows blk * (64 / C) .. + 64 / C - 1 (C pieces of 16 bytes per row);
    // lane L fills piece L % C of row r = blk * (64 / C) + L / C with the
    // global piece (L % C) ^ (r % C).  A wave's blocks start at row 16 wave
    // (a multiple of C), so r % C = (j * (64 / C)) % C + L / C with no carry:
    // the piece is xk ^ ((j * (64 / C)) % C), xk = (L % C) ^ (L / C).
    const long long vstride = H * DV * 2;        // bytes between V rows
    const int xk = (lane % L::KC) ^ (lane / L::KC);
    const int xv = (lane % L::VC) ^ (lane / L::VC);
    const int yk = 16 * L::KC * (lane / L::KC);  // byte offset of the lane's row in a block
    const int yv = (int)((lane / L::VC) * vstride);
    auto load_k = [&](int t, int buf) {
        const int kt0 = kstart + t * KB;
        const __amdgpu_buffer_rsrc_t rs =
            make_rsrc(kbase + (long long)kt0 * DK, (long long)(kend - kt0) * DK * 2);
#pragma unroll
        for (int j = 0; j < L::KLW; ++j) {
            const int blk = wave * L::KLW + j;
            const int jp = (j * (64 / L::KC)) % L::KC;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(kbuf(buf) + blk * 1024), 16,
                                                     yk + 16 * (xk ^ jp), blk * 1024, 0, 0);
        }
    };
    auto load_v = [&](int t, int buf) {
        const int kt0 = kstart + t * KB;
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(vbase + (long long)kt0 * H * DV,
                                                    (long long)(kend - kt0 - 1) * vstride + DV * 2);
#pragma unroll
        for (int j = 0; j < L::VLW; ++j) {
            const int blk = wave * L::VLW + j;
            const int jp = (j * (64 / L::VC)) % L::VC;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(vbuf(buf) + blk * 1024), 16,
                                                     yv + 16 * (xv ^ jp),
                                                     (int)(blk * (64 / L::VC) * vstride), 0, 0);
        }
    };

    // this lane's queries; Q^T as B operands: column = query, k = dk 32 ks + 8 lg .. +7
    int tq[NQ];
    bool qvalid[NQ];
    bf16x8 qB[NQ][KSQ];
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
        tq[j] = qw0 + 16 * j + lc;
        qvalid[j] = tq[j] < a.T;
        const __bf16 *qp = a.q + (((long long)b * T + (qvalid[j] ? tq[j] : 0)) * H + h) * DK;
#pragma unroll
        for (int ks = 0; ks < KSQ; ++ks) {
            bf16x8 x = *(const bf16x8 *)(qp + 32 * ks + 8 * lg);
            if (!qvalid[j]) x = bf16x8{};
            qB[j][ks] = x;
        }
    }
    // LDS operand offsets: K row lc, piece 4 ks + lg; V^T rows 4 lg + lc / 4
    // (+ 16, + 32 k2), columns 16 dt + 4 (lc % 4) .. +3.  Pieces are XOR-ed
    // with the row's key; the XOR of the piece index's upper bits with the
    // key (ks and dt) is formed where the address is used (one instruction),
    // from two per-lane bases.
    const int kx = lc % L::KC;                   // K rows 16 kt + lc: key lc % KC
    const int vr = 4 * lg + (lc >> 2);           // V rows 32 k2 + 16 half + vr: key vr % VC
    const int vx = vr % L::VC;
    const int kbase_off = lc * DK * 2 + 16 * ((lg ^ kx) & 3);
    const int vbase_off = vr * DV * 2 + 16 * ((((lc & 3) >> 1) ^ vx) & 1) + 8 * (lc & 1);
    float m[NQ], l[NQ];                          // running maximum (log2 units), partial sums
    f32x4 o[NQ][NDV];
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
        m[j] = -INFINITY;
        l[j] = 0.f;
#pragma unroll
        for (int dt = 0; dt < NDV; ++dt) o[j][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // tiles holding no key of any of the wave's queries' windows are skipped
    auto active = [&](int t) {
        const int kt0 = kstart + t * KB;
        return t < ntile && kt0 <= qw0 + QW - 1 && kt0 + KB - 1 > qw0 - a.window && qw0 < a.T;
    };
    // tiles inside every window of the wave's queries need no mask
    auto inside = [&](int t) {
        const int kt0 = kstart + t * KB;
        return kt0 + KB - 1 <= qw0 && kt0 > qw0 + QW - 1 - a.window && kt0 + KB <= kend &&
               qw0 + QW - 1 < a.T;
    };

    f32x4 sc[NQ][NKT];
    if (ntile > 0) {
        load_k(0, 0);
        load_v(0, 0);
        if (ntile > 1) load_k(1, 1);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (active(0)) tile_scores<DK>(sc, kbuf(0), kbase_off, kx, qB);
    }
    for (int t = 0; t < ntile; ++t) {
        // K of tile t + 1 and V of tile t are in LDS; every wave is done with
        // tile t - 1 (and with tile 0's scores)
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        // per-iteration copies, so the address arithmetic is not hoisted out
        // of the loop into long-lived registers
        int kbo = kbase_off, vbo = vbase_off, kxi = kx, vxi = vx;
        asm volatile("" : "+v"(kbo), "+v"(vbo), "+v"(kxi), "+v"(vxi));
        if (t + 2 < ntile) load_k(t + 2, t & 1);
        if (t + 1 < ntile) load_v(t + 1, (t + 1) & 1);
        const bool ac = active(t), an = active(t + 1);
        f32x4 sn[NQ][NKT];
        const unsigned char *kn = kbuf((t + 1) & 1);
        if (ac) {
            int dq[NQ];
#pragma unroll
            for (int j = 0; j < NQ; ++j) dq[j] = tq[j] - (kstart + t * KB) - 4 * lg;
            float corr[NQ];
            bool resc = false;
            bf16x8 ph[KB / 32][NQ], pl[KB / 32][NQ];
            // the next tile's score MFMAs and this tile's softmax in one block
            const bool ins = inside(t);
            if (an && ins) {
                tile_scores<DK>(sn, kn, kbo, kxi, qB);
                tile_softmax<false>(sc, m, l, corr, resc, ph, pl, a.scale_log2, dq, W);
            } else if (an) {
                tile_scores<DK>(sn, kn, kbo, kxi, qB);
                tile_softmax<true>(sc, m, l, corr, resc, ph, pl, a.scale_log2, dq, W);
            } else if (ins) {
                tile_softmax<false>(sc, m, l, corr, resc, ph, pl, a.scale_log2, dq, W);
            } else {
                tile_softmax<true>(sc, m, l, corr, resc, ph, pl, a.scale_log2, dq, W);
            }
            if (__builtin_amdgcn_ballot_w64(resc) != 0) {
#pragma unroll
                for (int j = 0; j < NQ; ++j)
#pragma unroll
                    for (int dt = 0; dt < NDV; ++dt) o[j][dt] *= corr[j];
            }
            // ---- O^T += V^T P^T over the tile's two 32-key k-steps
            const unsigned char *vb = vbuf(t & 1);
#pragma unroll
            for (int k2 = 0; k2 < KB / 32; ++k2) {
#pragma unroll
                for (int dt = 0; dt < NDV; ++dt) {
                    // piece 2 dt + e of row vr at (2 dt + e) ^ vx: bit 0 is in vbo
                    const unsigned char *vp = vb + vbo + 32 * ((dt ^ (vxi >> 1)) & (NDV - 1));
                    const bf16x4 vlo = lds_read_tr(vp + (32 * k2) * DV * 2);
                    const bf16x4 vhi = lds_read_tr(vp + (32 * k2 + 16) * DV * 2);
                    const bf16x8 A = cat(vlo, vhi);
#pragma unroll
                    for (int j = 0; j < NQ; ++j)
                        o[j][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, pl[k2][j], o[j][dt], 0, 0, 0);
#pragma unroll
                    for (int j = 0; j < NQ; ++j)
                        o[j][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, ph[k2][j], o[j][dt], 0, 0, 0);
                }
            }
        } else if (an) {
            tile_scores<DK>(sn, kn, kbo, kxi, qB);
        }
#pragma unroll
        for (int j = 0; j < NQ; ++j)
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt) sc[j][kt] = sn[j][kt];
    }

    // ---- o / l: lane holds dv 16 dt + 4 lg .. +3 of query tq[j]
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
        const float lt = rows_sum(l[j]);
        if (qvalid[j]) {
            const float inv = lt > 0.f ? 1.f / lt : 0.f;
            float *op = a.out + (((long long)b * T + tq[j]) * H + h) * DV;
#pragma unroll
            for (int dt = 0; dt < NDV; ++dt)
                __builtin_nontemporal_store(o[j][dt] * inv, (f32x4 *)(op + 16 * dt + 4 * lg));
        }
    }
}

template <int DK, int DV>
hipError_t launch_typed(int B, int T, int H, int window, float scale, const void *q,
                        const void *k, const void *v, float *out, hipStream_t stream)
{
    typedef Cfg<DK, DV> L;
    static std::atomic<bool> lds_set[kMaxDevices];
    hipError_t e = set_lds_limit_once((const void *)swska_fwd_kernel<DK, DV>, L::bytes, lds_set);
    if (e != hipSuccess) return e;
    Args a;
    a.T = T; a.H = H; a.window = window;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.q = (const __bf16 *)q; a.k = (const __bf16 *)k; a.v = (const __bf16 *)v;
    a.out = out;
    const long long blocks = (long long)B * ((T + QB - 1) / QB) * H;
    a.remap = blocks % 8 == 0 ? 1 : 0;
    hipLaunchKernelGGL((swska_fwd_kernel<DK, DV>), dim3((unsigned)blocks), dim3(NT), L::bytes,
                       stream, a);
    return hipGetLastError();
}

}  // namespace swska_detail

hipError_t launch_swska(int B, int T, int H, int dk, int dv, int window, float scale,
                        const void *q, const void *k, const void *v, float *out,
                        hipStream_t stream)
{
    using namespace swska_detail;
#define RODIMUS_SWSKA_DV(DK)                                                                   \
    switch (dv) {                                                                              \
    case 64: return launch_typed<DK, 64>(B, T, H, window, scale, q, k, v, out, stream);        \
    case 128: return launch_typed<DK, 128>(B, T, H, window, scale, q, k, v, out, stream);      \
    }                                                                                          \
    break;
    switch (dk) {
    case 64: RODIMUS_SWSKA_DV(64)
    case 128: RODIMUS_SWSKA_DV(128)
    }
#undef RODIMUS_SWSKA_DV
    return hipErrorInvalidValue;
}

}  // namespace rodimus
