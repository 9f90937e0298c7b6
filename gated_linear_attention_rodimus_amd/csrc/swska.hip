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
//  - an online softmax in fp32 per query (running maximum and sum, the
//    output rescaled when the maximum moves), exponentials as exp2;
//  - O^T += V^T P^T, V^T read with the transposing LDS read once for both
//    query blocks, P split into two bf16 terms (hi + lo, ~16 bits) so the
//    product keeps fp32-level accuracy.
// K and V tiles are double-buffered in LDS: the next tile's rows are loaded
// into registers while the current one is used, and written to the other
// buffer before the one barrier per tile.  Tiles that no window edge of a
// wave's queries crosses skip the mask, tiles wholly outside them are
// skipped by that wave, and the outputs are rescaled only when some query's
// maximum moved.  Block ids put the heads of one query block on one XCD, so
// the shared key tile is read from HBM once and from that XCD's L2 by the
// other heads.
#include "internal.h"

#include <math.h>

namespace rodimus {
namespace swska_detail {

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int NQ = 2;         // 16-query column blocks per wave
constexpr int QW = 16 * NQ;   // queries per wave
constexpr int NWV = 4;        // waves per workgroup
constexpr int QB = QW * NWV;  // queries per workgroup
constexpr int KB = 64;        // keys per tile
constexpr int NKT = KB / 16;  // 16-key blocks per tile
constexpr int LBW = 2;        // workgroups per CU the registers are sized for
constexpr int NT = 64 * NWV;  // threads per workgroup

template <int DK, int DV>
struct Cfg {
    static constexpr int KS = DK + 8;     // K row stride in LDS (bf16)
    static constexpr int VS = DV + 8;     // V row stride
    static constexpr size_t k_bytes = (size_t)KB * KS * 2;
    static constexpr size_t buf = k_bytes + (size_t)KB * VS * 2;   // one K + V tile
    static constexpr size_t bytes = 2 * buf;
    static constexpr int KL = KB * DK / 8 / NT;   // 16-byte K loads per thread per tile
    static constexpr int VL = KB * DV / 8 / NT;   // 16-byte V loads per thread per tile
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

// Transposed LDS read (ds_read_b64_tr_b16): within each 16-lane group, lane m
// passes the address of 4 consecutive 16-bit values (row m/4, columns
// 4*(m%4)..+3 of a 4 x 16 block); lane i receives column i, rows 0..3.
__device__ __forceinline__ bf16x4 lds_read_tr(const __bf16 *p) {
    typedef short v4s __attribute__((ext_vector_type(4)));
    v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4s *)(const_cast<__bf16 *>(p)));
    return __builtin_bit_cast(bf16x4, r);
}

// Two fp32 values split into hi and lo bf16 pairs (round to nearest even;
// the residual x - hi is exact in fp32).
__device__ __forceinline__ void split2(float x0, float x1, unsigned &hi, unsigned &lo) {
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
    typedef float f2 __attribute__((ext_vector_type(2)));
    const f2 x = {x0, x1};
    const bf2 h = __builtin_convertvector(x, bf2);
    const f2 hf = __builtin_convertvector(h, f2);
    const f2 r = x - hf;
    hi = __builtin_bit_cast(unsigned, h);
    lo = __builtin_bit_cast(unsigned, __builtin_convertvector(r, bf2));
}

template <int DK, int DV>
__global__ __launch_bounds__(NT, LBW) void swska_fwd_kernel(Args a)
{
    typedef Cfg<DK, DV> L;
    constexpr int KSQ = DK / 32;                 // MFMA k-steps over dk
    constexpr int NDV = DV / 16;                 // output tiles over dv
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    auto sK = [&](int buf) { return (__bf16 *)(smem + buf * L::buf); };
    auto sV = [&](int buf) { return (__bf16 *)(smem + buf * L::buf + L::k_bytes); };

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
    int tq[NQ];                                  // this lane's queries
    bool qvalid[NQ];
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
        tq[j] = qw0 + 16 * j + lc;
        qvalid[j] = tq[j] < a.T;
    }

    // Q^T as B operands: column = query tq[j], k = dk {32 ks + 4 lg .. +3, 32 ks + 16 + 4 lg .. +3}
    bf16x8 qB[NQ][KSQ];
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
        const __bf16 *qp = a.q + (((long long)b * T + (qvalid[j] ? tq[j] : 0)) * H + h) * DK;
#pragma unroll
        for (int ks = 0; ks < KSQ; ++ks) {
            bf16x4 lo = *(const bf16x4 *)(qp + 32 * ks + 4 * lg);
            bf16x4 hi = *(const bf16x4 *)(qp + 32 * ks + 16 + 4 * lg);
            if (!qvalid[j]) {
#pragma unroll
                for (int e = 0; e < 4; ++e) lo[e] = hi[e] = (__bf16)0.f;
            }
            qB[j][ks] = cat(lo, hi);
        }
    }

    // keys of the block: [kstart, kend)
    const int kstart = q0 - a.window + 1 > 0 ? q0 - a.window + 1 : 0;
    const int kend = q0 + QB < a.T ? q0 + QB : a.T;
    const __bf16 *kbase = a.k + (long long)b * T * DK;
    const __bf16 *vbase = a.v + ((long long)b * T * H + h) * DV;

    // a tile's K and V rows into registers (rows past kend: zero), and from
    // there into an LDS buffer
    u32x4 rk[L::KL], rv[L::VL];
    auto load_tile = [&](int kt0) {
#pragma unroll
        for (int j = 0; j < L::KL; ++j) {
            const int c = tid + NT * j;                    // 16-byte piece
            const int r = c / (DK / 8), col = (c % (DK / 8)) * 8;
            rk[j] = kt0 + r < kend ? *(const u32x4 *)(kbase + (long long)(kt0 + r) * DK + col)
                                   : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int j = 0; j < L::VL; ++j) {
            const int c = tid + NT * j;
            const int r = c / (DV / 8), col = (c % (DV / 8)) * 8;
            rv[j] = kt0 + r < kend ? *(const u32x4 *)(vbase + (long long)(kt0 + r) * H * DV + col)
                                   : u32x4{0u, 0u, 0u, 0u};
        }
    };
    auto stage_tile = [&](int buf) {
        __bf16 *k_ = sK(buf), *v_ = sV(buf);
#pragma unroll
        for (int j = 0; j < L::KL; ++j) {
            const int c = tid + NT * j;
            const int r = c / (DK / 8), col = (c % (DK / 8)) * 8;
            *(u32x4 *)(k_ + r * L::KS + col) = rk[j];
        }
#pragma unroll
        for (int j = 0; j < L::VL; ++j) {
            const int c = tid + NT * j;
            const int r = c / (DV / 8), col = (c % (DV / 8)) * 8;
            *(u32x4 *)(v_ + r * L::VS + col) = rv[j];
        }
    };

    float m[NQ], l[NQ];                         // running maximum (log2 units), sum
    f32x4 o[NQ][NDV];
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
        m[j] = -INFINITY;
        l[j] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < NQ; ++j)
#pragma unroll
        for (int dt = 0; dt < NDV; ++dt) o[j][dt] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (kstart < kend) {
        load_tile(kstart);
        stage_tile(0);
    }
    __syncthreads();
    int it = 0;
    for (int kt0 = kstart; kt0 < kend; kt0 += KB, ++it) {
        const int cb = it & 1;
        const bool more = kt0 + KB < kend;
        if (more) load_tile(kt0 + KB);                 // in flight during this tile

        // tiles holding no key of any of the wave's queries' windows are skipped
        const bool active = kt0 <= qw0 + QW - 1 && kt0 + KB - 1 > qw0 - a.window && qw0 < a.T;
        if (active) {
            const __bf16 *k_ = sK(cb), *v_ = sV(cb);
            // ---- S^T = K Q^T for the tile's 4 key blocks of 16, both query blocks
            f32x4 s[NQ][NKT];
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt) {
#pragma unroll
                for (int j = 0; j < NQ; ++j) s[j][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
                const __bf16 *kr = k_ + (16 * kt + lc) * L::KS;
#pragma unroll
                for (int ks = 0; ks < KSQ; ++ks) {
                    const bf16x8 A = cat(*(const bf16x4 *)(kr + 32 * ks + 4 * lg),
                                         *(const bf16x4 *)(kr + 32 * ks + 16 + 4 * lg));
#pragma unroll
                    for (int j = 0; j < NQ; ++j)
                        s[j][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, qB[j][ks], s[j][kt], 0, 0, 0);
                }
            }
            // ---- window mask (only on tiles that cross a window edge of the
            // wave's queries), online softmax per query; scores stay unscaled
            // (the scale is positive) until the exponent s * scale - m
            const bool inside = kt0 + KB - 1 <= qw0 && kt0 > qw0 + QW - 1 - a.window &&
                                kt0 + KB <= kend && qw0 + QW - 1 < a.T;
            float corr[NQ];
            bool moved = false;
#pragma unroll
            for (int j = 0; j < NQ; ++j) {
                float mloc = -INFINITY;
                if (inside) {
#pragma unroll
                    for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
                        for (int r = 0; r < 4; ++r) mloc = fmaxf(mloc, s[j][kt][r]);
                } else {
#pragma unroll
                    for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int key = kt0 + 16 * kt + 4 * lg + r;
                            const bool ok = qvalid[j] && key < kend && key <= tq[j] && key > tq[j] - a.window;
                            s[j][kt][r] = ok ? s[j][kt][r] : -INFINITY;
                            mloc = fmaxf(mloc, s[j][kt][r]);
                        }
                }
                mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
                mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
                const float mnew = fmaxf(m[j], mloc * a.scale_log2);     // log2 units
                const bool any = mnew != -INFINITY;
                corr[j] = (any && m[j] != -INFINITY) ? __builtin_amdgcn_exp2f(m[j] - mnew) : (any ? 0.f : 1.f);
                float psum = 0.f;
                const float nm = any ? -mnew : 0.f;
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[j][kt][r], a.scale_log2, nm));
                        s[j][kt][r] = p;
                        psum += p;
                    }
                psum += __shfl_xor(psum, 16);
                psum += __shfl_xor(psum, 32);
                l[j] = l[j] * corr[j] + psum;
                m[j] = mnew;
                moved = moved || corr[j] != 1.f;
            }
            // rescale the outputs only when some query's maximum moved
            if (__builtin_amdgcn_ballot_w64(moved) != 0) {
#pragma unroll
                for (int j = 0; j < NQ; ++j)
#pragma unroll
                    for (int dt = 0; dt < NDV; ++dt) o[j][dt] *= corr[j];
            }

            // ---- O^T += V^T P^T over the tile's two 32-key k-steps
#pragma unroll
            for (int k2 = 0; k2 < KB / 32; ++k2) {
                bf16x8 pH[NQ], pL[NQ];
#pragma unroll
                for (int j = 0; j < NQ; ++j) {
                    unsigned h01, l01, h23, l23, h45, l45, h67, l67;
                    split2(s[j][2 * k2][0], s[j][2 * k2][1], h01, l01);
                    split2(s[j][2 * k2][2], s[j][2 * k2][3], h23, l23);
                    split2(s[j][2 * k2 + 1][0], s[j][2 * k2 + 1][1], h45, l45);
                    split2(s[j][2 * k2 + 1][2], s[j][2 * k2 + 1][3], h67, l67);
                    pH[j] = __builtin_bit_cast(bf16x8, u32x4{h01, h23, h45, h67});
                    pL[j] = __builtin_bit_cast(bf16x8, u32x4{l01, l23, l45, l67});
                }
                const int row = 32 * k2 + 4 * lg + (lc >> 2), col = 4 * (lc & 3);
#pragma unroll
                for (int dt = 0; dt < NDV; ++dt) {
                    const bf16x4 vlo = lds_read_tr(v_ + row * L::VS + 16 * dt + col);
                    const bf16x4 vhi = lds_read_tr(v_ + (row + 16) * L::VS + 16 * dt + col);
                    const bf16x8 A = cat(vlo, vhi);
#pragma unroll
                    for (int j = 0; j < NQ; ++j)
                        o[j][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, pL[j], o[j][dt], 0, 0, 0);
#pragma unroll
                    for (int j = 0; j < NQ; ++j)
                        o[j][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, pH[j], o[j][dt], 0, 0, 0);
                }
            }
        }
        // the next tile into the other buffer (its last readers finished
        // before the previous barrier), then one barrier
        if (more) stage_tile(cb ^ 1);
        __syncthreads();
    }

    // ---- o / l: lane holds dv 16 dt + 4 lg .. +3 of query tq[j]
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
        if (qvalid[j]) {
            const float inv = l[j] > 0.f ? 1.f / l[j] : 0.f;
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
