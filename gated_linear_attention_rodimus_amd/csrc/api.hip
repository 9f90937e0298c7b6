// api.hip -- the extern "C" boundary: argument validation, execution plan,
// dispatch.  Every check runs on the host before any HIP call; nothing here
// allocates device memory.
#include "../../include/rodimus_ddts.h"
#include "internal.h"

#include <stdint.h>

#include <math.h>
#include <mutex>

using namespace rodimus;

// Scratch of rodimus_ddts_chunk_fwd_static_scratch: one array per device
// (each device that loads the library holds its own copy until the process
// ends).  In host code the name `scratch` is only a host-side stand-in: the
// device address is looked up once per device with hipGetSymbolAddress (with
// that device current) and kept in scratch_addr, and only that address is
// passed to kernels.
static __device__ __align__(256) unsigned char scratch[RODIMUS_STATIC_SCRATCH_BYTES];

namespace {

constexpr size_t kLdsLimit = 160 * 1024;   // LDS per CU on gfx950
constexpr int kTargetBlocks = 256;         // compute units on MI355X

bool width_ok(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

struct Span {
    uintptr_t lo, hi;   // [lo, hi)
};

Span span(const void *p, size_t bytes) { return {(uintptr_t)p, (uintptr_t)p + bytes}; }

bool overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi && a.hi > a.lo && b.hi > b.lo; }

// Pick chunk length, dv tile, segment count and transfer pieces.  Returns
// false if no instantiated tile shape fits the LDS.
//  - chunk: the longest of 64/32/16 that is <= the requested one and fits;
//  - dv tile: min(dv, 64) columns (4 consumer waves at 64, so the dk-side
//    gate work is shared by as many columns as possible);
//  - segments (when the caller passes 0): one sweep while the (b, h, tile)
//    units fill more than half the CUs, else pieces of >= 8 chunks, as many
//    as run at once, on the whole-head 128-column tile where it is compiled
//    (the gate work then done once per head; measured: long prefill 584 ->
//    505 us, 1.6B layer 143 -> 135 us), otherwise with 32-token chunks where
//    those kernels hold two workgroups per CU;
//  - transfer pieces per segment: below.
bool make_plan(int B, int T, int H, int dk, int dv, int chunk, int segments, bool f32,
               ChunkPlan *P, bool fused = false)
{
    const int chunks_try[3] = {64, 32, 16};
    P->Ct = 0;
    bool found = false;
    for (int ci = 0; ci < 3 && !found; ++ci) {
        const int C = chunks_try[ci];
        if (chunk != 0 && C > chunk) continue;
        // shapes that are not compiled report 0 bytes
        const size_t lds = chunk_lds_bytes(dk, dv < 64 ? dv : 64, C, f32, fused);
        if (lds == 0 || lds > kLdsLimit) continue;
        P->C = C;
        found = true;
    }
    if (!found) return false;
    const long long heads = (long long)B * H;
    int dvt = dv < 64 ? dv : 64;
    long long units = heads * (dv / dvt);
    int seg = segments;
    if (seg == 0) {
        seg = 1;
        // few units and long sequences: the whole-head tile at the longest
        // chunk it has, when segments of >= 8 chunks, as many as run at once,
        // fill the CUs
        if (units <= kTargetBlocks / 2 && dv == 128) {
            for (int ci = 0; ci < 3; ++ci) {
                const int C = chunks_try[ci];
                if (chunk != 0 && C > chunk) continue;
                const size_t lds = chunk_lds_bytes(dk, 128, C, f32, fused);
                if (lds == 0 || lds > kLdsLimit) continue;
                const long long nch = T > 0 ? (T + C - 1) / C : 0;
                const long long want = (long long)kTargetBlocks * chunk_per_cu(dk, 128, C, f32, true, fused) / heads;
                if (want >= 2 && nch / 8 >= want) {
                    P->C = C;
                    dvt = 128;
                    units = heads;
                    seg = (int)want;
                    // transfers in half-length chunks where that kernel holds
                    // two workgroups per CU (measured: long prefill, transfer
                    // pass 177 -> 160 us)
                    if (C == 64 && chunk_per_cu(dk, 128, 32, f32, false, fused) == 2 &&
                        chunk_lds_bytes(dk, 128, 32, f32, fused) != 0)
                        P->Ct = 32;
                }
                break;
            }
        }
        // one sweep per (b, h, dv tile) while that fills more than half the
        // CUs; at half or fewer, split the sequences into segments of at least
        // 8 chunks, as many as run at once.  Chunks of 32 tokens are taken
        // there when that kernel holds two workgroups per CU (twice the
        // segments; measured: long prefill, 16 heads x 2 tiles, 16 segments
        // of C = 32 584 us against 8 of C = 64 630 us; 1.6B layer, 64 heads x
        // 2 tiles, 4 of C = 32 142 us against 2 of C = 64 151 us)
        if (dvt != 128 && units <= kTargetBlocks / 2) {
            int Cs = P->C;
            if (P->C > 32 && chunk_per_cu(dk, dvt, 32, f32, true, fused) == 2 &&
                chunk_lds_bytes(dk, dvt, 32, f32, fused) != 0)
                Cs = 32;
            const long long nch = T > 0 ? (T + Cs - 1) / Cs : 0;
            if (nch >= 16) {
                long long want = (long long)kTargetBlocks * chunk_per_cu(dk, dvt, Cs, f32, true, fused) / units;
                long long cap = nch / 8;
                seg = (int)(want < cap ? want : cap);
                if (seg < 1) seg = 1;
                if (seg > 1) P->C = Cs;
            }
        }
    }
    P->n_chunks = T > 0 ? (T + P->C - 1) / P->C : 0;
    P->DVT = dvt;
    P->lds_bytes = chunk_lds_bytes(dk, dvt, P->C, f32, fused);
    if (P->lds_bytes == 0 || P->lds_bytes > kLdsLimit) return false;
    if (seg > P->n_chunks) seg = P->n_chunks > 0 ? P->n_chunks : 1;
    if (seg < 1) seg = 1;
    P->chunks_per_seg = P->n_chunks > 0 ? (P->n_chunks + seg - 1) / seg : 0;
    // drop empty trailing segments
    if (P->chunks_per_seg > 0) seg = (P->n_chunks + P->chunks_per_seg - 1) / P->chunks_per_seg;
    P->segments = seg;
    if (P->Ct == 0 || seg == 1) P->Ct = P->C;
    // the transfers cover the segments before the last (the output pass of
    // the last one writes S_T from its true incoming state); each is cut into
    // 2 pieces where they all still run at once (measured: 1.6B layer, 64
    // heads x 2 tiles x 2 segments of C = 64, 180 -> 153 us), and into 4
    // pieces of at least 8 chunks where the CUs hold that many transfer
    // workgroups
    const long long xfer_cap = (long long)kTargetBlocks * chunk_per_cu(dk, dvt, P->Ct, f32, false, fused);
    const int cps_t = P->chunks_per_seg * (P->C / P->Ct);             // transfer chunks per segment
    P->tr_per_seg = 1;
    if (seg > 1 && cps_t % 2 == 0 && units * (seg - 1) * 2 <= xfer_cap) P->tr_per_seg = 2;
    if (seg > 1 && cps_t % 4 == 0 && cps_t / 4 >= 8 && units * (seg - 1) * 4 <= xfer_cap)
        P->tr_per_seg = 4;
    const int tr = (seg - 1) * P->tr_per_seg;
    P->ws_slots = seg > tr ? seg : tr;
    P->ws_bytes = seg > 1 ? (size_t)B * H * P->ws_slots * ((size_t)dk * dv + dk) * sizeof(float) : 0;
    return true;
}

rodimus_status check_chunk_args(int B, int T, int H, int dk, int dv, int chunk, int segments,
                                rodimus_dtype dt)
{
    if (B <= 0 || H <= 0 || T < 0 || segments < 0) return RODIMUS_ERR_INVALID_ARG;
    if (dt != RODIMUS_DTYPE_F32 && dt != RODIMUS_DTYPE_BF16) return RODIMUS_ERR_UNSUPPORTED;
    if (!width_ok(dk) || !width_ok(dv)) return RODIMUS_ERR_UNSUPPORTED;
    if (chunk != 0 && chunk != 16 && chunk != 32 && chunk != 64) return RODIMUS_ERR_UNSUPPORTED;
    // index arithmetic inside the kernels is 64-bit; keep the token count in int
    if ((long long)B * T > (1LL << 31) - 1) return RODIMUS_ERR_INVALID_ARG;
    // per-chunk byte offsets inside the kernels are 32-bit
    if ((long long)H * 128 * 4 * 64 > (1LL << 31) - 1) return RODIMUS_ERR_INVALID_ARG;
    return RODIMUS_OK;
}

}  // namespace

extern "C" {

int rodimus_abi_version(void) { return RODIMUS_ABI_VERSION; }

const char *rodimus_status_string(rodimus_status s)
{
    switch (s) {
    case RODIMUS_OK: return "ok";
    case RODIMUS_ERR_INVALID_ARG: return "invalid argument";
    case RODIMUS_ERR_UNSUPPORTED: return "unsupported shape, chunk or dtype";
    case RODIMUS_ERR_WORKSPACE: return "workspace missing or too small";
    case RODIMUS_ERR_HIP: return "HIP runtime error";
    default: break;
    }
    return "unknown status";
}

rodimus_status rodimus_ddts_chunk_fwd_plan(int B, int T, int H, int dk, int dv, int chunk,
                                           int segments, rodimus_dtype in_dtype,
                                           rodimus_chunk_plan *plan)
{
    if (!plan) return RODIMUS_ERR_INVALID_ARG;
    rodimus_status st = check_chunk_args(B, T, H, dk, dv, chunk, segments, in_dtype);
    if (st != RODIMUS_OK) return st;
    ChunkPlan P;
    if (!make_plan(B, T, H, dk, dv, chunk, segments, in_dtype == RODIMUS_DTYPE_F32, &P))
        return RODIMUS_ERR_UNSUPPORTED;
    plan->chunk = P.C;
    plan->dv_tile = P.DVT;
    plan->segments = P.segments;
    plan->transfer_pieces = P.segments > 1 ? P.tr_per_seg : 0;
    plan->workspace_bytes = P.ws_bytes;
    return RODIMUS_OK;
}

size_t rodimus_ddts_chunk_fwd_ex_workspace_bytes(int B, int T, int H, int dk, int dv, int chunk,
                                                 int segments)
{
    // dtype only changes the tile choice; report the larger of the two
    size_t best = 0;
    for (int f = 0; f < 2; ++f) {
        if (check_chunk_args(B, T, H, dk, dv, chunk, segments,
                             f ? RODIMUS_DTYPE_F32 : RODIMUS_DTYPE_BF16) != RODIMUS_OK)
            return 0;
        ChunkPlan P;
        if (make_plan(B, T, H, dk, dv, chunk, segments, f != 0, &P) && P.ws_bytes > best)
            best = P.ws_bytes;
    }
    return best;
}

size_t rodimus_ddts_chunk_fwd_workspace_bytes(int B, int T, int H, int dk, int dv, int chunk)
{
    return rodimus_ddts_chunk_fwd_ex_workspace_bytes(B, T, H, dk, dv, chunk, 0);
}

}  // extern "C"

namespace {

// Every host-side check of a forward call (sizes, dtype, pointers,
// alignment, overlaps) and its plan.  With check_ws, also the workspace
// (size, alignment, overlaps); without, the caller supplies scratch that no
// tensor can overlap.  No HIP call.
// The fused-step descriptor's own checks (sizes, pointers); fills the spans of
// its tensors.  No HIP call.
rodimus_status check_fused(const rodimus_fused *f, int B, int T, int H, int dk, int dv,
                           size_t esz, Span *spans)
{
    if (!f) return RODIMUS_ERR_INVALID_ARG;
    if (f->conv_width < 1 || f->conv_width > 4) return RODIMUS_ERR_UNSUPPORTED;
    if (f->u && f->rank != 16 && f->rank != 32) return RODIMUS_ERR_UNSUPPORTED;
    const size_t ntok = (size_t)B * T * H;
    for (int i = 0; i < 6; ++i) spans[i] = Span{0, 0};
    if (f->u) {
        if (!f->w || !aligned16(f->u) || !aligned16(f->w)) return RODIMUS_ERR_INVALID_ARG;
        spans[0] = span(f->u, ntok * f->rank * esz);
        spans[1] = span(f->w, (size_t)H * f->rank * dv * esz);
    }
    if (f->d) {
        if (!aligned16(f->d)) return RODIMUS_ERR_INVALID_ARG;
        spans[2] = span(f->d, (size_t)H * dv * sizeof(float));
    }
    if (f->conv_width > 1) {
        const float *c[3] = {f->conv_q, f->conv_k, f->conv_v};
        for (const float *p : c)
            if (!p || !aligned16(p)) return RODIMUS_ERR_INVALID_ARG;
        spans[3] = span(f->conv_q, (size_t)H * dk * f->conv_width * sizeof(float));
        spans[4] = span(f->conv_k, (size_t)H * dk * f->conv_width * sizeof(float));
        spans[5] = span(f->conv_v, (size_t)H * dv * f->conv_width * sizeof(float));
    }
    return RODIMUS_OK;
}

rodimus_status chunk_fwd_check(
    int B, int T, int H, int dk, int dv, int chunk, int segments, rodimus_dtype in_dtype,
    const void *q, const void *k, const void *g, const void *tau,
    const void *v, const void *beta_hat,
    const float *initial_state, const float *out, const float *final_state,
    bool check_ws, const void *workspace, size_t workspace_bytes, ChunkPlan *P,
    const rodimus_fused *fu = nullptr)
{
    rodimus_status st = check_chunk_args(B, T, H, dk, dv, chunk, segments, in_dtype);
    if (st != RODIMUS_OK) return st;
    const bool f32 = in_dtype == RODIMUS_DTYPE_F32;
    const size_t esz = f32 ? 4 : 2;
    const size_t ntok = (size_t)B * T * H;
    const size_t state_bytes = (size_t)B * H * dk * dv * sizeof(float);
    // q, k, v carry the ShortConv's history rows
    const int cwid = fu ? fu->conv_width : 1;
    const size_t ntok_x = (size_t)B * (T + cwid - 1) * H;
    Span s_fu[6] = {};
    if (fu) {
        st = check_fused(fu, B, T, H, dk, dv, esz, s_fu);
        if (st != RODIMUS_OK) return st;
    }
    const bool dense_beta = !fu || !fu->u;

    if (T > 0) {
        const void *ins[6] = {q, k, g, tau, v, beta_hat};
        for (int i = 0; i < 6; ++i) {
            if (i == 5 && !dense_beta) continue;
            if (!ins[i] || !aligned16(ins[i])) return RODIMUS_ERR_INVALID_ARG;
        }
        if (!out || !aligned16(out)) return RODIMUS_ERR_INVALID_ARG;
    }
    if (initial_state && !aligned16(initial_state)) return RODIMUS_ERR_INVALID_ARG;
    if (final_state && !aligned16(final_state)) return RODIMUS_ERR_INVALID_ARG;

    // aliasing: out may overlap nothing; final_state may equal initial_state
    const Span s_in[12] = {span(q, ntok_x * dk * esz), span(k, ntok_x * dk * esz),
                           span(g, ntok * dk * esz), span(tau, ntok * dk * esz),
                           span(v, ntok_x * dv * esz),
                           span(beta_hat, dense_beta ? ntok * dv * esz : 0),
                           s_fu[0], s_fu[1], s_fu[2], s_fu[3], s_fu[4], s_fu[5]};
    const Span s_out = span(out, ntok * dv * sizeof(float));
    const Span s_s0 = span(initial_state, initial_state ? state_bytes : 0);
    const Span s_sf = span(final_state, final_state ? state_bytes : 0);
    if (T > 0) {
        for (const Span &x : s_in)
            if (overlap(s_out, x)) return RODIMUS_ERR_INVALID_ARG;
        if (overlap(s_out, s_s0) || overlap(s_out, s_sf)) return RODIMUS_ERR_INVALID_ARG;
    }
    if (final_state) {
        if (T > 0)
            for (const Span &x : s_in)
                if (overlap(s_sf, x)) return RODIMUS_ERR_INVALID_ARG;
        if (initial_state && final_state != initial_state && overlap(s_sf, s_s0))
            return RODIMUS_ERR_INVALID_ARG;
    }

    if (!make_plan(B, T, H, dk, dv, chunk, segments, f32, P, fu != nullptr))
        return RODIMUS_ERR_UNSUPPORTED;
    if (check_ws && P->ws_bytes > 0) {
        if (!workspace || workspace_bytes < P->ws_bytes) return RODIMUS_ERR_WORKSPACE;
        if (!aligned16(workspace)) return RODIMUS_ERR_INVALID_ARG;
        const Span s_ws = span(workspace, P->ws_bytes);
        for (const Span &x : s_in)
            if (overlap(s_ws, x)) return RODIMUS_ERR_INVALID_ARG;
        if (overlap(s_ws, s_out) || overlap(s_ws, s_s0) || overlap(s_ws, s_sf))
            return RODIMUS_ERR_INVALID_ARG;
    }
    return RODIMUS_OK;
}

// Tracing aid: the calling host thread's pass events (rodimus_trace_forward_events).
thread_local hipEvent_t *trace_ev = nullptr;

hipError_t trace(int i, hipStream_t stream)
{
    return trace_ev ? hipEventRecord(trace_ev[i], stream) : hipSuccess;
}

// The launches of a checked forward call; `workspace` holds at least
// P.ws_bytes bytes when P.segments > 1.
rodimus_status chunk_fwd_launch(
    const ChunkPlan &P, int B, int T, int H, int dk, int dv, rodimus_dtype in_dtype,
    const void *q, const void *k, const void *g, const void *tau,
    const void *v, const void *beta_hat,
    const float *initial_state, float *out, float *final_state,
    void *workspace, hipStream_t stream, const rodimus_fused *fu = nullptr)
{
    hipError_t e = hipSuccess;
    if (T == 0) {
        if (final_state && final_state != initial_state)
            e = launch_state_copy(initial_state, final_state, (size_t)B * H * dk * dv, stream);
        return e == hipSuccess ? RODIMUS_OK : RODIMUS_ERR_HIP;
    }
    ChunkLaunch Lc;
    Lc.B = B; Lc.T = T; Lc.H = H; Lc.dk = dk; Lc.dv = dv;
    Lc.C = P.C; Lc.DVT = P.DVT; Lc.chunks_per_seg = P.chunks_per_seg;
    Lc.f32_inputs = in_dtype == RODIMUS_DTYPE_F32;
    Lc.in = TokenInputs{q, k, g, tau, v, beta_hat};
    Lc.gam_out = nullptr;
    Lc.gam_bh_stride = 0;
    if (fu) {
        Lc.fused = true;
        Lc.fu.u = fu->u; Lc.fu.w = fu->w; Lc.fu.rank = fu->rank; Lc.fu.d = fu->d;
        Lc.fu.conv_w = fu->conv_width;
        Lc.fu.cq = fu->conv_q; Lc.fu.ck = fu->conv_k; Lc.fu.cv = fu->conv_v;
    }
    const long long sz = (long long)dk * dv;
    if (P.segments == 1) {
        Lc.n_seg = 1; Lc.mode = 0;
        Lc.s_in = initial_state; Lc.s_in_bh_stride = sz; Lc.s_in_seg_stride = 0;
        Lc.out = out;
        Lc.s_out = final_state; Lc.s_out_bh_stride = sz; Lc.s_out_seg_stride = 0;
        Lc.s_out_last_only = 0;
        if (trace(0, stream) != hipSuccess) return RODIMUS_ERR_HIP;
        e = launch_chunk(Lc, stream);
        if (e == hipSuccess) e = trace(1, stream);
        return e == hipSuccess ? RODIMUS_OK : RODIMUS_ERR_HIP;
    }
    // segmented: (1) transfers from a zero state over the chunks before the
    // last segment, tr_per_seg pieces per segment, (2) ordered combination into
    // each segment's incoming state, (3) outputs (the last segment's also
    // writes S_T).
    const int n_seg = P.segments, per = P.tr_per_seg, slots = P.ws_slots;
    float *ws_ds = (float *)workspace;                                // [BH][slots][dk][dv]
    float *ws_gam = ws_ds + (size_t)B * H * slots * dk * dv;          // [BH][slots][dk]
    Lc.n_seg = (n_seg - 1) * per; Lc.mode = 1;
    Lc.C = P.Ct; Lc.chunks_per_seg = P.chunks_per_seg * (P.C / P.Ct) / per;
    Lc.s_in = nullptr; Lc.s_in_bh_stride = 0; Lc.s_in_seg_stride = 0;
    Lc.out = nullptr;
    Lc.s_out = ws_ds; Lc.s_out_bh_stride = (long long)slots * sz; Lc.s_out_seg_stride = sz;
    Lc.s_out_last_only = 0;
    Lc.gam_out = ws_gam; Lc.gam_bh_stride = (long long)slots * dk;
    if (trace(0, stream) != hipSuccess) return RODIMUS_ERR_HIP;
    e = launch_chunk(Lc, stream);
    if (e == hipSuccess) e = trace(1, stream);
    if (e != hipSuccess) return RODIMUS_ERR_HIP;
    e = launch_segment_combine(B * H, n_seg, per, slots, dk, dv, initial_state, ws_ds, ws_gam, stream);
    if (e == hipSuccess) e = trace(2, stream);
    if (e != hipSuccess) return RODIMUS_ERR_HIP;
    Lc.n_seg = n_seg; Lc.C = P.C; Lc.chunks_per_seg = P.chunks_per_seg; Lc.mode = 0;
    Lc.s_in = ws_ds; Lc.s_in_bh_stride = (long long)slots * sz; Lc.s_in_seg_stride = sz;
    Lc.out = out;
    Lc.s_out = final_state; Lc.s_out_bh_stride = sz; Lc.s_out_seg_stride = 0;
    Lc.s_out_last_only = 1;
    Lc.gam_out = nullptr;
    e = launch_chunk(Lc, stream);
    if (e == hipSuccess) e = trace(3, stream);
    return e == hipSuccess ? RODIMUS_OK : RODIMUS_ERR_HIP;
}

// ---------------------------------------------------------------- static scratch
std::mutex scratch_mu;
void *scratch_addr[kMaxDevices] = {};

// The current device's address of `scratch`, looked up on the first call on
// that device.
hipError_t scratch_ptr(void **p)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_addr[dev]) {
        void *a = nullptr;
        e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        scratch_addr[dev] = a;
    }
    *p = scratch_addr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

rodimus_status rodimus_trace_forward_events(hipEvent_t *events, int count)
{
    if (count == 0) {
        trace_ev = nullptr;
        return RODIMUS_OK;
    }
    if (count != 4 || !events) return RODIMUS_ERR_INVALID_ARG;
    trace_ev = events;
    return RODIMUS_OK;
}

rodimus_status rodimus_ddts_chunk_fwd_ex(
    int B, int T, int H, int dk, int dv, int chunk, int segments, rodimus_dtype in_dtype,
    const void *q, const void *k, const void *g, const void *tau,
    const void *v, const void *beta_hat,
    const float *initial_state, float *out, float *final_state,
    void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    ChunkPlan P;
    rodimus_status st = chunk_fwd_check(B, T, H, dk, dv, chunk, segments, in_dtype, q, k, g, tau,
                                        v, beta_hat, initial_state, out, final_state, true,
                                        workspace, workspace_bytes, &P);
    if (st != RODIMUS_OK) return st;
    return chunk_fwd_launch(P, B, T, H, dk, dv, in_dtype, q, k, g, tau, v, beta_hat,
                            initial_state, out, final_state, workspace, stream);
}

rodimus_status rodimus_ddts_chunk_fwd_fused(
    int B, int T, int H, int dk, int dv, int chunk, int segments, rodimus_dtype in_dtype,
    const void *q, const void *k, const void *g, const void *tau,
    const void *v, const void *beta_hat, const rodimus_fused *fused,
    const float *initial_state, float *out, float *final_state,
    void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    ChunkPlan P;
    rodimus_status st = chunk_fwd_check(B, T, H, dk, dv, chunk, segments, in_dtype, q, k, g, tau,
                                        v, beta_hat, initial_state, out, final_state, true,
                                        workspace, workspace_bytes, &P, fused);
    if (st != RODIMUS_OK) return st;
    return chunk_fwd_launch(P, B, T, H, dk, dv, in_dtype, q, k, g, tau, v, beta_hat,
                            initial_state, out, final_state, workspace, stream, fused);
}

size_t rodimus_ddts_chunk_fwd_fused_workspace_bytes(int B, int T, int H, int dk, int dv,
                                                    int chunk, int segments)
{
    size_t best = 0;
    for (int f = 0; f < 2; ++f) {
        if (check_chunk_args(B, T, H, dk, dv, chunk, segments,
                             f ? RODIMUS_DTYPE_F32 : RODIMUS_DTYPE_BF16) != RODIMUS_OK)
            return 0;
        ChunkPlan P;
        if (make_plan(B, T, H, dk, dv, chunk, segments, f != 0, &P, true) && P.ws_bytes > best)
            best = P.ws_bytes;
    }
    return best;
}

rodimus_status rodimus_ddts_chunk_fwd_static_scratch(
    int B, int T, int H, int dk, int dv, int chunk, int segments, rodimus_dtype in_dtype,
    const void *q, const void *k, const void *g, const void *tau,
    const void *v, const void *beta_hat,
    const float *initial_state, float *out, float *final_state, hipStream_t stream)
{
    ChunkPlan P;
    rodimus_status st = chunk_fwd_check(B, T, H, dk, dv, chunk, segments, in_dtype, q, k, g, tau,
                                        v, beta_hat, initial_state, out, final_state, false,
                                        nullptr, 0, &P);
    if (st != RODIMUS_OK) return st;
    if (P.ws_bytes > RODIMUS_STATIC_SCRATCH_BYTES) return RODIMUS_ERR_WORKSPACE;
    void *ws = nullptr;
    if (T > 0 && P.segments > 1 && scratch_ptr(&ws) != hipSuccess) return RODIMUS_ERR_HIP;
    return chunk_fwd_launch(P, B, T, H, dk, dv, in_dtype, q, k, g, tau, v, beta_hat,
                            initial_state, out, final_state, ws, stream);
}

rodimus_status rodimus_ddts_chunk_fwd(
    int B, int T, int H, int dk, int dv, int chunk, rodimus_dtype in_dtype,
    const void *q, const void *k, const void *g, const void *tau,
    const void *v, const void *beta_hat,
    const float *initial_state, float *out, float *final_state,
    void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    return rodimus_ddts_chunk_fwd_ex(B, T, H, dk, dv, chunk, 0, in_dtype, q, k, g, tau, v, beta_hat,
                                     initial_state, out, final_state, workspace, workspace_bytes,
                                     stream);
}

rodimus_status rodimus_ddts_decode_step(
    int N, int H, int dk, int dv, rodimus_dtype in_dtype,
    const void *q, const void *k, const void *g, const void *tau,
    const void *v, const void *beta_hat,
    float *state, float *out, hipStream_t stream)
{
    if (N <= 0 || H <= 0) return RODIMUS_ERR_INVALID_ARG;
    if (in_dtype != RODIMUS_DTYPE_F32 && in_dtype != RODIMUS_DTYPE_BF16) return RODIMUS_ERR_UNSUPPORTED;
    if (!width_ok(dk) || !width_ok(dv)) return RODIMUS_ERR_UNSUPPORTED;
    if ((long long)N * H > (1LL << 31) - 1) return RODIMUS_ERR_INVALID_ARG;
    const void *ins[6] = {q, k, g, tau, v, beta_hat};
    for (const void *p : ins)
        if (!p || !aligned16(p)) return RODIMUS_ERR_INVALID_ARG;
    if (!state || !out || !aligned16(state) || !aligned16(out)) return RODIMUS_ERR_INVALID_ARG;
    const size_t esz = in_dtype == RODIMUS_DTYPE_F32 ? 4 : 2;
    const size_t pairs = (size_t)N * H;
    const Span s_st = span(state, pairs * dk * dv * sizeof(float));
    const Span s_o = span(out, pairs * dv * sizeof(float));
    const Span s_in[6] = {span(q, pairs * dk * esz), span(k, pairs * dk * esz),
                          span(g, pairs * dk * esz), span(tau, pairs * dk * esz),
                          span(v, pairs * dv * esz), span(beta_hat, pairs * dv * esz)};
    if (overlap(s_st, s_o)) return RODIMUS_ERR_INVALID_ARG;
    for (const Span &x : s_in)
        if (overlap(s_st, x) || overlap(s_o, x)) return RODIMUS_ERR_INVALID_ARG;
    hipError_t e = launch_decode(N, H, dk, dv, in_dtype == RODIMUS_DTYPE_F32,
                                 TokenInputs{q, k, g, tau, v, beta_hat}, state, out, stream);
    return e == hipSuccess ? RODIMUS_OK : RODIMUS_ERR_HIP;
}

rodimus_status rodimus_ddts_decode_step_fused(
    int N, int H, int dk, int dv, rodimus_dtype in_dtype,
    const void *q, const void *k, const void *g, const void *tau,
    const void *v, const void *beta_hat, const rodimus_fused *fused,
    float *state, float *out, hipStream_t stream)
{
    if (N <= 0 || H <= 0) return RODIMUS_ERR_INVALID_ARG;
    if (in_dtype != RODIMUS_DTYPE_F32 && in_dtype != RODIMUS_DTYPE_BF16) return RODIMUS_ERR_UNSUPPORTED;
    if (!width_ok(dk) || !width_ok(dv)) return RODIMUS_ERR_UNSUPPORTED;
    if ((long long)N * H > (1LL << 31) - 1) return RODIMUS_ERR_INVALID_ARG;
    const size_t esz = in_dtype == RODIMUS_DTYPE_F32 ? 4 : 2;
    Span s_fu[6] = {};
    rodimus_status st = check_fused(fused, N, 1, H, dk, dv, esz, s_fu);
    if (st != RODIMUS_OK) return st;
    const bool dense_beta = !fused->u;
    const void *ins[6] = {q, k, g, tau, v, beta_hat};
    for (int i = 0; i < 6; ++i) {
        if (i == 5 && !dense_beta) continue;
        if (!ins[i] || !aligned16(ins[i])) return RODIMUS_ERR_INVALID_ARG;
    }
    if (!state || !out || !aligned16(state) || !aligned16(out)) return RODIMUS_ERR_INVALID_ARG;
    const size_t pairs = (size_t)N * H, W = (size_t)fused->conv_width;
    const Span s_st = span(state, pairs * dk * dv * sizeof(float));
    const Span s_o = span(out, pairs * dv * sizeof(float));
    const Span s_in[12] = {span(q, W * pairs * dk * esz), span(k, W * pairs * dk * esz),
                           span(g, pairs * dk * esz), span(tau, pairs * dk * esz),
                           span(v, W * pairs * dv * esz),
                           span(beta_hat, dense_beta ? pairs * dv * esz : 0),
                           s_fu[0], s_fu[1], s_fu[2], s_fu[3], s_fu[4], s_fu[5]};
    if (overlap(s_st, s_o)) return RODIMUS_ERR_INVALID_ARG;
    for (const Span &x : s_in)
        if (overlap(s_st, x) || overlap(s_o, x)) return RODIMUS_ERR_INVALID_ARG;
    FusedSteps f;
    f.u = fused->u; f.w = fused->w; f.rank = fused->rank; f.d = fused->d;
    f.conv_w = fused->conv_width; f.cq = fused->conv_q; f.ck = fused->conv_k; f.cv = fused->conv_v;
    hipError_t e = launch_decode(N, H, dk, dv, in_dtype == RODIMUS_DTYPE_F32,
                                 TokenInputs{q, k, g, tau, v, beta_hat}, state, out, stream, &f);
    return e == hipSuccess ? RODIMUS_OK : RODIMUS_ERR_HIP;
}

rodimus_status rodimus_swska_fwd(int B, int T, int H, int dk, int dv, int window, float scale,
                                 rodimus_dtype in_dtype, const void *q, const void *k,
                                 const void *v, float *out, hipStream_t stream)
{
    if (B <= 0 || H <= 0 || T < 0 || window < 1) return RODIMUS_ERR_INVALID_ARG;
    if (in_dtype != RODIMUS_DTYPE_BF16) return RODIMUS_ERR_UNSUPPORTED;
    if ((dk != 64 && dk != 128) || (dv != 64 && dv != 128)) return RODIMUS_ERR_UNSUPPORTED;
    if (!(scale >= 0.f) || scale > 3.0e38f) return RODIMUS_ERR_INVALID_ARG;   // NaN, negative, Inf
    if ((long long)B * ((T + 63) / 64) * H > (1LL << 31) - 1) return RODIMUS_ERR_INVALID_ARG;
    if ((long long)B * T > (1LL << 31) - 1) return RODIMUS_ERR_INVALID_ARG;
    // byte offsets within a 64-key tile of v are 32-bit
    if ((long long)64 * H * dv * 2 > (1LL << 31) - 1) return RODIMUS_ERR_INVALID_ARG;
    if (T == 0) return RODIMUS_OK;
    const void *ins[3] = {q, k, v};
    for (const void *p : ins)
        if (!p || !aligned16(p)) return RODIMUS_ERR_INVALID_ARG;
    if (!out || !aligned16(out)) return RODIMUS_ERR_INVALID_ARG;
    const size_t ntok = (size_t)B * T;
    const Span s_o = span(out, ntok * H * dv * sizeof(float));
    if (overlap(s_o, span(q, ntok * H * dk * 2)) || overlap(s_o, span(k, ntok * dk * 2)) ||
        overlap(s_o, span(v, ntok * H * dv * 2)))
        return RODIMUS_ERR_INVALID_ARG;
    const float sc = scale > 0.f ? scale : 1.f / sqrtf((float)dk);
    hipError_t e = launch_swska(B, T, H, dk, dv, window, sc, q, k, v, out, stream);
    return e == hipSuccess ? RODIMUS_OK : RODIMUS_ERR_HIP;
}

size_t rodimus_ddts_chunk_bwd_workspace_bytes(int B, int T, int H, int dk, int dv)
{
    if (B <= 0 || H <= 0 || T <= 0 || !width_ok(dk) || !width_ok(dv)) return 0;
    const int C = chunk_bwd_chunk(dk);
    return (size_t)B * H * (2 * ((T + C - 1) / C) + 1) * dk * dv * sizeof(float);
}

rodimus_status rodimus_ddts_chunk_bwd(
    int B, int T, int H, int dk, int dv, rodimus_dtype in_dtype,
    const void *q, const void *k, const void *g, const void *tau,
    const void *v, const void *beta_hat, const float *initial_state,
    const float *d_out, const float *d_final_state,
    float *dq, float *dk_, float *dg, float *dtau, float *dv_, float *dbeta_hat,
    float *d_initial_state, void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    rodimus_status st = check_chunk_args(B, T, H, dk, dv, 0, 0, in_dtype);
    if (st != RODIMUS_OK) return st;
    const size_t lds = chunk_bwd_lds_bytes(dk, dv, in_dtype == RODIMUS_DTYPE_F32);
    if (lds == 0 || lds > kLdsLimit) return RODIMUS_ERR_UNSUPPORTED;
    const bool f32 = in_dtype == RODIMUS_DTYPE_F32;
    const size_t esz = f32 ? 4 : 2;
    const size_t ntok = (size_t)B * T * H;
    const size_t state_bytes = (size_t)B * H * dk * dv * sizeof(float);
    if (T > 0) {
        const void *ins[7] = {q, k, g, tau, v, beta_hat, d_out};
        for (const void *p : ins)
            if (!p || !aligned16(p)) return RODIMUS_ERR_INVALID_ARG;
        float *outs[6] = {dq, dk_, dg, dtau, dv_, dbeta_hat};
        for (const float *p : outs)
            if (!p || !aligned16(p)) return RODIMUS_ERR_INVALID_ARG;
    }
    const void *opt[3] = {initial_state, d_final_state, d_initial_state};
    for (const void *p : opt)
        if (p && !aligned16(p)) return RODIMUS_ERR_INVALID_ARG;
    // every output overlaps nothing else
    const Span s_in[9] = {span(q, ntok * dk * esz), span(k, ntok * dk * esz),
                          span(g, ntok * dk * esz), span(tau, ntok * dk * esz),
                          span(v, ntok * dv * esz), span(beta_hat, ntok * dv * esz),
                          span(d_out, ntok * dv * sizeof(float)),
                          span(initial_state, initial_state ? state_bytes : 0),
                          span(d_final_state, d_final_state ? state_bytes : 0)};
    const Span s_out[7] = {span(dq, T > 0 ? ntok * dk * 4 : 0), span(dk_, T > 0 ? ntok * dk * 4 : 0),
                           span(dg, T > 0 ? ntok * dk * 4 : 0), span(dtau, T > 0 ? ntok * dk * 4 : 0),
                           span(dv_, T > 0 ? ntok * dv * 4 : 0), span(dbeta_hat, T > 0 ? ntok * dv * 4 : 0),
                           span(d_initial_state, d_initial_state ? state_bytes : 0)};
    for (int i = 0; i < 7; ++i) {
        for (const Span &x : s_in)
            if (overlap(s_out[i], x)) return RODIMUS_ERR_INVALID_ARG;
        for (int j = i + 1; j < 7; ++j)
            if (overlap(s_out[i], s_out[j])) return RODIMUS_ERR_INVALID_ARG;
    }
    const size_t wsb = rodimus_ddts_chunk_bwd_workspace_bytes(B, T, H, dk, dv);
    if (wsb > 0) {
        if (!workspace || workspace_bytes < wsb) return RODIMUS_ERR_WORKSPACE;
        if (!aligned16(workspace)) return RODIMUS_ERR_INVALID_ARG;
        const Span s_ws = span(workspace, wsb);
        for (const Span &x : s_in)
            if (overlap(s_ws, x)) return RODIMUS_ERR_INVALID_ARG;
        for (const Span &x : s_out)
            if (overlap(s_ws, x)) return RODIMUS_ERR_INVALID_ARG;
    }

    hipError_t e = hipSuccess;
    if (T == 0) {
        if (d_initial_state)
            e = launch_state_copy(d_final_state, d_initial_state, (size_t)B * H * dk * dv, stream);
        return e == hipSuccess ? RODIMUS_OK : RODIMUS_ERR_HIP;
    }
    // workspace: the state entering every chunk, S_T, dL/dS leaving every chunk
    const int C = chunk_bwd_chunk(dk);
    const int n_chunks = (T + C - 1) / C;
    const size_t sd = (size_t)dk * dv;
    float *ws_states = (float *)workspace;                                  // [BH][n_chunks][dk][dv]
    float *ws_final = ws_states + (size_t)B * H * n_chunks * sd;            // [BH][dk][dv]
    float *ws_adj = ws_final + (size_t)B * H * sd;                          // [BH][n_chunks][dk][dv]
    ChunkBwdLaunch Lc;
    Lc.B = B; Lc.T = T; Lc.H = H; Lc.dk = dk; Lc.dv = dv; Lc.f32_inputs = f32;
    Lc.in = TokenInputs{q, k, g, tau, v, beta_hat};
    Lc.s0 = initial_state; Lc.dout = d_out; Lc.dsf = d_final_state;
    Lc.s_chunks = ws_states; Lc.s_final = ws_final; Lc.d_chunks = ws_adj;
    Lc.dq = dq; Lc.dk_ = dk_; Lc.dg = dg; Lc.dtau = dtau; Lc.dv_ = dv_; Lc.dbeta = dbeta_hat;
    Lc.ds0 = d_initial_state;
    e = launch_chunk_bwd(Lc, stream);
    return e == hipSuccess ? RODIMUS_OK : RODIMUS_ERR_HIP;
}

}  // extern "C"
