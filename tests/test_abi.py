"""CPU tests of the C-ABI library: it loads, exports every declared symbol, and
rejects bad arguments on the host before any HIP call (no GPU needed: every
call here fails validation, so nothing is launched)."""
import ctypes
import os
import re

import pytest

import gated_linear_attention_rodimus_amd as R

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rodimus_ddts.h")

# fake, 16-byte aligned, never dereferenced device addresses
BASE = 0x7F0000000000
MB = 1 << 20


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rodimus_\w+)\s*\(", text)))


def test_header_symbols_exported():
    names = _declared_functions()
    assert "rodimus_ddts_chunk_fwd" in names and "rodimus_ddts_decode_step" in names
    L = ctypes.CDLL(R.LIB_PATH)
    for n in names:
        assert hasattr(L, n), f"{n} declared in rodimus_ddts.h but not exported"


def test_version_and_status_strings():
    assert R.abi_version() == 1
    L = R.lib()
    for s in range(5):
        assert L.rodimus_status_string(s)
    assert L.rodimus_status_string(0) == b"ok"
    assert L.rodimus_status_string(99) == b"unknown status"
    assert L.rodimus_status_string(-1) == b"unknown status"


def _chunk(B=1, T=128, H=2, dk=64, dv=128, chunk=0, segments=0, dtype=R.DTYPE_BF16,
           ptrs=None, s0=None, out=None, sf=None, ws=None, wsb=0):
    esz = 4 if dtype == R.DTYPE_F32 else 2
    ntok = B * T * H
    if ptrs is None:
        ptrs = []
        a = BASE
        for d in (dk, dk, dk, dk, dv, dv):
            ptrs.append(a)
            a += ((ntok * d * esz + MB) // 16) * 16
        if out is None:
            out = a
    vp = ctypes.c_void_p
    return R.lib().rodimus_ddts_chunk_fwd_ex(
        B, T, H, dk, dv, chunk, segments, dtype, *(vp(p) if p else None for p in ptrs),
        vp(s0) if s0 else None, vp(out) if out else None, vp(sf) if sf else None,
        vp(ws) if ws else None, wsb, None)


def test_chunk_rejects_bad_sizes():
    assert _chunk(B=0) == R.ERR_INVALID_ARG
    assert _chunk(H=0) == R.ERR_INVALID_ARG
    assert _chunk(T=-1) == R.ERR_INVALID_ARG
    assert _chunk(segments=-1) == R.ERR_INVALID_ARG
    assert _chunk(dk=48) == R.ERR_UNSUPPORTED
    assert _chunk(dv=256) == R.ERR_UNSUPPORTED
    assert _chunk(chunk=8) == R.ERR_UNSUPPORTED
    assert _chunk(chunk=128) == R.ERR_UNSUPPORTED
    assert _chunk(dtype=7) == R.ERR_UNSUPPORTED


def test_chunk_rejects_bad_pointers():
    good = [BASE + i * 64 * MB for i in range(6)]
    out = BASE + 6 * 64 * MB
    for i in range(6):
        p = list(good)
        p[i] = 0
        assert _chunk(ptrs=p, out=out) == R.ERR_INVALID_ARG, f"null input {i}"
        p = list(good)
        p[i] += 2
        assert _chunk(ptrs=p, out=out) == R.ERR_INVALID_ARG, f"misaligned input {i}"
    assert _chunk(ptrs=good, out=0) == R.ERR_INVALID_ARG
    assert _chunk(ptrs=good, out=out + 4) == R.ERR_INVALID_ARG
    # out overlapping an input
    assert _chunk(ptrs=good, out=good[3] + 1024) == R.ERR_INVALID_ARG
    # final state overlapping out, or partially overlapping the initial state
    s0 = BASE + 8 * 64 * MB
    assert _chunk(ptrs=good, out=out, s0=s0, sf=out + 4096) == R.ERR_INVALID_ARG
    assert _chunk(ptrs=good, out=out, s0=s0, sf=s0 + 4096) == R.ERR_INVALID_ARG
    # initial state misaligned
    assert _chunk(ptrs=good, out=out, s0=s0 + 8) == R.ERR_INVALID_ARG


def test_chunk_workspace_required_for_segments():
    B, T, H, dk, dv = 1, 4096, 2, 64, 128
    need = R.workspace_bytes(B, T, H, dk, dv, 0, 4)
    # a state slot and a decay row per transfer: the 3 segments before the last,
    # each cut in 2 (2 heads x 2 dv tiles x 6 transfers fill far fewer than 256 CUs)
    assert need == B * H * 6 * (dk * dv + dk) * 4
    good = [BASE + i * 64 * MB for i in range(6)]
    out = BASE + 6 * 64 * MB
    ws = BASE + 8 * 64 * MB
    assert _chunk(B, T, H, dk, dv, segments=4, ptrs=good, out=out) == R.ERR_WORKSPACE
    assert _chunk(B, T, H, dk, dv, segments=4, ptrs=good, out=out, ws=ws,
                  wsb=need - 1) == R.ERR_WORKSPACE
    # workspace overlapping an input is rejected
    assert _chunk(B, T, H, dk, dv, segments=4, ptrs=good, out=out, ws=good[0],
                  wsb=need) == R.ERR_INVALID_ARG


def test_workspace_bytes_plan():
    # one sweep when the (b, h, dv tile) units fill more than half the CUs: no workspace
    assert R.workspace_bytes(8, 2048, 12, 64, 128) == 0
    # 64 heads x 2 dv tiles = half the CUs: segmented.  bf16 inputs: the
    # whole-head tile, 4 segments (256 workgroups), 3 transfers cut in 2 (6
    # slots); fp32 inputs: 2 segments of 64-token chunks, the first one's
    # transfer cut in 2.  The larger need, 6 slots per head:
    assert R.workspace_bytes(4, 4096, 16, 64, 128) == 4 * 16 * 6 * (64 * 128 + 64) * 4
    # two segments asked for: 64-token chunks, the first segment's transfer
    # cut in 2 (bf16 and fp32 alike), 2 slots per head
    assert R.workspace_bytes(4, 4096, 16, 64, 128, 0, 2) == 4 * 16 * 2 * (64 * 128 + 64) * 4
    # long sequence, few heads: segmented
    ws = R.workspace_bytes(1, 65536, 16, 64, 128)
    assert ws > 0 and ws % (16 * (64 * 128 + 64) * 4) == 0
    # forcing one sweep
    assert R.workspace_bytes(1, 65536, 16, 64, 128, 0, 1) == 0
    # invalid arguments report 0
    assert R.workspace_bytes(1, 100, 1, 48, 128) == 0


def _decode(N=4, H=2, dk=64, dv=128, dtype=R.DTYPE_BF16, ptrs=None, state=None, out=None):
    if ptrs is None:
        ptrs = [BASE + i * MB for i in range(6)]
    if state is None:
        state = BASE + 16 * MB
    if out is None:
        out = BASE + 32 * MB
    vp = ctypes.c_void_p
    return R.lib().rodimus_ddts_decode_step(
        N, H, dk, dv, dtype, *(vp(p) if p else None for p in ptrs),
        vp(state) if state else None, vp(out) if out else None, None)


def test_decode_rejects_bad_args():
    assert _decode(N=0) == R.ERR_INVALID_ARG
    assert _decode(H=0) == R.ERR_INVALID_ARG
    assert _decode(dk=24) == R.ERR_UNSUPPORTED
    assert _decode(dtype=3) == R.ERR_UNSUPPORTED
    assert _decode(state=0) == R.ERR_INVALID_ARG
    assert _decode(out=0) == R.ERR_INVALID_ARG
    assert _decode(out=BASE + 16 * MB + 64) == R.ERR_INVALID_ARG      # out inside state
    assert _decode(state=BASE + 2 * MB - 4096) == R.ERR_INVALID_ARG    # state over inputs
    p = [BASE + i * MB for i in range(6)]
    p[4] = 0
    assert _decode(ptrs=p) == R.ERR_INVALID_ARG
    p = [BASE + i * MB for i in range(6)]
    p[2] += 4
    assert _decode(ptrs=p) == R.ERR_INVALID_ARG


def test_binding_requires_gpu_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(1, 4, 1, 16)
    with pytest.raises(ValueError):
        R.chunk_fwd(x, x, x, x, x, x)
    with pytest.raises(ValueError):
        R.decode_step(x[0], x[0], x[0], x[0], x[0], x[0], torch.zeros(4, 1, 16, 16))


def _bwd(B=1, T=64, H=2, dk=64, dv=128, dtype=R.DTYPE_BF16, ws=None, wsb=0, misalign=None,
         alias=None, null=None):
    """rodimus_ddts_chunk_bwd with fake device pointers in argument order:
    q, k, g, tau, v, beta_hat (0-5), initial_state (6), d_out (7),
    d_final_state (8), dq, dk, dg, dtau, dv, dbeta_hat (9-14), d_initial_state
    (15), laid out one after another."""
    esz = 4 if dtype == R.DTYPE_F32 else 2
    ntok = B * T * H
    state = B * H * dk * dv * 4
    sizes = [ntok * d * esz for d in (dk, dk, dk, dk, dv, dv)] + [state, ntok * dv * 4, state]
    sizes += [ntok * d * 4 for d in (dk, dk, dk, dk, dv, dv)] + [B * H * dk * dv * 4]   # outputs
    ptrs, a = [], BASE
    for s in sizes:
        ptrs.append(a)
        a += ((s + MB) // 16) * 16
    if misalign is not None:
        ptrs[misalign] += 4
    if alias is not None:
        ptrs[alias[0]] = ptrs[alias[1]]
    if null is not None:
        ptrs[null] = 0
    vp = ctypes.c_void_p
    p = [vp(x) if x else None for x in ptrs]
    return R.lib().rodimus_ddts_chunk_bwd(B, T, H, dk, dv, dtype, *p, vp(ws) if ws else None, wsb, None)


def test_bwd_workspace_bytes():
    # the state entering and the adjoint leaving every 64-token chunk, and S_T
    assert R.bwd_workspace_bytes(2, 100, 3, 64, 128) == 2 * 3 * (2 * 2 + 1) * 64 * 128 * 4
    # 32-token chunks at dk = 128
    assert R.bwd_workspace_bytes(1, 100, 2, 128, 64) == 1 * 2 * (2 * 4 + 1) * 128 * 64 * 4
    assert R.bwd_workspace_bytes(1, 0, 1, 64, 64) == 0


def test_bwd_validation():
    assert _bwd() == R.ERR_WORKSPACE                                       # no workspace
    assert _bwd(dk=128, dv=128) == R.ERR_WORKSPACE                         # supported shape
    assert _bwd(dk=48) == R.ERR_UNSUPPORTED
    assert _bwd(dtype=7) == R.ERR_UNSUPPORTED
    assert _bwd(misalign=0) == R.ERR_INVALID_ARG                           # q misaligned
    assert _bwd(misalign=9) == R.ERR_INVALID_ARG                           # dq misaligned
    assert _bwd(null=7) == R.ERR_INVALID_ARG                               # no d_out
    assert _bwd(null=6) == R.ERR_WORKSPACE                                 # no S0: allowed
    assert _bwd(null=10) == R.ERR_INVALID_ARG                              # no dk
    assert _bwd(alias=(9, 0)) == R.ERR_INVALID_ARG                         # dq over q
    assert _bwd(alias=(10, 9)) == R.ERR_INVALID_ARG                        # dk over dq
    assert _bwd(alias=(15, 6)) == R.ERR_INVALID_ARG                        # dS0 over S0
    assert _bwd(alias=(14, 7)) == R.ERR_INVALID_ARG                        # dbeta over d_out
    assert _bwd(B=0) == R.ERR_INVALID_ARG
    # workspace overlapping an output
    assert _bwd(ws=BASE + 16, wsb=1 << 40) == R.ERR_INVALID_ARG


def _plan(*a, **k):
    return R.chunk_fwd_plan(*a, **k)


def test_plan_one_sweep_when_units_fill_the_gpu():
    # 130M layer: 96 heads x 2 dv tiles of 64 = 192 workgroups: one sweep, 64-token chunks
    p = _plan(8, 2048, 12, 64, 128)
    assert p == {"chunk": 64, "dv_tile": 64, "segments": 1, "transfer_pieces": 0,
                 "workspace_bytes": 0}
    assert _plan(8, 2048, 12, 64, 128, dtype="f32")["segments"] == 1


def test_plan_segmented_bf16_takes_whole_heads_or_short_chunks():
    # 1.6B layer: 64 heads x 2 tiles = 128 units, half the CUs: segmented.
    # bf16, dv = 128, sequences long enough: the whole-head tile (one
    # workgroup per CU), 256 / 64 = 4 segments of 64-token chunks; the 3
    # transfers run 32-token chunks at two workgroups per CU, each cut in 2
    p = _plan(4, 4096, 16, 64, 128)
    assert (p["chunk"], p["dv_tile"], p["segments"], p["transfer_pieces"]) == (64, 128, 4, 2)
    assert p["workspace_bytes"] == 4 * 16 * 6 * (64 * 128 + 64) * 4
    # long prefill: 16 heads -> 16 segments of 64 chunks, 15 x 2 transfers
    p = _plan(1, 65536, 16, 64, 128)
    assert (p["chunk"], p["dv_tile"], p["segments"], p["transfer_pieces"]) == (64, 128, 16, 2)
    # too short for whole-head segments that fill the CUs: 64-column tiles,
    # 32-token chunks (two workgroups per CU), the segment count capped at
    # one per 8 chunks
    p = _plan(1, 1024, 2, 64, 128)
    assert (p["chunk"], p["dv_tile"], p["segments"]) == (32, 64, 4)
    # no whole-head tile for fp32 inputs or dv < 128
    assert _plan(1, 65536, 16, 64, 128, dtype="f32")["dv_tile"] == 64
    assert _plan(1, 65536, 16, 64, 64)["dv_tile"] == 64
    # nor at dk = 128
    assert _plan(1, 65536, 16, 128, 128)["dv_tile"] == 64


def test_plan_segmented_fp32_keeps_long_chunks():
    # fp32 kernels run one workgroup per CU: 64-token chunks, 256 / 128 = 2
    # segments, the first segment's transfer cut in 2
    p = _plan(4, 4096, 16, 64, 128, dtype="f32")
    assert (p["chunk"], p["segments"], p["transfer_pieces"]) == (64, 2, 2)
    assert p["workspace_bytes"] == 4 * 16 * 2 * (64 * 128 + 64) * 4


def test_plan_explicit_segments_and_chunk():
    # an explicit segment count keeps the longest chunk that fits; with 32
    # chunks per segment the transfers (64 x 64 tiles of 64-token chunks: one
    # per CU) are cut in 2
    p = _plan(4, 4096, 16, 64, 128, 0, 2)
    assert (p["chunk"], p["segments"], p["transfer_pieces"]) == (64, 2, 2)
    # narrower dv tiles run two transfers per CU: cut in 4
    p = _plan(4, 4096, 16, 64, 32, 0, 2)
    assert (p["chunk"], p["dv_tile"], p["segments"], p["transfer_pieces"]) == (64, 32, 2, 4)
    # segments = 1 forces one sweep; the chunk request is an upper bound
    assert _plan(1, 65536, 16, 64, 128, 0, 1)["segments"] == 1
    assert _plan(8, 2048, 12, 64, 128, 16)["chunk"] == 16
    # dk = 128: 64-token tiles do not fit the LDS
    assert _plan(8, 2048, 12, 128, 128)["chunk"] == 32
    # sequences of fewer than 16 chunks are not split; 16 give 2 segments of 8
    assert _plan(1, 15 * 32, 1, 64, 128)["segments"] == 1
    assert _plan(1, 15 * 32 + 1, 1, 64, 128)["segments"] == 2


def test_plan_rejects_what_the_forward_rejects():
    with pytest.raises(R.RodimusError):
        _plan(1, 100, 1, 48, 128)
    with pytest.raises(R.RodimusError):
        _plan(1, 100, 1, 64, 128, 48)
    with pytest.raises(R.RodimusError):
        _plan(0, 100, 1, 64, 128)


def test_named_workspace_query_agrees_with_ex():
    """rodimus_ddts_chunk_fwd_workspace_bytes is the _ex query with the
    library's own segment choice (segments = 0), for every chunk request."""
    L = R.lib()
    for shape in ((8, 2048, 12, 64, 128), (4, 4096, 16, 64, 128), (1, 65536, 16, 64, 128),
                  (1, 300, 1, 16, 32), (2, 1000, 3, 128, 64)):
        for chunk in (0, 16, 32, 64):
            a = L.rodimus_ddts_chunk_fwd_workspace_bytes(*shape, chunk)
            b = L.rodimus_ddts_chunk_fwd_ex_workspace_bytes(*shape, chunk, 0)
            assert a == b, (shape, chunk, a, b)
    assert L.rodimus_ddts_chunk_fwd_workspace_bytes(1, 65536, 16, 64, 128, 0) > 0
    assert L.rodimus_ddts_chunk_fwd_workspace_bytes(0, 10, 1, 64, 128, 0) == 0


def test_binding_checks_a_supplied_workspace():
    """A caller's workspace is checked before any library call: its device,
    contiguity and size in bytes (numel * element_size, any dtype)."""
    import torch
    dev = torch.device("cuda:0")
    assert R._check_workspace(None, 0, dev) == 0
    cpu = torch.empty(1024, dtype=torch.uint8)
    with pytest.raises(ValueError, match="device"):
        R._check_workspace(cpu, 16, dev)
    meta = torch.empty(1024, dtype=torch.uint8, device="meta")
    with pytest.raises(ValueError, match="device"):
        R._check_workspace(meta, 16, dev)
    with pytest.raises(TypeError):
        R._check_workspace(bytearray(64), 16, dev)
    # sizes are counted in bytes: 256 float32 elements hold 1024 bytes
    f = torch.empty(256, dtype=torch.float32)
    assert R._check_workspace(f, 1024, torch.device("cpu")) == 1024
    with pytest.raises(ValueError, match="needs 1025"):
        R._check_workspace(f, 1025, torch.device("cpu"))
    nc = torch.empty(64, 4, dtype=torch.uint8).t()
    with pytest.raises(ValueError, match="contiguous"):
        R._check_workspace(nc, 16, torch.device("cpu"))


def test_static_scratch_entry_rejects_plans_beyond_its_buffer():
    """The allocation-free forward returns RODIMUS_ERR_WORKSPACE, before any
    HIP call, when the plan's workspace exceeds the fixed buffer (64 heads in
    64 segments need ~135 MB), and validates its arguments like the others."""
    L = R.lib()
    vp = ctypes.c_void_p
    B, T, H, dk, dv = 1, 65536, 64, 64, 128
    need = L.rodimus_ddts_chunk_fwd_ex_workspace_bytes(B, T, H, dk, dv, 0, 64)
    assert need > R.STATIC_SCRATCH_BYTES
    ntok = B * T * H
    ptrs, a = [], BASE
    for d in (dk, dk, dk, dk, dv, dv):
        ptrs.append(a)
        a += ((ntok * d * 2 + MB) // 16) * 16
    out = a
    st = L.rodimus_ddts_chunk_fwd_static_scratch(B, T, H, dk, dv, 0, 64, R.DTYPE_BF16,
                                                 *(vp(p) for p in ptrs), None, vp(out), None, None)
    assert st == R.ERR_WORKSPACE
    st = L.rodimus_ddts_chunk_fwd_static_scratch(B, T, H, 48, dv, 0, 0, R.DTYPE_BF16,
                                                 *(vp(p) for p in ptrs), None, vp(out), None, None)
    assert st == R.ERR_UNSUPPORTED
    st = L.rodimus_ddts_chunk_fwd_static_scratch(B, T, H, dk, dv, 0, 0, R.DTYPE_BF16,
                                                 *(vp(p) for p in ptrs), None, vp(ptrs[0]), None,
                                                 None)
    assert st == R.ERR_INVALID_ARG            # out overlaps q


def test_trace_events_argument_checks():
    """The tracing aid takes exactly four events, or none to stop; nothing
    else reaches the runtime."""
    L = R.lib()
    assert L.rodimus_trace_forward_events(None, 0) == R.OK
    assert L.rodimus_trace_forward_events(None, 4) == R.ERR_INVALID_ARG
    arr = (ctypes.c_void_p * 4)(1, 2, 3, 4)
    assert L.rodimus_trace_forward_events(arr, 3) == R.ERR_INVALID_ARG
    assert L.rodimus_trace_forward_events(arr, 4) == R.OK
    assert L.rodimus_trace_forward_events(None, 0) == R.OK


def test_swska_argument_checks():
    """SW-SKA rejects bad sizes, dtypes, widths, scales, pointers and overlaps
    on the host (no GPU needed)."""
    L = R.lib()
    vp = ctypes.c_void_p
    B, T, H, dk, dv = 2, 100, 4, 128, 128
    q, k, v, o = BASE, BASE + 64 * MB, BASE + 128 * MB, BASE + 192 * MB

    def call(B=B, T=T, H=H, dk=dk, dv=dv, window=16, scale=0.0, dt=R.DTYPE_BF16,
             q=q, k=k, v=v, o=o):
        return L.rodimus_swska_fwd(B, T, H, dk, dv, window, scale, dt,
                                   vp(q) if q else None, vp(k) if k else None,
                                   vp(v) if v else None, vp(o) if o else None, None)

    assert call(window=0) == R.ERR_INVALID_ARG
    assert call(B=0) == R.ERR_INVALID_ARG
    assert call(T=-1) == R.ERR_INVALID_ARG
    assert call(dt=R.DTYPE_F32) == R.ERR_UNSUPPORTED
    assert call(dk=32) == R.ERR_UNSUPPORTED
    assert call(dv=16) == R.ERR_UNSUPPORTED
    assert call(scale=-1.0) == R.ERR_INVALID_ARG
    assert call(scale=float("nan")) == R.ERR_INVALID_ARG
    assert call(scale=float("inf")) == R.ERR_INVALID_ARG
    assert call(q=0) == R.ERR_INVALID_ARG
    assert call(v=v + 2) == R.ERR_INVALID_ARG           # misaligned
    assert call(o=q) == R.ERR_INVALID_ARG               # out over q
    assert call(o=k + 1024) == R.ERR_INVALID_ARG        # out over k
    # byte offsets within a 64-key tile of v are 32-bit: 64 * H * dv * 2 < 2^31
    assert call(H=(1 << 31) // (64 * 128 * 2)) == R.ERR_INVALID_ARG
    assert call(T=0) == R.OK                             # nothing to do, nothing launched
