"""GPU: the boundary's own forward symbol and workspace query, called straight
through ctypes (not through the binding or the _ex variant), and the
behaviour of non-finite inputs that the header documents.

Bars as everywhere: max |x_hat - x| / RMS(x) <= 1e-2 for bf16 inputs against
the fp64 oracle on the same bf16-rounded values, outputs and states apart.
"""
import ctypes

import numpy as np
import pytest

import ddts_inputs as D
import oracle

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

NAMES = ("q", "k", "v", "g", "tau", "beta_hat")


@pytest.fixture(scope="module")
def R():
    import gated_linear_attention_rodimus_amd as mod
    mod.lib()
    return mod


def _vp(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _named_fwd(R, x, s0, want_final):
    """rodimus_ddts_chunk_fwd with a workspace sized by
    rodimus_ddts_chunk_fwd_workspace_bytes, on torch's current stream."""
    dev = torch.device("cuda:0")
    wl = x.wl
    L = R.lib()
    t = [x.torch(n, dev) for n in NAMES]
    out = torch.empty(wl.B, wl.T, wl.H, wl.dv, device=dev)
    fs = torch.empty(wl.B, wl.H, wl.dk, wl.dv, device=dev) if want_final else None
    s0d = None if s0 is None else torch.from_numpy(np.ascontiguousarray(s0, np.float32)).to(dev)
    wsb = L.rodimus_ddts_chunk_fwd_workspace_bytes(wl.B, wl.T, wl.H, wl.dk, wl.dv, 0)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    code = R.DTYPE_BF16 if wl.dtype == "bf16" else R.DTYPE_F32
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    q, k, v, g, tau, beta = t
    st = L.rodimus_ddts_chunk_fwd(wl.B, wl.T, wl.H, wl.dk, wl.dv, 0, code,
                                  _vp(q), _vp(k), _vp(g), _vp(tau), _vp(v), _vp(beta),
                                  _vp(s0d), _vp(out), _vp(fs), _vp(ws), ctypes.c_size_t(wsb),
                                  stream)
    assert st == R.OK, R.lib().rodimus_status_string(st)
    torch.cuda.synchronize()
    return out.cpu().numpy(), (None if fs is None else fs.cpu().numpy()), wsb


def test_named_forward_layer1p6b_returns_final_state(R):
    """The 1.6B-layer shape (B4 T4096 H16, returns S_T) through the named
    symbol; the library's own plan segments it, so the workspace is used."""
    x = D.make("layer1p6b")
    o, sf, wsb = _named_fwd(R, x, None, True)
    assert wsb > 0
    ro, rs = oracle.fwd(*(x.f32(n) for n in NAMES), None)
    eo, es = oracle.rel_to_rms_error(o, ro), oracle.rel_to_rms_error(sf, rs)
    print(f"[named layer1p6b] out err {eo:.2e} state err {es:.2e} workspace {wsb}", flush=True)
    assert eo <= 1e-2 and es <= 1e-2


def test_named_forward_long_prefill_slice_with_initial_state(R):
    """A slice of the long prefill (B1 T12288 H16, N(0, 0.1) initial state,
    ragged against every chunk length), no final state asked for."""
    x = D.make("long_prefill", T=12288 + 37)
    o, sf, wsb = _named_fwd(R, x, x.initial_state, False)
    assert wsb > 0 and sf is None
    ro, _ = oracle.fwd(*(x.f32(n) for n in NAMES), x.initial_state)
    eo = oracle.rel_to_rms_error(o, ro)
    print(f"[named long_prefill slice] out err {eo:.2e} workspace {wsb}", flush=True)
    assert eo <= 1e-2


# ---------------------------------------------------------------- non-finite inputs


def _poison(x, name, b, t, h, i, value):
    a = getattr(x, name)
    if a.dtype == np.uint16:
        a[b, t, h, i] = D.bf16_round_bits(np.array([value], np.float32))[0]
    else:
        a[b, t, h, i] = value


def test_forward_propagates_nan_and_inf(R):
    """Every output the recurrence makes depend on a NaN or Inf input is
    non-finite on the GPU too.  The chunk form may also spread it to the
    earlier tokens of the poisoned token's chunk (their products with it are
    masked by multiplication, and 0 * NaN is NaN), but never to earlier
    chunks or to other heads, which stay finite and within the bar."""
    x = D.make("layer130m", B=2, T=300, H=3)
    poison = [("v", 0, 150, 1, 5, np.nan), ("q", 1, 20, 0, 3, np.inf),
              ("g", 1, 250, 2, 7, np.nan), ("k", 0, 40, 2, 0, -np.inf)]
    for p in poison:
        _poison(x, *p)
    C = R.chunk_fwd_plan(2, 300, 3, 64, 128)["chunk"]
    dev = torch.device("cuda:0")
    o, sf = R.chunk_fwd(*(x.torch(n, dev) for n in NAMES), output_final_state=True)
    torch.cuda.synchronize()
    o, sf = o.cpu().numpy(), sf.cpu().numpy()
    with np.errstate(invalid="ignore", over="ignore"):
        ro, rs = oracle.fwd(*(x.f32(n) for n in NAMES), None)
    poisoned = {(b, h): t for (_, b, t, h, _, _) in poison}
    for b in range(2):
        for h in range(3):
            g_o, r_o = o[b, :, h], ro[b, :, h]
            bad_ref = ~np.isfinite(r_o)
            bad_gpu = ~np.isfinite(g_o)
            if (b, h) not in poisoned:
                assert not bad_ref.any() and not bad_gpu.any(), (b, h)
                assert oracle.rel_to_rms_error(g_o, r_o) <= 1e-2
                assert oracle.rel_to_rms_error(sf[b, h], rs[b, h]) <= 1e-2
                continue
            t0 = poisoned[(b, h)]
            assert bad_ref.any(), (b, h)
            assert not (bad_ref & ~bad_gpu).any(), f"non-finite reference output finite on GPU {(b, h)}"
            first = (t0 // C) * C
            assert not bad_gpu[:first].any(), f"non-finite before the poisoned chunk {(b, h)}"
            if first > 0:
                assert oracle.rel_to_rms_error(g_o[:first], r_o[:first]) <= 1e-2
            assert not (~np.isfinite(rs[b, h]) & np.isfinite(sf[b, h])).any()


def test_decode_step_propagates_nan_and_inf(R):
    """One decode step: non-finite outputs and state entries on the GPU are
    exactly those of the oracle; every other value is within the bar."""
    sets, st = D.make_decode_pool("decode_batch", pool=1, B=8, H=4)
    x = sets[0]
    _poison(x, "k", 1, 0, 2, 9, np.nan)
    _poison(x, "q", 3, 0, 0, 1, np.inf)
    _poison(x, "v", 5, 0, 3, 100, -np.inf)
    _poison(x, "tau", 6, 0, 1, 4, np.nan)
    dev = torch.device("cuda:0")
    S = torch.from_numpy(st).to(dev)
    o = R.decode_step(*(x.torch(n, dev)[:, 0] for n in NAMES), S)
    torch.cuda.synchronize()
    o, S = o.cpu().numpy(), S.cpu().numpy()
    with np.errstate(invalid="ignore", over="ignore"):
        ro, rs = oracle.decode(*(x.f32(n)[:, 0] for n in NAMES), st)
    for g_, r_ in ((o, ro), (S, rs)):
        bad = ~np.isfinite(r_)
        assert bad.any()
        assert np.array_equal(bad, ~np.isfinite(g_))
        assert oracle.rel_to_rms_error(g_[~bad], r_[~bad]) <= 1e-2


def test_trace_events_bracket_the_passes(R):
    """The library's pass events: ordered in time, their spans add up to the
    call, and tracing leaves the results unchanged (segmented and one-sweep
    shapes)."""
    dev = torch.device("cuda:0")
    for x, s0 in ((D.make("long_prefill", T=20000, H=4), True), (D.make("layer130m", B=2, T=500), False)):
        t = [x.torch(n, dev) for n in NAMES]
        s0d = torch.from_numpy(x.initial_state).to(dev) if s0 else None
        o_ref, _ = R.chunk_fwd(*t, initial_state=s0d)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        for e in ev:
            e.record()
        torch.cuda.synchronize()
        R.trace_forward_events(ev)
        try:
            o, _ = R.chunk_fwd(*t, initial_state=s0d)
        finally:
            R.trace_forward_events(None)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref)
        seg = R.chunk_fwd_plan(*[x.wl.B, x.wl.T, x.wl.H, 64, 128])["segments"] > 1
        spans = [ev[j].elapsed_time(ev[j + 1]) for j in range(3 if seg else 1)]
        print(f"[trace] segmented={seg} spans ms {spans}", flush=True)
        assert all(sp >= 0.0 for sp in spans) and sum(spans) > 0.0
