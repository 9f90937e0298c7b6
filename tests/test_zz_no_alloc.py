"""GPU: the allocation-free forward entry (rodimus_ddts_chunk_fwd_static_scratch),
called through the C ABI, against the workspace-taking entry it mirrors
(rodimus_ddts_chunk_fwd_ex): two calls in a row, the second on a smaller
input, both on the segmented path that uses the scratch.  The two entries run
the same kernels with the same plan, so their results are compared bit for
bit, and the smaller call also against the fp64 oracle (bar 1e-2, bf16)."""
import ctypes

import numpy as np
import pytest

import ddts_inputs as D
import oracle

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

NAMES = ("q", "k", "v", "g", "tau", "beta_hat")


def _vp(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _args(x, dev):
    wl = x.wl
    t = [x.torch(n, dev) for n in NAMES]
    s0 = torch.from_numpy(x.initial_state).to(dev)
    return wl, t, s0


def _static(R, wl, t, s0, out, fs):
    q, k, v, g, tau, beta = t
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return R.lib().rodimus_ddts_chunk_fwd_static_scratch(
        wl.B, wl.T, wl.H, wl.dk, wl.dv, 0, 0, R.DTYPE_BF16, _vp(q), _vp(k), _vp(g), _vp(tau),
        _vp(v), _vp(beta), _vp(s0), _vp(out), _vp(fs), stream)


def _ex(R, wl, t, s0, out, fs):
    q, k, v, g, tau, beta = t
    wsb = R.lib().rodimus_ddts_chunk_fwd_ex_workspace_bytes(wl.B, wl.T, wl.H, wl.dk, wl.dv, 0, 0)
    ws = torch.empty(wsb, dtype=torch.uint8, device=out.device)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    st = R.lib().rodimus_ddts_chunk_fwd_ex(
        wl.B, wl.T, wl.H, wl.dk, wl.dv, 0, 0, R.DTYPE_BF16, _vp(q), _vp(k), _vp(g), _vp(tau),
        _vp(v), _vp(beta), _vp(s0), _vp(out), _vp(fs), _vp(ws), ctypes.c_size_t(wsb), stream)
    torch.cuda.synchronize()
    return st


def test_static_scratch_entry_matches_workspace_entry():
    import gated_linear_attention_rodimus_amd as R
    dev = torch.device("cuda:0")
    big = D.make("long_prefill", T=20000)                 # 16 heads, segmented
    small = D.make("long_prefill", T=5003, H=4)           # 4 heads, segmented, ragged
    cases = []
    for x in (big, small):
        wl, t, s0 = _args(x, dev)
        plan = R.chunk_fwd_plan(wl.B, wl.T, wl.H, wl.dk, wl.dv)
        assert plan["segments"] > 1 and 0 < plan["workspace_bytes"] <= R.STATIC_SCRATCH_BYTES, plan
        out = torch.full((wl.B, wl.T, wl.H, wl.dv), float("nan"), device=dev)
        fs = torch.full((wl.B, wl.H, wl.dk, wl.dv), float("nan"), device=dev)
        cases.append((x, wl, t, s0, out, fs, plan))
    # two calls in a row on the static scratch, the second smaller
    for (x, wl, t, s0, out, fs, plan) in cases:
        print(f"static-scratch call B{wl.B} T{wl.T} H{wl.H} plan {plan}", flush=True)
        assert _static(R, wl, t, s0, out, fs) == R.OK
    torch.cuda.synchronize()
    for (x, wl, t, s0, out, fs, plan) in cases:
        out_r = torch.empty_like(out)
        fs_r = torch.empty_like(fs)
        assert _ex(R, wl, t, s0, out_r, fs_r) == R.OK
        assert torch.equal(out, out_r), f"out differs, T={wl.T} H={wl.H}"
        assert torch.equal(fs, fs_r), f"final state differs, T={wl.T} H={wl.H}"
    x, wl, t, s0, out, fs, plan = cases[1]
    ro, rs = oracle.fwd(*(x.f32(n) for n in NAMES), x.initial_state)
    eo = oracle.rel_to_rms_error(out.cpu().numpy(), ro)
    es = oracle.rel_to_rms_error(fs.cpu().numpy(), rs)
    print(f"static-scratch small call vs oracle: out {eo:.2e} state {es:.2e}", flush=True)
    assert eo <= 1e-2 and es <= 1e-2


def test_static_scratch_binding_allocates_nothing_new():
    """The binding's no-alloc call matches chunk_fwd on a sweep-path shape
    (no scratch needed) and on a segmented one."""
    import gated_linear_attention_rodimus_amd as R
    dev = torch.device("cuda:0")
    for x in (D.make("layer130m", B=2, T=700, H=12), D.make("long_prefill", T=9000, H=2)):
        wl = x.wl
        t = [x.torch(n, dev) for n in NAMES]
        s0 = None if x.initial_state is None else torch.from_numpy(x.initial_state).to(dev)
        o_ref, s_ref = R.chunk_fwd(*t, initial_state=s0, output_final_state=True)
        out = torch.empty_like(o_ref)
        fs = torch.empty_like(s_ref)
        R.chunk_fwd_no_alloc(*t, out, initial_state=s0, final_state=fs)
        torch.cuda.synchronize()
        assert torch.equal(out, o_ref) and torch.equal(fs, s_ref)
