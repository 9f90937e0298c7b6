"""GPU parity of the backward (rodimus_ddts_chunk_bwd through the C ABI) against
the fp64 reverse-mode oracle.

Bars, for every gradient separately (max |x_hat - x| / RMS(x)): 1e-4 for fp32
inputs, 1e-2 for bf16 inputs (the oracle on the same bf16-rounded values).
dL/d out and dL/d S_T are seeded N(0, 1) draws passed to both sides.
"""
import numpy as np
import pytest

import ddts_inputs as D
import oracle

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

NAMES = ("q", "k", "v", "g", "tau", "beta_hat")
GRADS = ("dq", "dk", "dg", "dtau", "dv", "dbeta_hat", "d_initial_state")
BAR = {"bf16": 1e-2, "f32": 1e-4}


@pytest.fixture(scope="module")
def R():
    import gated_linear_attention_rodimus_amd as mod
    mod.lib()
    return mod


@pytest.fixture(scope="module")
def dev():
    return torch.device("cuda:0")


def cotangents(x, seed, final=True):
    W = x.wl
    rng = np.random.default_rng(seed)
    d_out = rng.standard_normal((W.B, W.T, W.H, W.dv), dtype=np.float32)
    d_sf = rng.standard_normal((W.B, W.H, W.dk, W.dv), dtype=np.float32) if final else None
    return d_out, d_sf


def check(R, dev, x, d_out, d_sf, s0, bar, heads=None):
    t = [x.torch(n, dev) for n in NAMES]
    tt = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)
    g = R.chunk_bwd(*t, tt(d_out), initial_state=tt(s0), d_final_state=tt(d_sf))
    torch.cuda.synchronize()
    g = {n: v.cpu().numpy() for n, v in g.items()}
    ins = [x.f32(n) for n in NAMES]
    if heads is None:
        r = oracle.bwd(*ins, d_out, s0, d_sf)
        errs = {n: oracle.rel_to_rms_error(g[n], r[n]) for n in GRADS if r[n].size}
    else:
        errs = {n: 0.0 for n in GRADS}
        for (b, h) in heads:
            sl = lambda a: np.ascontiguousarray(a[b:b + 1, :, h:h + 1])
            ss = lambda a: None if a is None else np.ascontiguousarray(a[b:b + 1, h:h + 1])
            r = oracle.bwd(*(sl(a) for a in ins), sl(d_out), ss(s0), ss(d_sf))
            for n in GRADS:
                gg = g[n][b:b + 1, :, h:h + 1] if n != "d_initial_state" else g[n][b:b + 1, h:h + 1]
                errs[n] = max(errs[n], oracle.rel_to_rms_error(gg, r[n]))
    for n in GRADS:
        assert np.all(np.isfinite(g[n])), n
    bad = {n: e for n, e in errs.items() if not e < bar}
    assert not bad, f"errors above {bar}: {bad} (all: {errs})"
    return errs


@pytest.mark.parametrize("T", [64, 37, 16, 1, 65, 200])
def test_bwd_tiny_fp32(R, dev, T):
    x = D.make("tiny", T=T)
    rng = np.random.default_rng(5)
    s0 = rng.standard_normal((x.wl.B, x.wl.H, x.wl.dk, x.wl.dv)).astype(np.float32)
    d_out, d_sf = cotangents(x, 7)
    check(R, dev, x, d_out, d_sf, s0, BAR["f32"])


@pytest.mark.parametrize("dk,dv", [(16, 16), (16, 128), (32, 64), (64, 16), (64, 32), (64, 128),
                                   (128, 16), (128, 32), (128, 64), (128, 128)])
def test_bwd_widths_bf16(R, dev, dk, dv):
    x = D.make("layer1p6b", B=2, T=93, H=3, dk=dk, dv=dv)
    d_out, d_sf = cotangents(x, 8)
    check(R, dev, x, d_out, d_sf, None, BAR["bf16"])


@pytest.mark.parametrize("dk,dv,T", [(64, 128, 70), (128, 128, 70), (32, 16, 130)])
def test_bwd_fp32_widths(R, dev, dk, dv, T):
    x = D.make("tiny", B=2, T=T, H=2, dk=dk, dv=dv)
    d_out, d_sf = cotangents(x, 9)
    check(R, dev, x, d_out, d_sf, None, BAR["f32"])


def test_bwd_no_final_cotangent_with_initial_state(R, dev):
    x = D.make("long_prefill", T=300, H=2)
    d_out, _ = cotangents(x, 10, final=False)
    check(R, dev, x, d_out, None, x.initial_state, BAR["bf16"])


def test_bwd_layer130m_full(R, dev):
    """The 130M layer at full size (B8 T2048 H12), a sample of heads checked."""
    x = D.make("layer130m")
    d_out, d_sf = cotangents(x, 11)
    check(R, dev, x, d_out, d_sf, None, BAR["bf16"], heads=[(0, 0), (3, 7), (7, 11)])


def test_bwd_gate_edges(R, dev):
    """g = 0 (alpha = 1, alpha_hat = 0) and tau = 0 (alpha = alpha_hat = 1) on
    some columns; the oracle's reading at g = 0 (g^tau terms 0) on both sides."""
    x = D.make("tiny", B=1, T=40, H=2, dk=16, dv=16)
    x.g[:, :, :, :4] = 0.0
    x.tau[:, :, :, 4:8] = 0.0
    d_out, d_sf = cotangents(x, 12)
    check(R, dev, x, d_out, d_sf, None, BAR["f32"])


def test_bwd_gate_edges_bf16(R, dev):
    """The same edges at the production shape (dk 64, dv 128, bf16 inputs), where
    the sweeps fold g^tau into one exponent and the gradient kernel stages the
    gates through LDS: g = 0, tau = 0 and both (0^0 = 1) on separate columns."""
    x = D.make("layer130m", B=1, T=100, H=2)
    x.g[:, :, 0, :4] = 0
    x.tau[:, :, 1, 4:8] = 0
    x.g[:, :50, :, 8:10] = 0
    x.tau[:, :50, :, 8:10] = 0
    d_out, d_sf = cotangents(x, 15)
    check(R, dev, x, d_out, d_sf, None, BAR["bf16"])


def test_bwd_no_tokens(R, dev):
    x = D.make("tiny", T=0)
    d_out, d_sf = cotangents(x, 13)
    t = [x.torch(n, dev) for n in NAMES]
    dsf = torch.from_numpy(d_sf).to(dev)
    g = R.chunk_bwd(*t, torch.from_numpy(d_out).to(dev), d_final_state=dsf)
    torch.cuda.synchronize()
    assert torch.equal(g["d_initial_state"], dsf)


def test_bwd_deterministic(R, dev):
    x = D.make("layer1p6b", B=1, T=200, H=2)
    d_out, d_sf = cotangents(x, 14)
    t = [x.torch(n, dev) for n in NAMES]
    a = R.chunk_bwd(*t, torch.from_numpy(d_out).to(dev), d_final_state=torch.from_numpy(d_sf).to(dev))
    b = R.chunk_bwd(*t, torch.from_numpy(d_out).to(dev), d_final_state=torch.from_numpy(d_sf).to(dev))
    torch.cuda.synchronize()
    for n in GRADS:
        assert torch.equal(a[n], b[n]), n
