"""Seeded random shapes through the C ABI against the fp64 oracle.

Each case draws B, T, H, the widths, the input dtype, the chunk length and the
segment count asked for, an initial state or none, a dL/dS_T or none and the
gate mean, and checks the forward (outputs and final state) and the backward
(every gradient).  The cases come from one fixed seed, so every run checks the
same ones; they cover ragged tails, single-token sequences, short sequences
split into more segments than they have chunks, and every (dk, dv) pair.

Bars as in the other parity tests (max |x_hat - x| / RMS(x)): 1e-4 for fp32
inputs, 1e-2 for bf16 inputs (the oracle on the same bf16-rounded values).
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
WIDTHS = (16, 32, 64, 128)


def draw_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        T = int(rng.choice([1, 2, 17, 63, 64, 65, 130, 257, 400]))
        cases.append(dict(
            i=i, B=int(rng.integers(1, 4)), T=T, H=int(rng.integers(1, 4)),
            dk=int(rng.choice(WIDTHS)), dv=int(rng.choice(WIDTHS)),
            dtype="f32" if rng.random() < 0.3 else "bf16",
            chunk=int(rng.choice([0, 16, 32, 64])),
            segments=int(rng.choice([0, 0, 1, 2, 3, 7])),
            s0=bool(rng.random() < 0.5), final=bool(rng.random() < 0.5),
            g_mean=float(rng.choice([-2.0, 0.0, 1.0, 2.0]))))
    return cases


CASES = draw_cases(24, 2024)


def case_id(c):
    return (f"{c['i']}-B{c['B']}T{c['T']}H{c['H']}-{c['dk']}x{c['dv']}-{c['dtype']}"
            f"-c{c['chunk']}s{c['segments']}{'-s0' if c['s0'] else ''}{'-dsf' if c['final'] else ''}")


@pytest.fixture(scope="module")
def R():
    import gated_linear_attention_rodimus_amd as mod
    mod.lib()
    return mod


@pytest.mark.parametrize("c", CASES, ids=case_id)
def test_random_shape(R, c):
    dev = torch.device("cuda:0")
    x = D.make("layer1p6b", sub=c["i"], B=c["B"], T=c["T"], H=c["H"], dk=c["dk"], dv=c["dv"],
               dtype=c["dtype"], g_mean=c["g_mean"], s0_std=0.1 if c["s0"] else 0.0)
    bar = BAR[c["dtype"]]
    W = x.wl
    s0 = x.initial_state
    ins = [x.f32(n) for n in NAMES]
    t = [x.torch(n, dev) for n in NAMES]
    tt = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)

    # forward
    o, sf = R.chunk_fwd(*t, initial_state=tt(s0), output_final_state=True, chunk=c["chunk"],
                        segments=c["segments"])
    torch.cuda.synchronize()
    ro, rs = oracle.fwd(*ins, s0)
    eo = oracle.rel_to_rms_error(o.cpu().numpy(), ro)
    es = oracle.rel_to_rms_error(sf.cpu().numpy(), rs)
    assert eo <= bar and es <= bar, (eo, es)

    # backward
    rng = np.random.default_rng(100 + c["i"])
    d_out = rng.standard_normal((W.B, W.T, W.H, W.dv), dtype=np.float32)
    d_sf = rng.standard_normal((W.B, W.H, W.dk, W.dv), dtype=np.float32) if c["final"] else None
    g = R.chunk_bwd(*t, tt(d_out), initial_state=tt(s0), d_final_state=tt(d_sf))
    torch.cuda.synchronize()
    r = oracle.bwd(*ins, d_out, s0, d_sf)
    errs = {n: oracle.rel_to_rms_error(g[n].cpu().numpy(), r[n]) for n in GRADS}
    bad = {n: e for n, e in errs.items() if not e <= bar}
    assert not bad, f"errors above {bar}: {bad} (all: {errs})"


def test_random_shape_sweep(R):
    """A wider sweep from a second seed: 160 forward shapes (outputs and final
    states) and the backward of every other one up to T = 257, each against the
    oracle at its bar; reports the worst error as a fraction of the bar."""
    dev = torch.device("cuda:0")
    tt = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)
    worst, bad = {}, []
    for c in draw_cases(160, 777):
        x = D.make("layer1p6b", sub=1000 + c["i"], B=c["B"], T=c["T"], H=c["H"], dk=c["dk"],
                   dv=c["dv"], dtype=c["dtype"], g_mean=c["g_mean"], s0_std=0.1 if c["s0"] else 0.0)
        bar = BAR[c["dtype"]]
        s0 = x.initial_state
        ins = [x.f32(n) for n in NAMES]
        t = [x.torch(n, dev) for n in NAMES]
        o, sf = R.chunk_fwd(*t, initial_state=tt(s0), output_final_state=True, chunk=c["chunk"],
                            segments=c["segments"])
        torch.cuda.synchronize()
        ro, rs = oracle.fwd(*ins, s0)
        errs = {"out": oracle.rel_to_rms_error(o.cpu().numpy(), ro),
                "state": oracle.rel_to_rms_error(sf.cpu().numpy(), rs)}
        if c["i"] % 2 == 0 and c["T"] <= 257:
            d_out = np.random.default_rng(c["i"]).standard_normal(ro.shape).astype(np.float32)
            g = R.chunk_bwd(*t, tt(d_out), initial_state=tt(s0))
            torch.cuda.synchronize()
            r = oracle.bwd(*ins, d_out, s0, None)
            errs.update({n: oracle.rel_to_rms_error(g[n].cpu().numpy(), r[n]) for n in GRADS})
        for n, e in errs.items():
            worst[c["dtype"]] = max(worst.get(c["dtype"], 0.0), e / bar)
            if not e <= bar:
                bad.append((case_id(c), n, e))
    print(f"[sweep] worst error as a fraction of the bar: {worst}", flush=True)
    assert not bad, bad
