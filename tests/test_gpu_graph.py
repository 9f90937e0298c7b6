"""The entry points inside a captured HIP graph (torch.cuda.CUDAGraph).

The library enqueues only kernel launches on the caller's stream (no memsets,
no allocations, no synchronisation), so a serving loop can capture it.  Each
test runs the call eagerly once, captures the same call on the same buffers,
then replays the graph several times with eager work on those buffers in
between (overwriting the outputs, restoring an in-place state), and checks
every replay against the eager result bit for bit: the kernels are
deterministic for a fixed launch configuration.
"""
import numpy as np
import pytest

import ddts_inputs as D

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

NAMES = ("q", "k", "v", "g", "tau", "beta_hat")
REPLAYS = 3


@pytest.fixture(scope="module")
def R():
    import gated_linear_attention_rodimus_amd as mod
    mod.lib()
    return mod


def capture(fn):
    """Warm fn up on a side stream, then capture it; returns the graph."""
    cur = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(cur)
    with torch.cuda.stream(side):
        fn()
    cur.wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("shape,segments", [((2, 300, 3), 0), ((1, 1100, 2), 0), ((1, 1100, 2), 3)])
def test_chunk_fwd_graph_replays(R, shape, segments):
    B, T, H = shape
    dev = torch.device("cuda:0")
    x = D.make("long_prefill", B=B, T=T, H=H)
    W = x.wl
    t = [x.torch(n, dev) for n in NAMES]
    s0 = torch.from_numpy(x.initial_state).to(dev)
    out = torch.empty(B, T, H, W.dv, device=dev)
    fs = torch.empty(B, H, W.dk, W.dv, device=dev)
    wsb = R.workspace_bytes(B, T, H, W.dk, W.dv, 0, segments)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)

    def call():
        R.chunk_fwd(*t, initial_state=s0, out=out, final_state=fs, workspace=ws, segments=segments)

    call()
    torch.cuda.synchronize()
    ref_o, ref_s = out.clone(), fs.clone()
    g = capture(call)
    for rep in range(REPLAYS):
        out.fill_(float("nan"))
        fs.fill_(float("nan"))
        ws.fill_(255)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o), f"replay {rep}: outputs differ from the eager call"
        assert torch.equal(fs, ref_s), f"replay {rep}: final state differs from the eager call"


def test_decode_step_graph_replays(R):
    dev = torch.device("cuda:0")
    steps, st = D.make_decode_pool("decode_batch")
    ins = [steps[0].torch(n, dev)[:, 0] for n in NAMES]
    S0 = torch.from_numpy(st).to(dev)
    S = S0.clone()
    o = torch.empty(S.shape[0], S.shape[1], S.shape[3], device=dev)

    def call():
        R.decode_step(*ins, S, out=o)

    call()
    torch.cuda.synchronize()
    ref_o, ref_s = o.clone(), S.clone()
    S.copy_(S0)
    g = capture(call)                      # the warm-up and the capture step S twice
    for rep in range(REPLAYS):
        S.copy_(S0)                        # restore the state the eager call started from
        o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o), f"replay {rep}: decode output differs"
        assert torch.equal(S, ref_s), f"replay {rep}: updated state differs"


def test_chunk_bwd_graph_replays(R):
    dev = torch.device("cuda:0")
    x = D.make("layer130m", B=2, T=300, H=2)
    W = x.wl
    t = [x.torch(n, dev) for n in NAMES]
    rng = np.random.default_rng(5)
    d_out = torch.from_numpy(rng.standard_normal((W.B, W.T, W.H, W.dv), dtype=np.float32)).to(dev)
    d_sf = torch.from_numpy(rng.standard_normal((W.B, W.H, W.dk, W.dv), dtype=np.float32)).to(dev)
    ws = torch.empty(R.bwd_workspace_bytes(W.B, W.T, W.H, W.dk, W.dv), dtype=torch.uint8, device=dev)
    ref = R.chunk_bwd(*t, d_out, d_final_state=d_sf, workspace=ws)
    torch.cuda.synchronize()
    ref = {n: a.clone() for n, a in ref.items()}
    held = {}

    def call():
        held.update(R.chunk_bwd(*t, d_out, d_final_state=d_sf, workspace=ws))

    g = capture(call)
    for rep in range(REPLAYS):
        for a in held.values():
            a.fill_(float("nan"))
        ws.fill_(255)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n, a in ref.items():
            assert torch.equal(held[n], a), f"replay {rep}: {n} differs from the eager call"


def test_swska_graph_replays(R):
    """The SW-SKA entry (direct global-to-LDS loads, no scratch) captured and
    replayed: every replay equals the eager call."""
    dev = torch.device("cuda:0")
    x = D.make_swska(B=2, T=777, H=4)
    q, k, v = (x.torch(n, dev) for n in ("q", "k", "v"))
    out = torch.empty(2, 777, 4, x.wl.dv, device=dev)

    def call():
        R.swska_fwd(q, k, v, 200, out=out)

    call()
    torch.cuda.synchronize()
    ref = out.clone()
    g = capture(call)
    for rep in range(REPLAYS):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {rep}: outputs differ from the eager call"
