"""GPU: the constant cost of a decode step (O(1) per-token generation, abstract
of the Rodimus paper page; the rebuttal's answer on barriers to adoption).

The state a prefill hands to decoding has the same size whatever the prefill
length, and a decode step costs the same at every step index and after any
prefill length (timed with HIP events on the launch stream; medians of
windows, a generous 30 % band so that clock noise does not fail the test).
Inputs are random draws made on the GPU: only sizes matter for timing.
"""
import pytest

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

N, H, DK, DV = 256, 16, 64, 128


@pytest.fixture(scope="module")
def R():
    import gated_linear_attention_rodimus_amd as mod
    mod.lib()
    return mod


def _tok(shape_k, shape_v, gen):
    dev = torch.device("cuda:0")
    bf = torch.bfloat16
    q = (torch.randn(shape_k, device=dev, generator=gen) / 8).to(bf)
    k = (torch.randn(shape_k, device=dev, generator=gen) / 8).to(bf)
    v = (torch.randn(shape_v, device=dev, generator=gen) / 8).to(bf)
    g = torch.sigmoid(torch.randn(shape_k, device=dev, generator=gen)).to(bf)
    tau = torch.sigmoid(torch.randn(shape_k, device=dev, generator=gen)).to(bf)
    beta = torch.sigmoid(torch.randn(shape_v, device=dev, generator=gen)).to(bf)
    return q, k, v, g, tau, beta


def _step_times(R, state, n_steps, gen):
    ins = _tok((N, H, DK), (N, H, DV), gen)
    out = torch.empty(N, H, DV, device=state.device)
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n_steps + 1)]
    R.decode_step(*ins, state, out=out)
    torch.cuda.synchronize()
    ev[0].record(stream)
    for s in range(n_steps):
        R.decode_step(*ins, state, out=out)
        ev[s + 1].record(stream)
    torch.cuda.synchronize()
    return [ev[s].elapsed_time(ev[s + 1]) for s in range(n_steps)]


def _median(x):
    x = sorted(x)
    return x[len(x) // 2]


def test_state_size_independent_of_prefill_length(R):
    gen = torch.Generator(device="cuda:0").manual_seed(3)
    sizes = set()
    for T0 in (1, 64, 1000):
        q, k, v, g, tau, beta = _tok((2, T0, 4, DK), (2, T0, 4, DV), gen)
        _, S = R.chunk_fwd(q, k, v, g, tau, beta, output_final_state=True)
        sizes.add((tuple(S.shape), S.numel() * S.element_size()))
    assert sizes == {((2, 4, DK, DV), 2 * 4 * DK * DV * 4)}


def test_decode_step_time_flat_over_step_index(R):
    gen = torch.Generator(device="cuda:0").manual_seed(4)
    state = torch.randn(N, H, DK, DV, device="cuda:0", generator=gen) * 0.1
    t = _step_times(R, state, 1000, gen)
    early, late = _median(t[:100]), _median(t[-100:])
    assert max(early, late) / min(early, late) < 1.3, (early, late)


def test_decode_step_time_flat_over_prefill_length(R):
    gen = torch.Generator(device="cuda:0").manual_seed(5)
    med = {}
    for T0 in (16, 2048):
        q, k, v, g, tau, beta = _tok((N, T0, H, DK), (N, T0, H, DV), gen)
        _, S = R.chunk_fwd(q, k, v, g, tau, beta, output_final_state=True)
        del q, k, v, g, tau, beta
        med[T0] = _median(_step_times(R, S, 300, gen))
    assert max(med.values()) / min(med.values()) < 1.3, med
