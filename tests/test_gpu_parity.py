"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Bars (max |x_hat - x| / RMS(x), for outputs and states separately): 1e-4 for
fp32 inputs, 1e-2 for bf16 inputs, the oracle running on the same bf16-rounded
values.  Every workload runs at its full size; the oracle checks all of it
where it finishes in seconds and a sample of heads / sequences otherwise.
"""
import numpy as np
import pytest

import ddts_inputs as D
import oracle

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

NAMES = ("q", "k", "v", "g", "tau", "beta_hat")
BAR = {"bf16": 1e-2, "f32": 1e-4}


@pytest.fixture(scope="module")
def R():
    import gated_linear_attention_rodimus_amd as mod
    mod.lib()
    return mod


@pytest.fixture(scope="module")
def dev():
    return torch.device("cuda:0")


def err(a, b):
    return oracle.rel_to_rms_error(a, b)


def to_dev(x, dev):
    return [x.torch(n, dev) for n in NAMES]


def ref(x, s0=None, heads=None):
    """Oracle on all (b, h) pairs, or on a list of (b, h) pairs."""
    ins = [x.f32(n) for n in NAMES]
    if heads is None:
        return oracle.fwd(*ins, s0)
    outs, states = [], []
    for (b, h) in heads:
        sl = [np.ascontiguousarray(a[b:b + 1, :, h:h + 1]) for a in ins]
        s = None if s0 is None else np.ascontiguousarray(s0[b:b + 1, h:h + 1])
        o, sf = oracle.fwd(*sl, s)
        outs.append(o[0, :, 0])
        states.append(sf[0, 0])
    return outs, states


def run_gpu(R, x, dev, s0=None, chunk=0, segments=0, final=True):
    t = to_dev(x, dev)
    s0d = None if s0 is None else torch.from_numpy(np.ascontiguousarray(s0, np.float32)).to(dev)
    o, sf = R.chunk_fwd(*t, initial_state=s0d, output_final_state=final, chunk=chunk,
                        segments=segments)
    torch.cuda.synchronize()
    return o.cpu().numpy(), (None if sf is None else sf.cpu().numpy())


def check_full(R, x, dev, s0=None, chunk=0, segments=0, label=""):
    o, sf = run_gpu(R, x, dev, s0, chunk, segments)
    ro, rs = ref(x, s0)
    bar = BAR[x.wl.dtype]
    eo, es = err(o, ro), err(sf, rs)
    print(f"[{label}] out err {eo:.2e} state err {es:.2e} bar {bar:g}", flush=True)
    assert np.isfinite(o).all() and np.isfinite(sf).all()
    assert eo <= bar and es <= bar
    return eo, es


# ---------------------------------------------------------------- the five workloads


def test_tiny_fp32(R, dev):
    x = D.make("tiny")
    check_full(R, x, dev, chunk=16, label="tiny B1 T64 H2 16x16 C16 fp32")


def test_layer130m_full(R, dev):
    x = D.make("layer130m")
    check_full(R, x, dev, label="layer130m B8 T2048 H12 64x128 bf16")


def test_layer1p6b_full_with_final_state(R, dev):
    x = D.make("layer1p6b")
    check_full(R, x, dev, label="layer1p6b B4 T4096 H16 64x128 bf16 + S_T")


@pytest.mark.parametrize("dk", [16, 32, 64])
def test_whole_head_tile_segmented(R, dev, dk):
    # 16 heads of dv = 128 over 8,229 tokens (ragged against 64-token chunks):
    # the planner takes the whole-head 128-column tile, 15 segments, with an
    # initial state and S_T
    x = D.make("long_prefill", B=1, T=8192 + 37, H=16, dk=dk)
    p = R.chunk_fwd_plan(1, x.wl.T, 16, dk, 128)
    assert p["dv_tile"] == 128 and p["segments"] > 1, p
    check_full(R, x, dev, s0=x.initial_state, label=f"whole-head dk {dk} {p}")


def test_whole_head_tile_batched_ragged(R, dev):
    # two sequences of 8,293 tokens x 8 heads (16 head-sequences, ragged against
    # 64- and 32-token chunks): whole-head tiles, 15 segments of 9 chunks,
    # transfers of half-length chunks cut in 2; initial state and S_T per (b, h)
    x = D.make("long_prefill", B=2, T=8192 + 101, H=8)
    p = R.chunk_fwd_plan(2, x.wl.T, 8, 64, 128)
    assert p["dv_tile"] == 128 and p["segments"] > 1 and p["transfer_pieces"] == 2, p
    check_full(R, x, dev, s0=x.initial_state, label=f"whole-head B2 H8 {p}")


@pytest.mark.timeout(600)
def test_long_prefill_full(R, dev):
    x = D.make("long_prefill")
    assert R.workspace_bytes(1, 65536, 16, 64, 128) > 0      # segmented path
    check_full(R, x, dev, s0=x.initial_state, label="long_prefill B1 T65536 H16 S0")


def test_decode_batch_1000_steps(R, dev):
    sets, st = D.make_decode_pool("decode_batch")
    N, H = st.shape[:2]
    steps = D.WORKLOADS["decode_batch"].steps
    dsets = [[x.torch(n, dev)[:, 0] for n in NAMES] for x in sets]
    S = torch.from_numpy(st).to(dev)
    check_at = {1, 10, 100, steps}
    outs = {}
    for s in range(1, steps + 1):
        o = R.decode_step(*dsets[(s - 1) % len(sets)], S)
        if s in check_at:
            outs[s] = o.cpu().numpy()
    S_gpu = S.cpu().numpy()
    f32sets = [[x.f32(n)[:, 0] for n in NAMES] for x in sets]
    # full batch for the first 10 steps
    Sref = st.astype(np.float64)
    for s in range(1, 11):
        ro, Sref = oracle.decode(*f32sets[(s - 1) % len(sets)], Sref)
        if s in outs:
            e = err(outs[s], ro)
            print(f"[decode full batch] step {s} out err {e:.2e}", flush=True)
            assert e <= 1e-2
    # 64 sampled (n, h) sequences over all steps, and their final states
    rng = np.random.default_rng(0)
    pick = rng.choice(N * H, size=64, replace=False)
    nn, hh = pick // H, pick % H
    Sref = st[nn, hh][:, None].astype(np.float64)              # [64, 1, dk, dv]
    picked = [[a[nn, hh][:, None] for a in fs] for fs in f32sets]
    for s in range(1, steps + 1):
        ro, Sref = oracle.decode(*picked[(s - 1) % len(sets)], Sref)
        if s in outs:
            e = err(outs[s][nn, hh], ro[:, 0])
            print(f"[decode sampled] step {s} out err {e:.2e}", flush=True)
            assert e <= 1e-2
    e = err(S_gpu[nn, hh], Sref[:, 0])
    print(f"[decode sampled] final state err {e:.2e}", flush=True)
    assert e <= 1e-2


def run_decode_steps(R, dev, x, s0, steps):
    """decode_step token by token against the oracle's decode; returns the worst
    output error and the final-state error."""
    t = to_dev(x, dev)
    S = torch.from_numpy(np.ascontiguousarray(s0, np.float32)).to(dev)
    Sref = s0.astype(np.float64)
    worst = 0.0
    for s in range(steps):
        o = R.decode_step(*(a[:, s].contiguous() for a in t), S)
        ro, Sref = oracle.decode(*(np.ascontiguousarray(x.f32(n)[:, s]) for n in NAMES), Sref)
        worst = max(worst, err(o.cpu().numpy(), ro))
    return worst, err(S.cpu().numpy(), Sref)


@pytest.mark.parametrize("dk", [16, 32, 64, 128])
@pytest.mark.parametrize("dv", [16, 32, 64, 128])
def test_decode_all_widths_bf16(R, dev, dk, dv):
    """Decode steps at every width: 5 sequences x 3 heads, so the small heads,
    several state slices to a workgroup, end on a partly filled workgroup."""
    x = D.make("layer1p6b", B=5, T=6, H=3, dk=dk, dv=dv)
    s0 = D.make("long_prefill", B=5, T=1, H=3, dk=dk, dv=dv).initial_state
    eo, es = run_decode_steps(R, dev, x, s0, 6)
    assert eo <= BAR["bf16"] and es <= BAR["bf16"], (eo, es)


@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (64, 128), (128, 32)])
def test_decode_fp32_inputs(R, dev, dk, dv):
    x = D.make("tiny", B=5, T=6, H=3, dk=dk, dv=dv)
    s0 = D.make("long_prefill", B=5, T=1, H=3, dk=dk, dv=dv).initial_state
    eo, es = run_decode_steps(R, dev, x, s0, 6)
    assert eo <= BAR["f32"] and es <= BAR["f32"], (eo, es)


# ---------------------------------------------------------------- shapes, chunking, paths


@pytest.mark.parametrize("dk", [16, 32, 64, 128])
@pytest.mark.parametrize("dv", [16, 32, 64, 128])
def test_all_widths_bf16(R, dev, dk, dv):
    x = D.make("layer1p6b", B=2, T=77, H=3, dk=dk, dv=dv)
    s0 = D.make("long_prefill", B=2, T=1, H=3, dk=dk, dv=dv).initial_state
    check_full(R, x, dev, s0=s0, label=f"widths {dk}x{dv} bf16 T77")


@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (64, 128), (128, 32)])
@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_fp32_inputs(R, dev, dk, dv, chunk):
    x = D.make("tiny", B=2, T=90, H=2, dk=dk, dv=dv)
    check_full(R, x, dev, s0=D.make("long_prefill", B=2, T=1, H=2, dk=dk, dv=dv).initial_state,
               chunk=chunk, label=f"fp32 {dk}x{dv} C{chunk}")


@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_chunk_size_invariance(R, dev, chunk):
    x = D.make("layer130m", B=2, T=333, H=2)
    check_full(R, x, dev, chunk=chunk, label=f"chunk {chunk}")


def test_chunk_sizes_agree_with_each_other(R, dev):
    x = D.make("layer130m", B=1, T=500, H=4)
    outs = [run_gpu(R, x, dev, chunk=c)[0] for c in (16, 32, 64)]
    for o in outs[1:]:
        assert err(o, outs[0]) <= 1e-3


@pytest.mark.parametrize("segments", [1, 2, 3, 5, 9])
def test_segmented_path(R, dev, segments):
    x = D.make("long_prefill", B=2, T=1500, H=2)
    check_full(R, x, dev, s0=x.initial_state, segments=segments, label=f"segments {segments}")


@pytest.mark.parametrize("T,segments", [(4096, 2), (6144, 3), (94 * 64 + 37, 3)])
def test_segmented_transfers_in_four_pieces(R, dev, T, segments):
    # 32 chunks per segment: each transfer before the last segment is cut
    # into 4 pieces of 8 chunks (bf16 transfers run two workgroups per CU);
    # the last case ends in a shorter segment with a ragged last chunk
    x = D.make("long_prefill", B=1, T=T, H=2)
    check_full(R, x, dev, s0=x.initial_state, segments=segments, label=f"T {T} segments {segments}")


@pytest.mark.parametrize("T", [1024, 1000])
def test_auto_plan_segmented_short_chunks(R, dev, T):
    # 2 heads x 2 dv tiles fill few CUs, so the planner segments the sequence
    # and, for bf16 inputs, takes 32-token chunks (4 segments of 8 chunks)
    x = D.make("long_prefill", B=1, T=T, H=2)
    check_full(R, x, dev, s0=x.initial_state, label=f"auto plan T {T}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("dk,dv", [(16, 16), (16, 128), (32, 64), (64, 16), (128, 32), (128, 128)])
def test_auto_plan_segmented_all_widths(R, dev, dk, dv, dtype):
    # one (b, h) pair over 1100 tokens: the planner segments it (bf16 at
    # dk <= 64: 32-token chunks, two workgroups per CU; otherwise the longest
    # chunk that fits); the plan it reports is the one the call runs
    x = D.make("long_prefill", B=1, T=1100, H=1, dk=dk, dv=dv, dtype=dtype)
    p = R.chunk_fwd_plan(1, 1100, 1, dk, dv, dtype=dtype)
    assert p["segments"] > 1
    assert p["chunk"] == (32 if dtype == "bf16" and dk <= 64 else 64 if dk <= 64 else 32)
    check_full(R, x, dev, s0=x.initial_state, label=f"auto plan {dk}x{dv} {dtype} {p}")


def test_split_sequence_carry_over(R, dev):
    x = D.make("layer1p6b", B=2, T=700, H=3)
    ro, rs = ref(x)
    t = to_dev(x, dev)
    T1 = 259
    first = [a[:, :T1].contiguous() for a in t]
    second = [a[:, T1:].contiguous() for a in t]
    o1, s1 = R.chunk_fwd(*first, output_final_state=True)
    o2, s2 = R.chunk_fwd(*second, initial_state=s1, final_state=s1)     # in place
    torch.cuda.synchronize()
    o = torch.cat([o1, o2], 1).cpu().numpy()
    eo, es = err(o, ro), err(s2.cpu().numpy(), rs)
    print(f"[carry-over T1={T1}] out {eo:.2e} state {es:.2e}", flush=True)
    assert eo <= 1e-2 and es <= 1e-2


def test_prefill_equals_token_by_token_decode(R, dev):
    x = D.make("layer1p6b", B=3, T=40, H=2)
    t = to_dev(x, dev)
    o_pre, s_pre = R.chunk_fwd(*t, output_final_state=True)
    S = torch.zeros(3, 2, 64, 128, device=dev)
    outs = []
    for s in range(40):
        outs.append(R.decode_step(*(a[:, s].contiguous() for a in t), S))
    torch.cuda.synchronize()
    o_dec = torch.stack(outs, 1).cpu().numpy()
    e1, e2 = err(o_dec, o_pre.cpu().numpy()), err(S.cpu().numpy(), s_pre.cpu().numpy())
    print(f"[prefill vs decode] out {e1:.2e} state {e2:.2e}", flush=True)
    assert e1 <= 1e-2 and e2 <= 1e-2


def test_prefill_then_decode_matches_oracle(R, dev):
    x = D.make("layer130m", B=2, T=130, H=2)
    ro, _ = ref(x)
    t = to_dev(x, dev)
    T1 = 100
    _, S = R.chunk_fwd(*(a[:, :T1].contiguous() for a in t), output_final_state=True)
    outs = [R.decode_step(*(a[:, s].contiguous() for a in t), S) for s in range(T1, 130)]
    torch.cuda.synchronize()
    e = err(torch.stack(outs, 1).cpu().numpy(), ro[:, T1:])
    assert e <= 1e-2


@pytest.mark.parametrize("segments", [1, 4])
def test_bitwise_deterministic(R, dev, segments):
    x = D.make("long_prefill", B=1, T=3000, H=3)
    a = run_gpu(R, x, dev, s0=x.initial_state, segments=segments)
    b = run_gpu(R, x, dev, s0=x.initial_state, segments=segments)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_canary_padded_outputs(R, dev):
    x = D.make("layer130m", B=2, T=201, H=3)
    t = to_dev(x, dev)
    n_out = 2 * 201 * 3 * 128
    n_st = 2 * 3 * 64 * 128
    pad = 4096
    buf = torch.full((n_out + 2 * pad,), float("nan"), device=dev)
    sbuf = torch.full((n_st + 2 * pad,), float("nan"), device=dev)
    out = buf[pad:pad + n_out].view(2, 201, 3, 128)
    fs = sbuf[pad:pad + n_st].view(2, 3, 64, 128)
    for seg in (1, 3):
        buf.fill_(float("nan")); sbuf.fill_(float("nan"))
        R.chunk_fwd(*t, out=out, final_state=fs, segments=seg)
        torch.cuda.synchronize()
        assert torch.isnan(buf[:pad]).all() and torch.isnan(buf[pad + n_out:]).all()
        assert torch.isnan(sbuf[:pad]).all() and torch.isnan(sbuf[pad + n_st:]).all()
        assert torch.isfinite(out).all() and torch.isfinite(fs).all()
    S = torch.zeros(6 * 64 * 128 + 2 * pad, device=dev)
    S[:pad] = float("nan"); S[-pad:] = float("nan")
    ob = torch.full((6 * 128 + 2 * pad,), float("nan"), device=dev)
    st = S[pad:-pad].view(2, 3, 64, 128)
    o = ob[pad:-pad].view(2, 3, 128)
    R.decode_step(*(a[:, 0].contiguous() for a in t), st, out=o)
    torch.cuda.synchronize()
    assert torch.isnan(S[:pad]).all() and torch.isnan(S[-pad:]).all()
    assert torch.isnan(ob[:pad]).all() and torch.isnan(ob[-pad:]).all()
    assert torch.isfinite(o).all()


# ---------------------------------------------------------------- edge cases


def test_empty_sequence_copies_state(R, dev):
    x = D.make("layer130m", B=2, T=0, H=2)
    t = to_dev(x, dev)
    s0 = torch.randn(2, 2, 64, 128, device=dev)
    o, sf = R.chunk_fwd(*t, initial_state=s0, output_final_state=True)
    torch.cuda.synchronize()
    assert o.numel() == 0 and torch.equal(sf, s0)
    o, sf = R.chunk_fwd(*t, output_final_state=True)
    torch.cuda.synchronize()
    assert torch.count_nonzero(sf) == 0


@pytest.mark.parametrize("T", [1, 2, 15, 63, 64, 65, 129])
def test_short_and_ragged_lengths(R, dev, T):
    x = D.make("layer130m", B=2, T=T, H=2)
    check_full(R, x, dev, s0=D.make("long_prefill", B=2, T=1, H=2).initial_state,
               label=f"T={T}")


def test_g_zero_keeps_state(R, dev):
    """g = 0: alpha = 1 and alpha_hat = 0, so S_T = S_0 and o_t = S_0^T q_t."""
    x = D.make("layer1p6b", B=1, T=150, H=2)
    x.g[...] = 0
    s0 = D.make("long_prefill", B=1, T=1, H=2).initial_state
    o, sf = run_gpu(R, x, dev, s0=s0)
    assert err(sf, s0) <= 1e-6
    want = np.einsum("bthi,bhij->bthj", x.f32("q").astype(np.float64), s0.astype(np.float64))
    assert err(o, want) <= 1e-2


def test_tau_zero_is_linear_attention(R, dev):
    """tau = 0 gives alpha = alpha_hat = 1 (also at g = 0, where 0^0 = 1)."""
    x = D.make("layer1p6b", B=1, T=120, H=2)
    x.tau[...] = 0
    x.g[0, :10] = 0
    check_full(R, x, dev, label="tau = 0")


def test_slow_decay_variant(R, dev):
    """g = sigmoid(N(-2, 1)) (mean alpha ~0.93): long memory, larger state values."""
    x = D.make("long_prefill", B=1, T=4000, H=4, g_mean=-2.0)
    check_full(R, x, dev, s0=x.initial_state, label="slow decay")


def test_explicit_workspace(R, dev):
    x = D.make("long_prefill", B=1, T=2000, H=2)
    t = to_dev(x, dev)
    wsb = R.workspace_bytes(1, 2000, 2, 64, 128, 0, 4)
    ws = torch.empty(wsb + 256, dtype=torch.uint8, device=dev)
    o, sf = R.chunk_fwd(*t, output_final_state=True, segments=4, workspace=ws)
    torch.cuda.synchronize()
    ro, rs = ref(x)
    assert err(o.cpu().numpy(), ro) <= 1e-2 and err(sf.cpu().numpy(), rs) <= 1e-2
