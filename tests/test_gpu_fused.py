"""GPU parity of the fused steps around the recurrence (beta_hat from low-rank
factors, ShortConv of q, k, v, the feedthrough d) through the C ABI, against
the fp64 oracle's fwd_fused / decode_fused on the same bf16-rounded (or fp32)
values.  Bars as everywhere: max |x_hat - x| / RMS(x) <= 1e-2 for bf16
inputs, 1e-4 for fp32, outputs and states separately."""
import numpy as np
import pytest

import ddts_inputs as D
import oracle

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

BAR = {"bf16": 1e-2, "f32": 1e-4}


@pytest.fixture(scope="module")
def R():
    import gated_linear_attention_rodimus_amd as mod
    mod.lib()
    return mod


DEV = None


def dev():
    return torch.device("cuda:0")


def run(R, f, use_u=True, use_d=True, use_conv=True, s0=None, final=True, chunk=0, segments=0):
    t = {n: f.torch(n, dev()) for n in ("q", "k", "v", "g", "tau", "beta_hat", "u", "w", "d",
                                         "conv_q", "conv_k", "conv_v")}
    s0d = None if s0 is None else torch.from_numpy(np.ascontiguousarray(s0, np.float32)).to(dev())
    q, k, v = t["q"], t["k"], t["v"]
    W = f.conv_width
    if not use_conv:                       # drop the history rows: plain q, k, v
        q, k, v = (x[:, W - 1:].contiguous() for x in (q, k, v))
    o, sf = R.chunk_fwd_fused(q, k, v, t["g"], t["tau"],
                              beta_hat=None if use_u else t["beta_hat"],
                              u=t["u"] if use_u else None, w=t["w"] if use_u else None,
                              d=t["d"] if use_d else None,
                              conv=(t["conv_q"], t["conv_k"], t["conv_v"]) if use_conv else None,
                              initial_state=s0d, output_final_state=final, chunk=chunk,
                              segments=segments)
    torch.cuda.synchronize()
    return o.cpu().numpy(), (None if sf is None else sf.cpu().numpy())


def ref(f, use_u=True, use_d=True, use_conv=True, s0=None):
    W = f.conv_width
    q, k, v = f.f32("q"), f.f32("k"), f.f32("v")
    if not use_conv:
        q, k, v = q[:, W - 1:], k[:, W - 1:], v[:, W - 1:]
    return oracle.fwd_fused(q, k, v, f.f32("g"), f.f32("tau"),
                            beta_hat=None if use_u else f.f32("beta_hat"),
                            u=f.f32("u") if use_u else None, w=f.f32("w") if use_u else None,
                            d=f.d if use_d else None,
                            conv=(f.conv_q, f.conv_k, f.conv_v) if use_conv else None,
                            initial_state=s0)


def check(R, f, label, **kw):
    s0 = kw.pop("s0", None)
    chunk = kw.pop("chunk", 0)
    segments = kw.pop("segments", 0)
    o, sf = run(R, f, s0=s0, chunk=chunk, segments=segments, **kw)
    ro, rs = ref(f, s0=s0, **kw)
    bar = BAR[f.base.wl.dtype]
    eo, es = oracle.rel_to_rms_error(o, ro), oracle.rel_to_rms_error(sf, rs)
    print(f"[{label}] out err {eo:.2e} state err {es:.2e} bar {bar:g}", flush=True)
    assert np.isfinite(o).all() and np.isfinite(sf).all()
    assert eo <= bar and es <= bar
    return o, sf


def test_layer130m_full_with_lowrank_beta(R):
    """The 130M layer (B8 T2048 H12) fed its rank-16 factors u, w instead of
    a dense beta_hat: 224 fewer bytes per token and head."""
    f = D.make_fused("layer130m", conv_width=1)
    check(R, f, "layer130m u,w rank16", use_d=False, use_conv=False)


@pytest.mark.parametrize("rank", [16, 32])
@pytest.mark.parametrize("W", [2, 3, 4])
def test_all_steps_ragged(R, rank, W):
    f = D.make_fused("layer130m", conv_width=W, rank=rank, B=2, T=333, H=3)
    rng = np.random.default_rng(W * 100 + rank)
    s0 = (0.1 * rng.standard_normal((2, 3, 64, 128))).astype(np.float32)
    check(R, f, f"all steps W{W} rank{rank} B2 T333 H3", s0=s0)


@pytest.mark.parametrize("which", ["u", "d", "conv"])
def test_each_step_alone(R, which):
    f = D.make_fused("layer130m", conv_width=4, B=1, T=200, H=4)
    check(R, f, f"only {which}", use_u=which == "u", use_d=which == "d", use_conv=which == "conv")


def test_no_history_is_a_sequence_start(R):
    f = D.make_fused("layer130m", conv_width=4, B=2, T=97, H=2, history=False)
    check(R, f, "zero history")


@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (128, 128), (64, 32)])
def test_widths(R, dk, dv):
    f = D.make_fused("layer130m", conv_width=3, B=1, T=150, H=2, dk=dk, dv=dv)
    check(R, f, f"widths dk{dk} dv{dv}")


def test_segmented_long_prefill_slice(R):
    """The long prefill's shape class (few heads, long sequence, initial
    state): the segmented plan, with every fused step in both passes."""
    f = D.make_fused("long_prefill", conv_width=4, T=8192 + 5, H=4)
    p = R.fused_workspace_bytes(1, 8192 + 5, 4, 64, 128)
    assert p > 0
    check(R, f, "segmented long prefill slice", s0=f.base.initial_state)


def test_explicit_segments_and_chunks(R):
    f = D.make_fused("layer130m", conv_width=4, B=1, T=700, H=2)
    for chunk, seg in ((16, 3), (32, 5), (64, 2), (32, 1)):
        check(R, f, f"chunk {chunk} segments {seg}", chunk=chunk, segments=seg)


@pytest.mark.parametrize("dk,dv", [(32, 16), (128, 32), (64, 128)])
def test_fp32_inputs(R, dk, dv):
    """fp32 inputs with every step on (the ShortConv windows read per lane, a
    run of tokens and its history rows at a time), ragged T, at three widths."""
    f = D.make_fused("tiny", conv_width=4, T=77, H=2, dk=dk, dv=dv)
    rng = np.random.default_rng(1)
    s0 = (0.1 * rng.standard_normal((1, 2, dk, dv))).astype(np.float32)
    check(R, f, f"fp32 all steps {dk}x{dv}", s0=s0)


def test_all_steps_off_matches_plain_forward(R):
    """With no step switched on the fused kernels reproduce the plain forward
    bit for bit (same plan on this one-sweep shape)."""
    x = D.make("layer130m", B=2, T=300, H=12)
    t = [x.torch(n, dev()) for n in ("q", "k", "v", "g", "tau", "beta_hat")]
    o1, s1 = R.chunk_fwd(*t, output_final_state=True)
    o2, s2 = R.chunk_fwd_fused(*t, output_final_state=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


# The fused steps without a ShortConv (u, w and d, q, k, v without history
# rows) run kernels compiled without the convolution; these cases cover them
# over the shapes, dtypes and plans the cases above cover with it.
NOCONV = [
    ("ragged rank16", "layer130m", dict(B=2, T=333, H=3), 16, True, 0, 0),
    ("ragged rank32", "layer130m", dict(B=2, T=333, H=3), 32, True, 0, 0),
    ("dk16 dv16", "layer130m", dict(B=1, T=150, H=2, dk=16, dv=16), 16, False, 0, 0),
    ("dk32 dv64", "layer130m", dict(B=1, T=150, H=2, dk=32, dv=64), 16, False, 0, 0),
    ("dk128 dv128", "layer130m", dict(B=1, T=150, H=2, dk=128, dv=128), 16, True, 0, 0),
    ("dk64 dv32", "layer130m", dict(B=1, T=150, H=2, dk=64, dv=32), 16, False, 0, 0),
    ("fp32", "tiny", dict(T=77, H=2, dk=32, dv=16), 16, True, 0, 0),
    ("segmented long prefill slice", "long_prefill", dict(T=8192 + 5, H=4), 16, True, 0, 0),
    ("chunk 16 segments 3", "layer130m", dict(B=1, T=700, H=2), 16, False, 16, 3),
    ("chunk 32 segments 5", "layer130m", dict(B=1, T=700, H=2), 16, False, 32, 5),
    ("chunk 64 segments 2", "layer130m", dict(B=1, T=700, H=2), 16, True, 64, 2),
]


@pytest.mark.parametrize("label,wl,shape,rank,with_s0,chunk,segments", NOCONV,
                         ids=[c[0].replace(" ", "_") for c in NOCONV])
def test_steps_without_conv(R, label, wl, shape, rank, with_s0, chunk, segments):
    f = D.make_fused(wl, conv_width=1, rank=rank, **shape)
    s0 = None
    if with_s0:
        b = f.base.wl
        rng = np.random.default_rng(len(label))
        s0 = (0.1 * rng.standard_normal((b.B, b.H, b.dk, b.dv))).astype(np.float32)
    check(R, f, f"no conv: {label}", use_conv=False, s0=s0, chunk=chunk, segments=segments)


def draw_fused_cases(n, seed):
    """Seeded random shapes of the fused forward: widths, dtype, chunk and
    segment counts asked for, the ShortConv width (1: the kernels without it),
    which of u w and d are on, the rank and the gate mean."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        cases.append(dict(
            i=i, B=int(rng.integers(1, 3)), T=int(rng.choice([1, 5, 63, 64, 65, 129, 300])),
            H=int(rng.integers(1, 4)), dk=int(rng.choice([16, 32, 64, 128])),
            dv=int(rng.choice([16, 32, 64, 128])),
            dtype="f32" if rng.random() < 0.25 else "bf16",
            chunk=int(rng.choice([0, 16, 32, 64])), segments=int(rng.choice([0, 0, 1, 2, 5])),
            W=int(rng.choice([1, 1, 2, 3, 4])), use_u=bool(rng.random() < 0.7),
            use_d=bool(rng.random() < 0.5), rank=int(rng.choice([16, 32])),
            s0=bool(rng.random() < 0.5), g_mean=float(rng.choice([0.0, 1.0, 2.0]))))
    return cases


FUSED_CASES = draw_fused_cases(20, 77)


def fused_case_id(c):
    return (f"{c['i']}-B{c['B']}T{c['T']}H{c['H']}-{c['dk']}x{c['dv']}-{c['dtype']}"
            f"-c{c['chunk']}s{c['segments']}-W{c['W']}{'-u' + str(c['rank']) if c['use_u'] else ''}"
            f"{'-d' if c['use_d'] else ''}{'-s0' if c['s0'] else ''}")


@pytest.mark.parametrize("c", FUSED_CASES, ids=fused_case_id)
def test_random_shapes(R, c):
    """Both fused kernel families (with the ShortConv when W > 1, without it
    otherwise) on seeded random shapes, dtypes and plans."""
    print(f"[fused random {c}]", flush=True)
    f = D.make_fused("layer130m", conv_width=c["W"], rank=c["rank"], B=c["B"], T=c["T"], H=c["H"],
                     dk=c["dk"], dv=c["dv"], dtype=c["dtype"], g_mean=c["g_mean"])
    s0 = None
    if c["s0"]:
        rng = np.random.default_rng(1000 + c["i"])
        s0 = (0.1 * rng.standard_normal((c["B"], c["H"], c["dk"], c["dv"]))).astype(np.float32)
    check(R, f, f"random {c['i']}", use_u=c["use_u"], use_d=c["use_d"], use_conv=c["W"] > 1,
          s0=s0, chunk=c["chunk"], segments=c["segments"])


def test_split_sequence_carry_over(R):
    """Two calls over halves, the second fed the last W - 1 raw rows of the
    first as its history and the first's final state, equal one call."""
    W, T1, T2 = 4, 160, 141
    f = D.make_fused("layer130m", conv_width=W, B=2, T=T1 + T2, H=3)
    t = {n: f.torch(n, dev()) for n in ("q", "k", "v", "g", "tau", "u", "w", "d",
                                         "conv_q", "conv_k", "conv_v")}
    conv = (t["conv_q"], t["conv_k"], t["conv_v"])
    kw = dict(u=None, w=t["w"], d=t["d"], conv=conv)
    o, sf = R.chunk_fwd_fused(t["q"], t["k"], t["v"], t["g"], t["tau"], u=t["u"], w=t["w"],
                              d=t["d"], conv=conv, output_final_state=True)
    cut = lambda x, a, b: x[:, a:b].contiguous()
    o1, s1 = R.chunk_fwd_fused(cut(t["q"], 0, W - 1 + T1), cut(t["k"], 0, W - 1 + T1),
                               cut(t["v"], 0, W - 1 + T1), cut(t["g"], 0, T1), cut(t["tau"], 0, T1),
                               u=cut(t["u"], 0, T1), w=t["w"], d=t["d"], conv=conv,
                               output_final_state=True)
    o2, s2 = R.chunk_fwd_fused(cut(t["q"], T1, W - 1 + T1 + T2), cut(t["k"], T1, W - 1 + T1 + T2),
                               cut(t["v"], T1, W - 1 + T1 + T2), cut(t["g"], T1, T1 + T2),
                               cut(t["tau"], T1, T1 + T2), u=cut(t["u"], T1, T1 + T2), w=t["w"],
                               d=t["d"], conv=conv, initial_state=s1, output_final_state=True)
    torch.cuda.synchronize()
    whole = o.cpu().numpy()
    parts = np.concatenate([o1.cpu().numpy(), o2.cpu().numpy()], axis=1)
    e = oracle.rel_to_rms_error(parts, whole)
    es = oracle.rel_to_rms_error(s2.cpu().numpy(), sf.cpu().numpy())
    print(f"[split carry] out {e:.2e} state {es:.2e}", flush=True)
    assert e <= 1e-3 and es <= 1e-3


# ---------------------------------------------------------------- decode


def test_decode_fused_steps(R):
    """Decode steps with rolling convolution windows, low-rank beta_hat and
    the feedthrough, from a prefill's carried state, against the oracle's
    fused forward over the whole sequence."""
    W, Tp, Td = 4, 96, 12
    f = D.make_fused("decode_batch", conv_width=W, B=8, T=Tp + Td, H=4)
    t = {n: f.torch(n, dev()) for n in ("q", "k", "v", "g", "tau", "u", "w", "d",
                                         "conv_q", "conv_k", "conv_v")}
    conv = (t["conv_q"], t["conv_k"], t["conv_v"])
    s0 = torch.from_numpy(f.base.initial_state).to(dev())
    cut = lambda x, a, b: x[:, a:b].contiguous()
    o_pre, S = R.chunk_fwd_fused(cut(t["q"], 0, W - 1 + Tp), cut(t["k"], 0, W - 1 + Tp),
                                 cut(t["v"], 0, W - 1 + Tp), cut(t["g"], 0, Tp), cut(t["tau"], 0, Tp),
                                 u=cut(t["u"], 0, Tp), w=t["w"], d=t["d"], conv=conv,
                                 initial_state=s0, output_final_state=True)
    outs = [o_pre.cpu().numpy()]
    for s in range(Td):
        tok = Tp + s
        win = [cut(t[n], tok, tok + W) for n in ("q", "k", "v")]
        o = R.decode_step_fused(*win, t["g"][:, tok].contiguous(), t["tau"][:, tok].contiguous(), S,
                                u=t["u"][:, tok].contiguous(), w=t["w"], d=t["d"], conv=conv)
        outs.append(o.cpu().numpy()[:, None])
    torch.cuda.synchronize()
    got = np.concatenate(outs, axis=1)
    ro, rs = oracle.fwd_fused(f.f32("q"), f.f32("k"), f.f32("v"), f.f32("g"), f.f32("tau"),
                              u=f.f32("u"), w=f.f32("w"), d=f.d,
                              conv=(f.conv_q, f.conv_k, f.conv_v), initial_state=f.base.initial_state)
    eo = oracle.rel_to_rms_error(got, ro)
    ed = oracle.rel_to_rms_error(got[:, Tp:], ro[:, Tp:])
    es = oracle.rel_to_rms_error(S.cpu().numpy(), rs)
    print(f"[prefill+decode fused] out {eo:.2e} decode part {ed:.2e} state {es:.2e}", flush=True)
    assert eo <= 1e-2 and ed <= 1e-2 and es <= 1e-2


@pytest.mark.parametrize("use_conv,use_u,use_d", [(False, True, False), (True, False, True),
                                                  (False, False, True)])
def test_decode_fused_one_step(R, use_conv, use_u, use_d):
    W = 3
    f = D.make_fused("decode_batch", conv_width=W, B=16, T=1, H=8)
    st = f.base.initial_state
    t = {n: f.torch(n, dev()) for n in ("q", "k", "v", "g", "tau", "beta_hat", "u", "w", "d",
                                         "conv_q", "conv_k", "conv_v")}
    if use_conv:
        q, k, v = t["q"], t["k"], t["v"]                       # [N, W, H, D] windows
        rq, rk, rv = f.f32("q"), f.f32("k"), f.f32("v")
        conv = (t["conv_q"], t["conv_k"], t["conv_v"])
        rconv = (f.conv_q, f.conv_k, f.conv_v)
    else:
        q, k, v = (t[n][:, W - 1].contiguous() for n in ("q", "k", "v"))
        rq, rk, rv = (f.f32(n)[:, W - 1] for n in ("q", "k", "v"))
        conv = rconv = None
    S = torch.from_numpy(st).to(dev())
    o = R.decode_step_fused(q, k, v, t["g"][:, 0].contiguous(), t["tau"][:, 0].contiguous(), S,
                            beta_hat=None if use_u else t["beta_hat"][:, 0].contiguous(),
                            u=t["u"][:, 0].contiguous() if use_u else None,
                            w=t["w"] if use_u else None, d=t["d"] if use_d else None, conv=conv)
    torch.cuda.synchronize()
    ro, rs = oracle.decode_fused(rq, rk, rv, f.f32("g")[:, 0], f.f32("tau")[:, 0], st,
                                 beta_hat=None if use_u else f.f32("beta_hat")[:, 0],
                                 u=f.f32("u")[:, 0] if use_u else None,
                                 w=f.f32("w") if use_u else None, d=f.d if use_d else None,
                                 conv=rconv)
    eo = oracle.rel_to_rms_error(o.cpu().numpy(), ro)
    es = oracle.rel_to_rms_error(S.cpu().numpy(), rs)
    print(f"[decode fused conv={use_conv} u={use_u} d={use_d}] out {eo:.2e} state {es:.2e}", flush=True)
    assert eo <= 1e-2 and es <= 1e-2


@pytest.mark.parametrize("dk,dv,dtype,rank,W", [(16, 16, "bf16", 16, 4), (32, 64, "bf16", 32, 2),
                                                (128, 128, "bf16", 16, 4), (64, 32, "f32", 32, 3),
                                                (128, 16, "f32", 16, 4)])
def test_decode_fused_widths(R, dk, dv, dtype, rank, W):
    """One decode step with every fused step on, over widths, dtypes, ranks and
    window lengths."""
    f = D.make_fused("decode_batch", conv_width=W, rank=rank, B=12, T=1, H=3, dk=dk, dv=dv,
                     dtype=dtype)
    st = f.base.initial_state
    t = {n: f.torch(n, dev()) for n in ("q", "k", "v", "g", "tau", "u", "w", "d",
                                         "conv_q", "conv_k", "conv_v")}
    S = torch.from_numpy(st).to(dev())
    o = R.decode_step_fused(t["q"], t["k"], t["v"], t["g"][:, 0].contiguous(),
                            t["tau"][:, 0].contiguous(), S, u=t["u"][:, 0].contiguous(), w=t["w"],
                            d=t["d"], conv=(t["conv_q"], t["conv_k"], t["conv_v"]))
    torch.cuda.synchronize()
    ro, rs = oracle.decode_fused(f.f32("q"), f.f32("k"), f.f32("v"), f.f32("g")[:, 0],
                                 f.f32("tau")[:, 0], st, u=f.f32("u")[:, 0], w=f.f32("w"), d=f.d,
                                 conv=(f.conv_q, f.conv_k, f.conv_v))
    eo = oracle.rel_to_rms_error(o.cpu().numpy(), ro)
    es = oracle.rel_to_rms_error(S.cpu().numpy(), rs)
    bar = BAR[dtype]
    print(f"[decode fused dk{dk} dv{dv} {dtype} rank{rank} W{W}] out {eo:.2e} state {es:.2e}", flush=True)
    assert eo <= bar and es <= bar


def test_random_shape_sweep(R):
    """A wider sweep from a second seed: 80 more shapes, dtypes, plans and step
    mixes of the fused forward against the oracle; reports the worst error as a
    fraction of the bar."""
    worst, bad = {}, []
    for c in draw_fused_cases(80, 99):
        f = D.make_fused("layer130m", conv_width=c["W"], rank=c["rank"], B=c["B"], T=c["T"], H=c["H"],
                         dk=c["dk"], dv=c["dv"], dtype=c["dtype"], g_mean=c["g_mean"], sub=500 + c["i"])
        s0 = None
        if c["s0"]:
            rng = np.random.default_rng(2000 + c["i"])
            s0 = (0.1 * rng.standard_normal((c["B"], c["H"], c["dk"], c["dv"]))).astype(np.float32)
        kw = dict(use_u=c["use_u"], use_d=c["use_d"], use_conv=c["W"] > 1)
        o, sf = run(R, f, s0=s0, chunk=c["chunk"], segments=c["segments"], **kw)
        ro, rs = ref(f, s0=s0, **kw)
        bar = BAR[f.base.wl.dtype]
        for n, e in (("out", oracle.rel_to_rms_error(o, ro)), ("state", oracle.rel_to_rms_error(sf, rs))):
            worst[c["dtype"]] = max(worst.get(c["dtype"], 0.0), e / bar)
            if not e <= bar:
                bad.append((fused_case_id(c), n, e))
    print(f"[fused sweep] worst error as a fraction of the bar: {worst}", flush=True)
    assert not bad, bad
