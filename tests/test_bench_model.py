"""CPU tests of the byte and flop model behind the bench line's roofline.

The figures are written out by hand from the operation's definition:
per token-head the forward reads q, k, g, tau (dk each) and v, beta_hat (dv
each) once in their storage dtype and writes o (dv, fp32); a state read or
written moves dk * dv fp32 values; the intra-chunk products count the causal
triangle once, (C + 1) / 2 tokens on average, over a multiply and an add.
"""
import bench


def test_chunk_bytes_130m_layer():
    # B=8 T=2048 H=12, dk 64, dv 128, bf16 inputs: (4*64 + 2*128) * 2 + 128 * 4 = 1536 B
    by, fl = bench.chunk_algorithmic(8, 2048, 12, 64, 128, 64)
    assert by == 8 * 2048 * 12 * 1536 == 301_989_888
    # flops per token-head: scores and A V' over the causal half, (C + 1) * (dk + dv),
    # plus Qt S' and the state update, 2 * dk * dv each
    assert fl == 8 * 2048 * 12 * (65 * (64 + 128) + 4 * 64 * 128) == 8_896_118_784


def test_chunk_bytes_with_states():
    # the 1.6B layer returns S_T; the long prefill reads S_0: one state each
    st = 64 * 128 * 4
    by, _ = bench.chunk_algorithmic(4, 4096, 16, 64, 128, 64, state_out=True)
    assert by == 4 * 4096 * 16 * 1536 + 4 * 16 * st
    by, _ = bench.chunk_algorithmic(1, 65536, 16, 64, 128, 64, state_in=True)
    assert by == 65536 * 16 * 1536 + 16 * st
    # fp32 inputs double the input bytes only
    by32, _ = bench.chunk_algorithmic(1, 10, 1, 16, 16, 16, in_bytes=4)
    assert by32 == 10 * ((4 * 16 + 2 * 16) * 4 + 16 * 4)


def test_decode_bytes():
    # 256 sequences x 16 heads: the fp32 state read and written (2 x 32 KiB per
    # head), the inputs once (bf16) and the output (fp32): ~274.7 MB per step
    by, fl = bench.decode_algorithmic(256, 16, 64, 128)
    n = 256 * 16
    assert by == n * (2 * 64 * 128 * 4 + (4 * 64 + 2 * 128) * 2 + 128 * 4) == 274_726_912
    assert fl == 5 * n * 64 * 128


def test_pass_traffic_record_is_consistent():
    """The committed counter summary of the long prefill: per-pass HBM bytes
    are FETCH_SIZE x the copy scale + WRITE_SIZE, their sum is the call's,
    and the bench reads the output pass's figure only while the kernel
    source is the one the counters were taken on."""
    import hashlib
    import json
    rec = json.load(open(bench.TRAFFIC_FILE))
    total = 0
    for name, p in rec["passes"].items():
        hbm = p["fetch_size_kib_per_dispatch"] * 1024 * rec["fetch_scale"] + \
            p["write_size_kib_per_dispatch"] * 1024 * rec["write_scale"]
        assert abs(hbm - p["hbm_bytes_per_launch"]) / hbm < 1e-4, name
        total += p["hbm_bytes_per_launch"]
    assert total == rec["call_hbm_bytes"]
    # the output pass's own bytes: the call's, with the incoming state of each
    # of the 16 segments read in place of the one initial state
    state = 64 * 128 * 4
    assert rec["passes"]["output"]["algorithmic_bytes_per_launch"] == \
        bench.chunk_algorithmic(1, 65536, 16, 64, 128, 64, state_in=True)[0] - 16 * state + 16 * 16 * state
    assert rec["call_algorithmic_bytes"] == bench.chunk_algorithmic(1, 65536, 16, 64, 128, 64, state_in=True)[0]
    sha = hashlib.sha256(open(bench.KERNEL_SRC, "rb").read()).hexdigest()
    got = bench.kernel_traffic("output")
    assert got == (rec["passes"]["output"]["hbm_bytes_per_launch"]
                   if sha == rec["kernel_source_sha256"] else None)


def test_swska_work_model():
    # T = 3, window 2: keys per token 1, 2, 2 -> 5 (b, h) key visits
    by, fl = bench.swska_algorithmic(1, 3, 2, 4, 8, 2)
    assert fl == 2 * 2 * 5 * (4 + 8)
    assert by == 3 * (2 * (4 + 8) * 2 + 4 * 2 + 2 * 8 * 4)
