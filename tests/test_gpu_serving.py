"""GPU: prefill then batched decode from the carried state (the pages' use:
training/prefill chunkwise, inference sequentially over the cached fixed-size
state; Rodimus* rebuttal page, answer on sequential processing bottlenecks).

A prefill of T0 tokens (rodimus_ddts_chunk_fwd with a final state) followed by
K decode steps (rodimus_ddts_decode_step on that state, in place) must equal
the oracle run over all T0 + K tokens: outputs of the prefill, of every decode
step and the final state, each within the bf16 bar.
"""
import numpy as np
import pytest

import ddts_inputs as D
import oracle

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

NAMES = ("q", "k", "v", "g", "tau", "beta_hat")


@pytest.mark.parametrize("T0,K", [(2048, 32), (24576, 8)])
def test_prefill_then_decode(T0, K):
    import gated_linear_attention_rodimus_amd as R
    dev = torch.device("cuda:0")
    x = D.make("decode_batch", B=4, T=T0 + K, H=4)         # the decode workload's distributions
    t = [x.torch(n, dev) for n in NAMES]
    s0 = torch.from_numpy(x.initial_state).to(dev)
    o_pre, S = R.chunk_fwd(*(a[:, :T0].contiguous() for a in t), initial_state=s0,
                           output_final_state=True)
    outs = []
    for s in range(K):
        outs.append(R.decode_step(*(a[:, T0 + s].contiguous() for a in t), S))
    torch.cuda.synchronize()
    ro, rs = oracle.fwd(*(x.f32(n) for n in NAMES), x.initial_state)
    err = oracle.rel_to_rms_error
    assert err(o_pre.cpu().numpy(), ro[:, :T0]) < 1e-2
    dec = np.stack([o.cpu().numpy() for o in outs], axis=1)
    assert err(dec, ro[:, T0:]) < 1e-2
    assert err(S.cpu().numpy(), rs) < 1e-2
