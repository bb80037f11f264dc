"""The per-instruction trace (the time breakdown's source) on the GPU: tracing changes no
result, and the marks of every instruction are ordered as the kernel sets them."""
import numpy as np
import pytest
import torch

from transformer_megakernel_amd import mk, synth
from transformer_megakernel_amd import trace_breakdown as tb
from transformer_megakernel_amd.synth import ModelShape

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("name,ctx", [("tiny", 16), ("llama1b", 128)])
def test_traced_step_is_bit_identical_and_marks_are_ordered(name, ctx):
    shape = ModelShape.named(name)
    print(f"[trace] {name} ctx {ctx}", flush=True)
    W = synth.make_weights(shape, seed=0, device=DEV)
    kv = synth.make_kv_cache(shape, ctx + 8, ctx, seed=1, device=DEV)
    m = mk.Megakernel(shape, ctx + 8, 0)
    m.load_weights(W)
    logits = torch.empty(shape.vocab, dtype=torch.float32, device=DEV)
    nxt = torch.zeros(1, dtype=torch.int32, device=DEV)
    m.decode_step(3, ctx, kv, logits, nxt)
    m.sync()
    plain = logits.clone()
    buf = m.enable_trace()
    buf.zero_()
    m.decode_step(3, ctx, kv, logits, nxt)
    m.sync()
    assert torch.equal(logits.view(torch.int32), plain.view(torch.int32))
    P = m.plan()
    tr = tb.reshape(buf.cpu().numpy(), P["n_cus"])
    m.disable_trace()
    off = P["offsets"]
    for cu in range(P["n_cus"]):
        t = tr[cu, :int(off[cu + 1] - off[cu])]
        assert np.all(t[:, 0] > 0) and np.all(t[:, 7] > 0) and np.all(t[:, 5] > 0)
        for i in range(len(t)):
            lead = [v for v in t[i, [0, 1, 2, 3, 4, 7]] if v > 0]
            assert lead == sorted(lead), (cu, i, t[i])
            assert t[i, 5] <= t[i, 6], (cu, i, t[i])
            if i + 1 < len(t):
                assert t[i + 1, 0] >= t[i, 7] and t[i + 1, 5] >= t[i, 5], (cu, i)
        # the compute waves' page waits (a sum over waves) fit between the leader freeing the
        # instruction's activation slot (no wave starts before it) and the last wave's end
        lo = np.where(t[:, 3] > 0, t[:, 3], t[:, 5])
        assert np.all(t[:, 9] <= tb.N_COMPUTE_WAVES * (t[:, 6] - lo + 1))
        # an instruction's first ring page is issued before its last page is consumed, and
        # the loaders' full-ring waits (a sum over the two loaders) fit in the step
        issued = t[:, 10] > 0
        assert np.all(t[issued, 10] <= t[issued, 6]), cu
        assert np.all(t[:, 11] >= 0) and t[:, 11].sum() <= tb.N_LOADERS * (t[:, 7].max() - t[0, 0] + 1)
    nch = max(int(r[7]) for r in P["records"] if r[0] == tb.DOWN)
    rep = tb.report([tr], P, shape.n_layers, nch, name)
    print(rep, flush=True)
    span = tb.step_span(tr)
    assert 0 < span < 100_000
