"""The allocation-free step (mk_decode_step_noalloc) against mk_decode_step, through the C
ABI: two calls in a row on the device's static scratch, the second with a smaller input
(a smaller model and a shorter context); each result must equal the allocating entry
point's bit for bit (same kernel, scratch elsewhere) and the oracle's within the parity
bar (identical token; logits within 5e-2 max-abs and 1e-2 relative L2)."""
import numpy as np
import pytest
import torch

import oracle
from transformer_megakernel_amd import mk, synth
from transformer_megakernel_amd.synth import ModelShape

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

SMALL = ModelShape(n_layers=2, hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=64, ffn=2048, vocab=4096,
                   rms_eps=1e-5, rope_theta=500000.0)


def _kv_bits(kv):
    return kv.detach().cpu().view(torch.int16).numpy().view(np.uint16).copy()


def _one(shape, max_ctx, ctx, tok, repeats=2):
    print(f"[noalloc] hidden {shape.hidden} ctx {ctx}", flush=True)
    W = synth.make_weights(shape, seed=0, device=DEV)
    kv_a = synth.make_kv_cache(shape, max_ctx, ctx, seed=1, device=DEV)
    kv_b = kv_a.clone()
    kv_o = _kv_bits(kv_a)
    m = mk.Megakernel(shape, max_ctx, 0)
    m.load_weights(W)
    la = torch.empty(shape.vocab, dtype=torch.float32, device=DEV)
    lb = torch.full((shape.vocab,), float("nan"), dtype=torch.float32, device=DEV)
    na = torch.zeros(1, dtype=torch.int32, device=DEV)
    nb = torch.full((1,), -1, dtype=torch.int32, device=DEV)
    m.decode_step(tok, ctx, kv_a, la, na)
    m.sync()
    for _ in range(repeats):   # the second call finds the scratch as the first left it
        lb.fill_(float("nan"))
        m.decode_step_noalloc(tok, ctx, kv_b, lb, nb)
        m.sync()
        assert torch.equal(la.view(torch.int32), lb.view(torch.int32))
        assert int(na.item()) == int(nb.item())
        assert torch.equal(kv_a.view(torch.int16), kv_b.view(torch.int16))
    ref, t = oracle.decode_step(shape, W.as_numpy_bits(), kv_o, tok, ctx, return_next=True)
    got = lb.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(got - ref)) < 5e-2 and np.linalg.norm(got - ref) / np.linalg.norm(ref) < 1e-2
    assert int(nb.item()) == t
    m.close()


def test_noalloc_step_matches_the_allocating_step_on_two_calls_the_second_smaller():
    _one(SMALL, 512, 300, 77)                                 # two key splits, merged across CUs
    _one(ModelShape.named("tiny"), 64, 16, 9)                 # smaller model, shorter context


def test_noalloc_rejects_a_shape_whose_scratch_does_not_fit():
    """26 layers at the Llama-3.2-1B widths need ~16.9 MiB of scratch (the split-attention
    partials dominate); the call must be refused before anything is launched (the weights
    are real, so even a wrong launch would compute a valid step)."""
    s = ModelShape.named("llama1b")
    s.n_layers = 26
    L, D, hq, hkv, hd, F = s.n_layers, s.hidden, s.n_q_heads, s.n_kv_heads, s.head_dim, s.ffn
    words = (2 * L + 1) * D + L * (hq + 2 * hkv) * hd + L * hkv * (hq // hkv) * 32 * (hd + 2) + L * hq * hd + L * F
    assert words * 8 > 16 << 20
    W = synth.make_weights(s, seed=0, device=DEV)
    m = mk.Megakernel(s, 64, 0)
    m.load_weights(W)
    kv = synth.make_kv_cache(s, 64, 16, seed=1, device=DEV)
    logits = torch.full((s.vocab,), -3.0, dtype=torch.float32, device=DEV)
    with pytest.raises(mk.MkError, match="static scratch") as e:
        m.decode_step_noalloc(3, 16, kv, logits)
    assert e.value.code == mk.MK_EINVAL
    m.sync()
    assert bool((logits == -3.0).all())
    m.close()
