"""Per-instruction parity: every intermediate the step exchanges between CUs (raw q/k/v,
attention output, SiLU(gate)*up, x after each residual) against the oracle's trace.

This localises a mismatch to the first instruction family that produces it."""
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
SMALL128 = ModelShape(n_layers=2, hidden=1024, n_q_heads=8, n_kv_heads=2, head_dim=128, ffn=3584, vocab=2048,
                      rms_eps=1e-5, rope_theta=500000.0, tied=False)


def stage_report(shape, dump, trace, epoch_ok=True):
    hd, hq, hkv = shape.head_dim, shape.n_q_heads, shape.n_kv_heads
    hpg = hq // hkv
    L, d, F = shape.n_layers, shape.hidden, shape.ffn
    xv, xe = dump["x"]
    qv, qe = dump["qkv"]
    ov, oe = dump["o"]
    av, ae = dump["a"]
    grp = (hpg + 2) * hd
    rows = []
    for l in range(L):
        q = qv[l * hkv * grp:(l + 1) * hkv * grp].reshape(hkv, hpg + 2, hd)
        gq = q[:, :hpg, :].reshape(hq, hd)
        rows.append((f"L{l} q", gq, trace["q"][l]))
        rows.append((f"L{l} k", q[:, hpg, :], trace["k"][l]))
        rows.append((f"L{l} v", q[:, hpg + 1, :], trace["v"][l]))
        rows.append((f"L{l} o", ov[l * hq * hd:(l + 1) * hq * hd], trace["o"][l]))
        rows.append((f"L{l} x_attn", xv[(2 * l + 1) * d:(2 * l + 2) * d], trace["x"][2 * l]))
        rows.append((f"L{l} a", av[l * F:(l + 1) * F], trace["a"][l]))
        rows.append((f"L{l} x_mlp", xv[(2 * l + 2) * d:(2 * l + 3) * d], trace["x"][2 * l + 1]))
    out = []
    for name, g, r in rows:
        g = np.asarray(g, np.float64).ravel()
        r = np.asarray(r, np.float64).ravel()
        err = float(np.max(np.abs(g - r))) if np.all(np.isfinite(g)) else float("nan")
        scale = float(np.max(np.abs(r))) + 1e-30
        out.append((name, err / scale, int(np.sum(~np.isfinite(g)))))
    return out


def run_stage_check(shape, max_ctx, ctx, pos, tok):
    W = synth.make_weights(shape, seed=0, device=DEV)
    kv = synth.make_kv_cache(shape, max_ctx, ctx, seed=1, device=DEV)
    Wn = W.as_numpy_bits()
    kvn = kv.cpu().view(torch.int16).numpy().view(np.uint16).copy()
    m = mk.Megakernel(shape, max_ctx, 0)
    m.load_weights(W)
    logits = torch.empty(shape.vocab, dtype=torch.float32, device=DEV)
    m.decode_step(tok, pos, kv, logits)
    code = m.sync_code()
    dump = m.debug_dump()
    trace = {}
    ref = oracle.decode_step(shape, Wn, kvn, tok, pos, trace=trace)
    rep = stage_report(shape, dump, trace)
    for name, rel, nonfinite in rep:
        print(f"{name:12s} rel_err={rel:.3e} nonfinite={nonfinite}", flush=True)
    got = logits.cpu().numpy()
    print("logits max|d|", float(np.max(np.abs(got - ref))), "sync", code, flush=True)
    assert code == 0
    bad = [r for r in rep if not (r[1] < 1e-3)]
    assert not bad, f"first mismatching stage: {bad[0]}"


def test_stages_small_shape_wide_rows():
    """hidden 512 (1 KiB rows), 4 query heads per KV head."""
    run_stage_check(SMALL, 64, 16, 16, 7)


def test_stages_small_shape_head_dim_128():
    """head_dim 128, 3584-wide down chunks (7 KiB rows), untied LM head."""
    run_stage_check(SMALL128, 64, 16, 16, 11)


def test_stages_llama1b():
    run_stage_check(ModelShape.named("llama1b"), 256, 128, 128, 1234)


def test_stages_small_shape_head_dim_128_split_kv():
    """head_dim 128 with the cached keys split over four CUs per KV head (256 keys each),
    the current position joining the last split, and the splits merged."""
    run_stage_check(SMALL128, 1100, 1024, 1024, 5)


@pytest.mark.parametrize("shape,pos", [(SMALL128, 1024 + 20), (SMALL128, 1024 + 70), (SMALL, 512 + 20),
                                       (SMALL, 512 + 100)])
def test_stages_split_kv_partial_last_split(shape, pos):
    """The last split with a partial page: head_dim 128 (256-key splits of 32-key pages,
    two waves a page) with one page of 20 keys (the pages' second pair of waves has none)
    or three pages (an odd count, the last of 6 keys); head_dim 64 (128-key splits of
    64-key pages, a wave per 16 keys) with 20 keys (three of the four waves see only keys
    past the end) or 100 (two pages, the second of 36 keys)."""
    run_stage_check(shape, pos + 8, pos, pos, 9)
