"""Parity of the HIP megakernel against the CPU oracle, through the C ABI (needs a GPU).

Bar (from the workload definition): identical greedy tokens, and logits within 5e-2
max-abs and 1e-2 relative L2 (||gpu - oracle|| / ||oracle|| over all vocab logits).
KV slots the step must not touch are compared bit for bit.  The appended K/V are the
bf16 rounding of fp32 values that the GPU sums in a different order than the oracle, so
the two roundings can differ only where the unrounded value lies next to a rounding
boundary: every appended element must be the bf16 rounding of some value within
2^-12 (relative) + 1e-4 (absolute) of the oracle's unrounded fp32 value (the fp32
difference of the two sides is ~1e-6 of the unit-scale values; the absolute term covers
elements that are small results of cancellation after RoPE).
"""
import numpy as np
import pytest
import torch

import oracle
from transformer_megakernel_amd import mk, synth
from transformer_megakernel_amd.synth import ModelShape

pytestmark = pytest.mark.gpu

MAX_ABS, REL_L2 = 5e-2, 1e-2
DEV = "cuda:0"


def close(got: np.ndarray, ref: np.ndarray, what=""):
    got = got.astype(np.float64)
    ref = ref.astype(np.float64)
    err = float(np.max(np.abs(got - ref)))
    rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    assert err < MAX_ABS and rel < REL_L2, f"{what}: max|d|={err:.3e} relL2={rel:.3e}"
    return err, rel


def kv_bits(kv: torch.Tensor) -> np.ndarray:
    return kv.detach().cpu().view(torch.int16).numpy().view(np.uint16).copy()


def unrounded_kv(shape, trace: dict, pos: int) -> np.ndarray:
    """The oracle's fp32 K (after RoPE) and V of one step, [layer][k|v][kv head][hd]."""
    cos, sin = oracle.rope_cos_sin(pos, shape.head_dim, shape.rope_theta)
    k = np.stack([oracle.apply_rope(t, cos, sin) for t in trace["k"]])
    v = np.stack(trace["v"])
    return np.stack([k, v], axis=1)


def check_kv(gpu_kv: np.ndarray, ora_kv: np.ndarray, new_slots, unrounded: np.ndarray):
    """``unrounded``: [layer][k|v][kv head][slot of new_slots][hd], the oracle's fp32 values."""
    slots = list(new_slots)
    mask = np.ones(gpu_kv.shape[3], bool)
    mask[slots] = False
    assert np.array_equal(gpu_kv[:, :, :, mask, :], ora_kv[:, :, :, mask, :]), "untouched KV slots changed"
    a = oracle.bf16_to_float(gpu_kv[:, :, :, slots, :]).astype(np.float64)
    b = oracle.bf16_to_float(ora_kv[:, :, :, slots, :]).astype(np.float64)
    u = unrounded.astype(np.float64)
    # The GPU rounds its own fp32 value g, |g - u| <= tol; rounding is monotone, so its
    # bf16 value lies between the roundings of u - tol and u + tol.
    tol = np.abs(u) * 2.0 ** -12 + 1e-4
    lo = oracle.bf16_to_float(oracle.float_to_bf16(u - tol)).astype(np.float64)
    hi = oracle.bf16_to_float(oracle.float_to_bf16(u + tol)).astype(np.float64)
    bad = (a < lo) | (a > hi)
    assert not bad.any(), (f"{int(bad.sum())} appended K/V elements are not a rounding of a value near the "
                           f"oracle's (max |gpu - oracle| {np.max(np.abs(a - b)):.3e}, "
                           f"{np.mean(a != b):.3%} differ in all)")


class Model:
    def __init__(self, name, max_ctx, ctx, wseed=0, kvseed=1):
        print(f"[setup] {name} max_ctx={max_ctx} ctx={ctx}", flush=True)
        self.shape = ModelShape.named(name)
        self.W = synth.make_weights(self.shape, seed=wseed, device=DEV)
        self.kv = synth.make_kv_cache(self.shape, max_ctx, ctx, seed=kvseed, device=DEV)
        self.Wn = self.W.as_numpy_bits()
        self.m = mk.Megakernel(self.shape, max_ctx, 0)
        self.m.load_weights(self.W)
        self.logits = torch.empty(self.shape.vocab, dtype=torch.float32, device=DEV)
        self.next = torch.zeros(1, dtype=torch.int32, device=DEV)


def greedy_compare(M: Model, tok0: int, pos0: int, n: int, dev_chain=False):
    kv_o = kv_bits(M.kv)
    tok_g, tok_o = tok0, tok0
    tokbuf = torch.tensor([tok0], dtype=torch.int32, device=DEV)
    worst = (0.0, 0.0)
    unr = []
    for i in range(n):
        if dev_chain:
            M.m.decode_step_dev(tokbuf, pos0 + i, M.kv, M.logits, tokbuf)
        else:
            M.m.decode_step(tok_g, pos0 + i, M.kv, M.logits, M.next)
        M.m.sync()
        tr = {}
        ref, tok_o = oracle.decode_step(M.shape, M.Wn, kv_o, tok_o, pos0 + i, return_next=True, trace=tr)
        unr.append(unrounded_kv(M.shape, tr, pos0 + i))
        err = close(M.logits.cpu().numpy(), ref, f"step {i} pos {pos0 + i}")
        worst = max(worst, err)
        tok_g = int((tokbuf if dev_chain else M.next).item())
        assert tok_g == tok_o, f"step {i}: gpu token {tok_g} != oracle {tok_o}"
    check_kv(kv_bits(M.kv), kv_o, range(pos0, pos0 + n), np.stack(unr, axis=3))
    return worst


def test_tiny_greedy_8_tokens_from_context_16():
    M = Model("tiny", 64, 16)
    print("worst", greedy_compare(M, synth.make_token(M.shape, 2), 16, 8))


def test_tiny_from_empty_cache_single_key_first():
    M = Model("tiny", 16, 0)
    greedy_compare(M, synth.make_token(M.shape, 3), 0, 8)


def test_tiny_device_token_chain():
    M = Model("tiny", 64, 16)
    greedy_compare(M, synth.make_token(M.shape, 2), 16, 8, dev_chain=True)


def test_tiny_two_splits_merge_path():
    """pos 300: keys split in two, merged across CUs."""
    M = Model("tiny", 512, 300)
    greedy_compare(M, 77, 300, 3)


def test_tiny_many_splits_long_context():
    M = Model("tiny", 4096, 4000)
    greedy_compare(M, 5, 4000, 2)


def test_bitwise_determinism_and_idempotent_repeat():
    M = Model("tiny", 64, 16)
    outs = []
    for _ in range(3):
        M.m.decode_step(9, 16, M.kv, M.logits, M.next)
        M.m.sync()
        outs.append(M.logits.cpu().numpy().copy())
    assert all(np.array_equal(outs[0], o) for o in outs[1:])


def test_watchdog_expiry_is_reported_and_recovered():
    M = Model("tiny", 64, 16)
    M.m.set_watchdog_us(0)
    M.m.decode_step(9, 16, M.kv, M.logits, M.next)
    code = M.m.sync_code()
    assert code in (mk.MK_ETIMEOUT, mk.MK_OK)   # an instant pass is allowed, never a hang
    M.m.set_watchdog_us(2_000_000)
    greedy_compare(M, 9, 16, 2)


def test_bad_device_token_is_flagged():
    M = Model("tiny", 64, 16)
    bad = torch.tensor([-5], dtype=torch.int32, device=DEV)
    M.m.decode_step_dev(bad, 16, M.kv, M.logits, M.next)
    assert M.m.sync_code() == mk.MK_ERANGE
    M.m.decode_step(3, 16, M.kv, M.logits, M.next)
    M.m.sync()


def test_host_side_range_errors():
    M = Model("tiny", 64, 16)
    with pytest.raises(mk.MkError):
        M.m.decode_step(0, 64, M.kv, M.logits, M.next)
    with pytest.raises(mk.MkError):
        M.m.decode_step(4096, 1, M.kv, M.logits, M.next)


@pytest.fixture(scope="module")
def llama1b():
    return Model("llama1b", 8200, 128)


def test_llama1b_context_128_one_step(llama1b):
    M = llama1b
    tok = synth.make_token(M.shape, 2)
    greedy_compare(M, tok, 128, 1)


def test_llama1b_context_1024_greedy(llama1b):
    M = llama1b
    # extend the pre-filled prefix to 1024 positions (same recipe, different seed)
    extra = synth.make_kv_cache(M.shape, 1024, 1024, seed=11, device=DEV)
    M.kv[:, :, :, 129:1024, :] = extra[:, :, :, 129:1024, :]
    greedy_compare(M, 1234, 1024, 4)


def test_llama1b_context_700_three_splits(llama1b):
    """701 keys: three splits of 256 keys per KV head, merged across CUs."""
    greedy_compare(llama1b, 4321, 700, 2)


def test_llama1b_context_8192_split_kv_repeatable(llama1b):
    M = llama1b
    extra = synth.make_kv_cache(M.shape, 8192, 8192, seed=12, device=DEV)
    M.kv[:, :, :, 1028:8192, :] = extra[:, :, :, 1028:8192, :]
    del extra
    outs = []
    for _ in range(3):
        M.m.decode_step(4321, 8192, M.kv, M.logits, M.next)
        M.m.sync()
        outs.append(M.logits.cpu().numpy().copy())
    assert all(np.array_equal(outs[0], o) for o in outs[1:])
    kv_o = kv_bits(M.kv)
    ref, t = oracle.decode_step(M.shape, M.Wn, kv_o, 4321, 8192, return_next=True)
    close(outs[0], ref, "ctx 8192")
    assert int(M.next.item()) == t


@pytest.mark.timeout(600)
def test_llama8b_context_2048_one_step():
    """Llama-3.1-8B shape: untied LM head, head_dim 128 with the keys split over CUs,
    4096-wide activations staged in two batches, 28 KiB down rows consumed in four
    7 KiB chunks.  One step at context 2048 against the full oracle step."""
    M = Model("llama8b", 2056, 2048)
    tok = synth.make_token(M.shape, 3)
    greedy_compare(M, tok, 2048, 1)
