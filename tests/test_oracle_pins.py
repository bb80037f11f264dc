"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test pins one part of the decode step (Megakernel article, section "Megakernel:
a fusion design from scratch", instruction list) to a closed form, an invariant, a
library routine that computes the same special case, or a brute-force recomputation.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import decode as od
from tests.bruteforce import full_forward
from transformer_megakernel_amd.synth import ModelShape, make_kv_cache, make_token, make_weights

RNG = np.random.default_rng(1234)


# ---------------------------------------------------------------- bf16 storage
def test_bf16_widening_is_exact_and_round_trips():
    bits = RNG.integers(0, 1 << 16, size=100_000, dtype=np.uint32).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]                    # drop inf/NaN patterns
    f = od.bf16_to_float(bits)
    assert np.array_equal(f.view(np.uint32), bits.astype(np.uint32) << 16)
    assert np.array_equal(od.float_to_bf16(f), bits)


def test_bf16_rounding_matches_torch_rne_including_ties():
    x = RNG.standard_normal(200_000).astype(np.float32) * 3.0
    # exact ties: low half 0x8000, with both parities of the kept bit
    u = RNG.integers(0, 1 << 31, size=20_000, dtype=np.uint64).astype(np.uint32)
    ties = ((u & 0xFFFF0000) | 0x8000).view(np.float32)
    ties = ties[np.isfinite(ties)]
    x = np.concatenate([x, ties, np.float32([0.0, -0.0, 1e-40, -1e-40, 65504.0])])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(od.float_to_bf16(x), ref)


# ---------------------------------------------------------------- RMSNorm
def test_rmsnorm_closed_form_and_library():
    for dt in (np.float32, np.float64):
        x = RNG.standard_normal(2048).astype(dt) * 0.7
        g = (1 + 0.1 * RNG.standard_normal(2048)).astype(dt)
        n = od.rms_norm(x, g, 1e-5)
        m = np.mean(x.astype(np.float64) ** 2)
        # unit RMS before the gain, up to the eps term: rms(n/g) = sqrt(m / (m + eps))
        rms = math.sqrt(np.mean((n.astype(np.float64) / g) ** 2))
        tol = 1e-12 if dt == np.float64 else 1e-6
        assert abs(rms - math.sqrt(m / (m + 1e-5))) < tol
        ref = torch.nn.functional.rms_norm(torch.from_numpy(x.astype(np.float64))[None], (2048,),
                                           torch.from_numpy(g.astype(np.float64)), eps=1e-5)[0]
        assert np.allclose(n, ref.numpy(), rtol=10 * np.finfo(dt).eps, atol=0)
    # scale invariance (eps negligible at large scale)
    x = RNG.standard_normal(256)
    g = np.ones(256)
    assert np.allclose(od.rms_norm(1e3 * x, g, 1e-5), od.rms_norm(x, g, 0.0), rtol=1e-9)


# ---------------------------------------------------------------- RoPE
def test_rope_is_a_norm_preserving_rotation_identity_at_zero():
    hd = 64
    v = RNG.standard_normal(hd)
    c0, s0 = od.rope_cos_sin(0, hd, 500000.0, np.float64)
    assert np.array_equal(od.apply_rope(v, c0, s0), v)
    for pos in (1, 17, 1000, 8192):
        c, s = od.rope_cos_sin(pos, hd, 500000.0, np.float64)
        r = od.apply_rope(v, c, s)
        half = hd // 2
        # each (i, i+half) pair keeps its length
        assert np.allclose(r[:half] ** 2 + r[half:] ** 2, v[:half] ** 2 + v[half:] ** 2, rtol=1e-12)


def test_rope_relative_position_and_frequency_ladder():
    hd, theta = 128, 500000.0
    q, k = RNG.standard_normal(hd), RNG.standard_normal(hd)
    rot = lambda x, p: od.apply_rope(x, *od.rope_cos_sin(p, hd, theta, np.float64))
    for m, n in ((5, 3), (100, 7), (4000, 1234)):
        assert abs(rot(q, m) @ rot(k, n) - rot(q, m - n) @ k) < 1e-9
    # angles of a basis vector per pair at pos = 1: pair 0 turns by exactly 1 rad and the
    # frequencies form a geometric ladder theta^(-2/hd)
    half = hd // 2
    ang = []
    for i in range(half):
        e = np.zeros(hd)
        e[i] = 1.0
        r = rot(e, 1)
        ang.append(math.atan2(r[i + half], r[i]))
    ang = np.array(ang)
    assert abs(ang[0] - 1.0) < 1e-15
    ratios = ang[1:] / ang[:-1]
    assert np.allclose(ratios, theta ** (-2.0 / hd), rtol=1e-9)
    # it is complex multiplication of (a_i + i b_i) by exp(i * angle_i)
    p = 37
    z = (q[:half] + 1j * q[half:]) * np.exp(1j * p * ang)
    assert np.allclose(rot(q, p), np.concatenate([z.real, z.imag]), atol=1e-9)


# ---------------------------------------------------------------- attention
def test_attention_single_key_returns_its_value_exactly():
    for dt in (np.float32, np.float64):
        q = RNG.standard_normal(64).astype(dt)
        K = RNG.standard_normal((1, 64)).astype(dt)
        V = RNG.standard_normal((1, 64)).astype(dt)
        assert np.array_equal(od.attend_one_head(q, K, V), V[0])


def test_attention_equal_keys_average_values_and_matches_sdpa():
    q = RNG.standard_normal(64)
    K = np.repeat(RNG.standard_normal((1, 64)), 9, axis=0)
    V = RNG.standard_normal((9, 64))
    assert np.allclose(od.attend_one_head(q, K, V), V.mean(axis=0), rtol=1e-12)
    K = RNG.standard_normal((33, 64))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, None, None], torch.from_numpy(K)[None, None],
        torch.from_numpy(V := RNG.standard_normal((33, 64)))[None, None])[0, 0, 0]
    assert np.allclose(od.attend_one_head(q, K, V), ref.numpy(), rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- GEMV and SiLU
def test_gemv_fp32_within_higham_bound_of_fp64():
    W = od.float_to_bf16(RNG.standard_normal((64, 4096)).astype(np.float32) * 0.02)
    x = RNG.standard_normal(4096).astype(np.float32)
    y32 = od.gemv(W, x).astype(np.float64)
    y64 = od.gemv(W, x.astype(np.float64))
    absprod = np.abs(od.bf16_to_float(W, np.float64)) @ np.abs(x.astype(np.float64))
    K = 4096
    u = 2.0 ** -24
    gamma = K * u / (1 - K * u)
    assert np.all(np.abs(y32 - y64) <= gamma * absprod)


def test_silu_identities_and_library():
    z = RNG.standard_normal(10_000) * 6
    assert od.silu(np.zeros(1))[0] == 0.0
    assert np.allclose(od.silu(z) - od.silu(-z), z, rtol=1e-12, atol=1e-12)
    assert np.allclose(od.silu(z), torch.nn.functional.silu(torch.from_numpy(z)).numpy(),
                       rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------- whole step
def _tiny(seed=0):
    shape = ModelShape.named("tiny")
    W = make_weights(shape, seed=seed, device="cpu").as_numpy_bits()
    return shape, W


def _empty_cache(shape, max_ctx):
    return np.zeros((shape.n_layers, 2, shape.n_kv_heads, max_ctx, shape.head_dim), np.uint16)


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_incremental_decode_matches_bruteforce_full_forward(dtype):
    """Prefix consistency: decoding 8 tokens one by one from an empty cache equals the
    causal full-sequence forward on every prefix (pins KV-append indexing, the RoPE
    position, the inclusive mask boundary and the GQA mapping)."""
    shape, W = _tiny()
    tokens = [int(t) for t in RNG.integers(0, shape.vocab, size=8)]
    ref = full_forward(shape, W, tokens).numpy()
    kv = _empty_cache(shape, 16)
    tol = 1e-9 if dtype == np.float64 else 2e-4
    for p, t in enumerate(tokens):
        logits = od.decode_step(shape, W, kv, t, p, dtype=dtype)
        err = np.max(np.abs(logits.astype(np.float64) - ref[p]))
        assert err < tol * max(1.0, np.max(np.abs(ref[p]))), (p, err)
    assert np.all(kv[:, :, :, 8:, :] == 0)      # nothing written beyond the last position


def test_mha_special_case_and_gqa_mapping():
    """With Hkv == Hq the step is plain multi-head attention; the brute force agrees."""
    shape = ModelShape(n_layers=1, hidden=128, n_q_heads=2, n_kv_heads=2, head_dim=64,
                       ffn=256, vocab=512, rms_eps=1e-5, rope_theta=10000.0)
    W = make_weights(shape, seed=3, device="cpu").as_numpy_bits()
    tokens = [5, 77, 300, 12]
    ref = full_forward(shape, W, tokens).numpy()
    kv = _empty_cache(shape, 8)
    for p, t in enumerate(tokens):
        assert np.allclose(od.decode_step(shape, W, kv, t, p, np.float64), ref[p], rtol=1e-9, atol=1e-12)


def test_decode_writes_only_slot_pos_and_prefilled_cache_is_read():
    shape, W = _tiny()
    kv = make_kv_cache(shape, 32, 16, seed=1).view(torch.int16).numpy().view(np.uint16).copy()
    before = kv.copy()
    od.decode_step(shape, W, kv, 7, 16)
    changed = np.argwhere(np.any(kv != before, axis=-1))
    assert set(changed[:, 3].tolist()) == {16}
    # the pre-filled keys matter: a different prefix gives different logits
    kv2 = kv.copy()
    kv2[:, :, :, :16, :] = 0
    assert not np.allclose(od.decode_step(shape, W, kv, 7, 16), od.decode_step(shape, W, kv2, 7, 16))


def test_greedy_takes_first_maximum_and_chains_tokens():
    shape, W = _tiny()
    kv = _empty_cache(shape, 16)
    tok0 = make_token(shape, seed=2)
    toks, logits = od.greedy_decode(shape, W, kv, tok0, 0, 4)
    for t, lg in zip(toks, logits):
        assert t == int(np.flatnonzero(lg == lg.max())[0])
    # the chain: step i+1 consumed token i (recompute step 1 from a cache that saw step 0)
    kv_b = _empty_cache(shape, 16)
    od.decode_step(shape, W, kv_b, tok0, 0)
    assert np.array_equal(od.decode_step(shape, W, kv_b, toks[0], 1), logits[1])


def test_fp32_oracle_close_to_fp64_on_tiny_greedy():
    shape, W = _tiny()
    kv32 = make_kv_cache(shape, 32, 16, seed=1).view(torch.int16).numpy().view(np.uint16).copy()
    kv64 = kv32.copy()
    tok = make_token(shape, seed=2)
    t32, l32 = od.greedy_decode(shape, W, kv32, tok, 16, 8, np.float32)
    t64, l64 = od.greedy_decode(shape, W, kv64, tok, 16, 8, np.float64)
    assert t32 == t64
    assert max(np.max(np.abs(a - b)) for a, b in zip(l32, l64)) < 1e-4


def test_widened_weights_give_bit_identical_steps():
    """Widening the bf16 weights once up front (for long greedy runs) is exact, so the
    logits and the cache writes are bit-identical to passing the bit patterns."""
    shape, W = _tiny()
    Wf = od.widen_weights(W)
    assert Wf["lm_head"] is Wf["embed"]
    for dt in (np.float32, np.float64):
        kv_a = make_kv_cache(shape, 32, 16, seed=1).view(torch.int16).numpy().view(np.uint16).copy()
        kv_b = kv_a.copy()
        for p, t in enumerate([5, 900, 4095]):
            la = od.decode_step(shape, W, kv_a, t, 16 + p, dt)
            lb = od.decode_step(shape, Wf, kv_b, t, 16 + p, dt)
            assert np.array_equal(la, lb)
        assert np.array_equal(kv_a, kv_b)


# ---------------------------------------------------------------- the pins have teeth
_MUTATIONS = [
    ("g = (h * Hkv) // Hq", "g = h % Hkv"),                                    # GQA index
    ("kv[layer, 1, :, pos, :] = float_to_bf16(v)", "kv[layer, 1, :, pos, :] = float_to_bf16(k)"),
    ("x = x + gemv(W[\"wo\"][layer], o.reshape(-1))", "x = gemv(W[\"wo\"][layer], o.reshape(-1))"),
    ("gemv(W[\"wo\"][layer], o.reshape(-1))", "gemv(W[\"wo\"][layer], o.T.reshape(-1))"),
    ("silu(gemv(W[\"w_gate\"][layer], n2)) * gemv(W[\"w_up\"][layer], n2)",
     "silu(gemv(W[\"w_up\"][layer], n2)) * gemv(W[\"w_gate\"][layer], n2)"),
    ("np.sqrt(ms + dt.type(eps))", "(np.sqrt(ms) + dt.type(eps))"),
    ("a * cos - b * sin, b * cos + a * sin", "a * cos + b * sin, b * cos - a * sin"),
    ("cos, sin = rope_cos_sin(pos,", "cos, sin = rope_cos_sin(pos + 1,"),
    ("np.sqrt(dt.type(q.shape[0]))", "dt.type(q.shape[0])"),
    ("K = bf16_to_float(kv[layer, 0, g, : pos + 1, :], dtype)\n"
     "            V = bf16_to_float(kv[layer, 1, g, : pos + 1, :], dtype)",
     "K = bf16_to_float(kv[layer, 0, g, max(0, pos - 2) : pos + 1, :], dtype)\n"
     "            V = bf16_to_float(kv[layer, 1, g, max(0, pos - 2) : pos + 1, :], dtype)"),
    ("x = x + gemv(W[\"w_down\"][layer], a)", "x = gemv(W[\"w_down\"][layer], a)"),
]


@pytest.mark.parametrize("orig,mutant", _MUTATIONS)
def test_planted_oracle_mistake_is_caught(orig, mutant):
    """A plausible mistake planted in a copy of the oracle (on the CPU) breaks the
    brute-force prefix-consistency pin."""
    import inspect
    import types
    src = inspect.getsource(od)
    assert orig in src
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(orig, mutant, 1), "oracle_mutant", "exec"), mod.__dict__)
    shape, W = _tiny()
    tokens = [11, 400, 3, 2000, 9, 77]
    ref = full_forward(shape, W, tokens).numpy()
    kv = _empty_cache(shape, 8)
    worst = 0.0
    for p, t in enumerate(tokens):
        lg = mod.decode_step(shape, W, kv, t, p, dtype=np.float64)
        worst = max(worst, float(np.max(np.abs(lg - ref[p]))))
    assert worst > 1e-6
