"""CPU oracle: one batch-1 decode step of a Llama-style decoder, written plainly.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or execute
this module; only the tests, the smoke check and the benchmark's CPU-baseline leg do.
It shares no code with the HIP path.

What it computes follows the Hazy Research "Megakernel" article on Llama-3.2-1B
(Chinese rewrite), section "Megakernel: a fusion design from scratch", whose list of
fused instructions fixes the order of one forward pass:

  1. RMSNorm + QKV projection + RoPE,
  2. attention matmul + reduction over the cache (grouped-query attention),
  3. O-projection + residual add,
  4. MLP RMSNorm + gate activation (SiLU) + up projection,
  5. down projection + residual add,
  6. final RMSNorm + language-model head.

The megakernel is a fusion and scheduling method, so the oracle is simply the
unfused definition of those steps (the article's 4-chunk split of the MLP
intermediate only changes when work may start, not the result).  Where the page
is silent the plainest Llama reading is taken:

* RMSNorm: n = x / sqrt(mean(x^2) + eps) * g, eps inside the root, gain applied in
  the working precision (no intermediate bf16 cast).
* RoPE: rotate-half pairing (i, i + hd/2), inverse frequency theta^(-2i/hd), angle
  pos * inv computed in float64, cos/sin rounded to the working precision; no
  Llama-3 frequency rescaling.
* GQA: query head h reads KV head floor(h * Hkv / Hq); scores scaled by 1/sqrt(hd);
  keys 0..pos inclusive.
* The new K and V are rounded to bf16 (round-to-nearest-even) when written into the
  bf16 cache, and attention reads the rounded values back.
* SiLU(z) = z / (1 + exp(-z)).
* Embedding: the raw row, no scaling.  Greedy choice: first index of the maximum.

Weights arrive as uint16 arrays holding bf16 bit patterns and are widened exactly
(bits << 16) to fp32.  ``dtype`` selects the working precision: float32 is the
parity reference, float64 serves the pins.  ``widen_weights`` performs that exact
widening once up front, for long greedy runs; every result is bit-identical to
passing the bit patterns (the widening is exact, the arithmetic is the same).

Parity status: every function here is pinned by the tests (closed forms,
invariants, library special cases, and a brute-force full-sequence forward).
"""
from __future__ import annotations

import numpy as np


# ---------------------------------------------------------------- bf16 helpers
def bf16_to_float(bits: np.ndarray, dtype=np.float32) -> np.ndarray:
    """Exact widening of bf16 bit patterns: the bf16 bits are the top half of an fp32."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(dtype)


def float_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round values to bf16 bit patterns, round-to-nearest, ties to even.

    The value is first rounded to fp32 (the cache stores what an fp32 pipeline would
    produce), then the low 16 bits are dropped with RNE.  NaN stays a quiet NaN.
    """
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(f)
    if np.any(nan):
        r = np.where(nan, ((u >> np.uint64(16)).astype(np.uint16) | np.uint16(0x0040)), r)
    return r


# ---------------------------------------------------------------- building blocks
def rms_norm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm of step 1/4/6: x / sqrt(mean(x^2) + eps), times the gain."""
    dt = x.dtype
    ms = np.mean(x * x, dtype=dt)
    return (x / np.sqrt(ms + dt.type(eps))) * g


def rope_cos_sin(pos: int, head_dim: int, theta: float, dtype=np.float32):
    """cos/sin of the rotary angles at one position, angle in float64."""
    half = head_dim // 2
    i = np.arange(half, dtype=np.float64)
    inv = np.power(np.float64(theta), -2.0 * i / head_dim)
    ang = np.float64(pos) * inv
    return np.cos(ang).astype(dtype), np.sin(ang).astype(dtype)


def apply_rope(v: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate-half RoPE of one head vector (length hd)."""
    half = v.shape[-1] // 2
    a, b = v[..., :half], v[..., half:]
    return np.concatenate([a * cos - b * sin, b * cos + a * sin], axis=-1)


def silu(z: np.ndarray) -> np.ndarray:
    one = z.dtype.type(1)
    return z / (one + np.exp(-z))


def attend_one_head(q: np.ndarray, K: np.ndarray, V: np.ndarray) -> np.ndarray:
    """Softmax attention of one query over keys K[j], values V[j] (rows), 1/sqrt(hd)."""
    dt = q.dtype
    s = (K @ q) / np.sqrt(dt.type(q.shape[0]))
    m = np.max(s)
    p = np.exp(s - m)
    p = p / np.sum(p, dtype=dt)
    return p @ V


def _values(w: np.ndarray, dtype) -> np.ndarray:
    """The values of a weight tensor given as bf16 bit patterns (uint16), or already
    widened exactly to a float type by ``widen_weights``."""
    if w.dtype == np.uint16:
        return bf16_to_float(w, dtype)
    return w.astype(dtype, copy=False)


def widen_weights(W: dict) -> dict:
    """The same weights with every bf16 bit pattern widened exactly to float32, once."""
    out = {}
    for k, v in W.items():
        out[k] = [bf16_to_float(t) for t in v] if isinstance(v, list) else bf16_to_float(v)
    if W.get("lm_head") is W.get("embed"):
        out["lm_head"] = out["embed"]
    return out


def gemv(W_bits: np.ndarray, x: np.ndarray) -> np.ndarray:
    """y = W x with W given as bf16 bits [out][in]; widened exactly, product in x's precision."""
    return _values(W_bits, x.dtype) @ x


# ---------------------------------------------------------------- the decode step
def decode_step(cfg, W: dict, kv: np.ndarray, token: int, pos: int, dtype=np.float32,
                return_next: bool = False, trace: dict = None):
    """One decode step: process ``token`` at position ``pos``.

    ``cfg`` has attributes n_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn,
    vocab, rms_eps, rope_theta.  ``W`` maps names to uint16 bf16-bit arrays (lists
    per layer).  ``kv`` is the uint16 cache [layer][k|v][kv_head][max_ctx][hd]; slot
    ``pos`` of every layer is overwritten (in place) with the new rounded K and V.
    Returns the logits (``dtype``, length vocab), and the argmax when asked.  When
    ``trace`` is a dict it receives the intermediates per layer: raw q/k/v (before
    RoPE), attention output o, SiLU(gate)*up, and x after each residual add.
    """
    hd, Hq, Hkv = cfg.head_dim, cfg.n_q_heads, cfg.n_kv_heads
    eps = cfg.rms_eps
    if not (0 <= pos < kv.shape[3]):
        raise ValueError("pos outside the cache")
    cos, sin = rope_cos_sin(pos, hd, cfg.rope_theta, dtype)

    x = _values(W["embed"][token], dtype)
    for layer in range(cfg.n_layers):
        # 1. RMSNorm + QKV projection + RoPE (+ append K, V to the cache)
        n = rms_norm(x, _values(W["attn_norm"][layer], dtype), eps)
        q = gemv(W["wq"][layer], n).reshape(Hq, hd)
        k = gemv(W["wk"][layer], n).reshape(Hkv, hd)
        v = gemv(W["wv"][layer], n).reshape(Hkv, hd)
        if trace is not None:
            trace.setdefault("q", []).append(q.copy())
            trace.setdefault("k", []).append(k.copy())
            trace.setdefault("v", []).append(v.copy())
        q = apply_rope(q, cos, sin)
        k = apply_rope(k, cos, sin)
        kv[layer, 0, :, pos, :] = float_to_bf16(k)
        kv[layer, 1, :, pos, :] = float_to_bf16(v)
        # 2. attention over keys 0..pos of the matching KV head
        o = np.empty((Hq, hd), dtype=dtype)
        for h in range(Hq):
            g = (h * Hkv) // Hq
            K = bf16_to_float(kv[layer, 0, g, : pos + 1, :], dtype)
            V = bf16_to_float(kv[layer, 1, g, : pos + 1, :], dtype)
            o[h] = attend_one_head(q[h], K, V)
        # 3. O-projection + residual
        x = x + gemv(W["wo"][layer], o.reshape(-1))
        if trace is not None:
            trace.setdefault("o", []).append(o.reshape(-1).copy())
            trace.setdefault("x", []).append(x.copy())
        # 4. MLP RMSNorm + SiLU(gate) * up
        n2 = rms_norm(x, _values(W["mlp_norm"][layer], dtype), eps)
        a = silu(gemv(W["w_gate"][layer], n2)) * gemv(W["w_up"][layer], n2)
        # 5. down projection + residual
        x = x + gemv(W["w_down"][layer], a)
        if trace is not None:
            trace.setdefault("a", []).append(a.copy())
            trace["x"].append(x.copy())
    # 6. final RMSNorm + LM head
    nf = rms_norm(x, _values(W["final_norm"], dtype), eps)
    logits = gemv(W["lm_head"], nf)
    if return_next:
        return logits, int(np.argmax(logits))
    return logits


def greedy_decode(cfg, W: dict, kv: np.ndarray, token: int, pos0: int, n_steps: int,
                  dtype=np.float32):
    """Greedy generation: feed the argmax back as the next token, one position at a time.

    Returns (tokens produced, list of per-step logits)."""
    toks, all_logits = [], []
    tok = token
    for i in range(n_steps):
        logits, tok = decode_step(cfg, W, kv, tok, pos0 + i, dtype, return_next=True)
        toks.append(tok)
        all_logits.append(logits)
    return toks, all_logits
