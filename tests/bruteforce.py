"""Brute-force full-sequence forward in float64, textbook matrix form (a test pin).

Independent of the oracle: torch instead of numpy, whole-sequence matrices with a
causal mask instead of an incremental cache.  It applies the same readings of the
Megakernel article's instruction list (rotate-half RoPE, contiguous GQA groups,
eps inside the root, K/V stored as bf16) so that an incremental decode from an
empty cache must reproduce every row of it.
"""
from __future__ import annotations

import math

import numpy as np
import torch


def _w(bits, dtype=torch.float64):
    u = (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.int32)
    return torch.from_numpy(u).view(torch.float32).to(dtype)


def _bf16_store(x: torch.Tensor) -> torch.Tensor:
    """What a bf16 cache holds: fp32 value rounded to bf16 by torch's own conversion."""
    return x.to(torch.float32).to(torch.bfloat16).to(torch.float64)


def full_forward(cfg, W: dict, tokens) -> torch.Tensor:
    """Logits [T][V] for every prefix of ``tokens`` starting at position 0."""
    T = len(tokens)
    d, hd, Hq, Hkv = cfg.hidden, cfg.head_dim, cfg.n_q_heads, cfg.n_kv_heads
    X = _w(W["embed"])[torch.tensor(tokens)]                       # [T][d]

    half = hd // 2
    freq = torch.tensor([cfg.rope_theta ** (-(2.0 * i) / hd) for i in range(half)],
                        dtype=torch.float64)
    ang = torch.arange(T, dtype=torch.float64)[:, None] * freq[None, :]   # [T][half]
    c, s = torch.cos(ang), torch.sin(ang)

    def rope(M):  # M [T][H][hd] -> rotated; the pair (i, i+half) turns by angle pos*freq_i
        re, im = M[..., :half], M[..., half:]
        cc, ss = c[:, None, :], s[:, None, :]
        return torch.cat([re * cc - im * ss, im * cc + re * ss], dim=-1)

    def norm(A, g):
        return A / torch.sqrt((A * A).mean(dim=-1, keepdim=True) + cfg.rms_eps) * g

    mask = torch.ones(T, T, dtype=torch.bool).tril()
    for layer in range(cfg.n_layers):
        N = norm(X, _w(W["attn_norm"][layer]))
        Q = (N @ _w(W["wq"][layer]).T).reshape(T, Hq, hd)
        K = (N @ _w(W["wk"][layer]).T).reshape(T, Hkv, hd)
        V = (N @ _w(W["wv"][layer]).T).reshape(T, Hkv, hd)
        Q, K = rope(Q), rope(K)
        K, V = _bf16_store(K), _bf16_store(V)
        rep = Hq // Hkv
        Kr = K.repeat_interleave(rep, dim=1)        # head h -> kv head h // rep
        Vr = V.repeat_interleave(rep, dim=1)
        S = torch.einsum("thd,uhd->htu", Q, Kr) / math.sqrt(hd)
        S = S.masked_fill(~mask[None], float("-inf"))
        P = torch.softmax(S, dim=-1)
        O = torch.einsum("htu,uhd->thd", P, Vr).reshape(T, Hq * hd)
        X = X + O @ _w(W["wo"][layer]).T
        N2 = norm(X, _w(W["mlp_norm"][layer]))
        G = N2 @ _w(W["w_gate"][layer]).T
        U = N2 @ _w(W["w_up"][layer]).T
        A = torch.nn.functional.silu(G) * U
        X = X + A @ _w(W["w_down"][layer]).T
    NF = norm(X, _w(W["final_norm"]))
    return NF @ _w(W["lm_head"]).T
