"""Algorithmic byte and flop model of one batch-1 decode step.

The Megakernel article (section "Why are traditional inference methods so
inefficient?") prices one Llama-1B forward as the bytes it must move: 2.48 GB per
forward against 3.35 TB/s gives ~1350 forwards/s, and 7 kernels per layer x 16
layers x 5 us of stall pull that under 770/s.  The same accounting is used here:

* every weight element (bf16) is read exactly once, norm gains included;
* only the embedding row of the token is read;
* the KV cache is read once per layer for keys 0..pos (GQA shares it between the
  query heads of a group), and the new K and V are written once;
* the fp32 logits are written once.

Activation traffic (a few KB per phase, served from cache) is not counted.
"""
from __future__ import annotations

MI355X_HBM_PEAK_GBS = 8000.0          # published HBM3E bandwidth, GB/s
MI355X_CUS = 256
MI355X_CLOCK_GHZ = 2.4


def weight_bytes(s) -> int:
    d, F, hd = s.hidden, s.ffn, s.head_dim
    nq, nkv = s.n_q_heads * hd, s.n_kv_heads * hd
    per_layer = (nq + 2 * nkv) * d + d * nq + 2 * F * d + d * F + 2 * d   # + 2 gains
    return 2 * (s.n_layers * per_layer + s.vocab * d + d)                  # + LM head + final gain


def kv_bytes_per_position_per_layer(s) -> int:
    return 2 * s.n_kv_heads * s.head_dim * 2            # K and V, bf16


def step_bytes(s, pos: int) -> dict:
    """Bytes one step at position ``pos`` must move (keys 0..pos are attended)."""
    w = weight_bytes(s)
    kvp = kv_bytes_per_position_per_layer(s)
    parts = dict(
        weights=w,
        embed_row=2 * s.hidden,
        kv_read=s.n_layers * (pos + 1) * kvp,
        kv_write=s.n_layers * kvp,
        logits=4 * s.vocab,
    )
    parts["total"] = sum(parts.values())
    return parts


def step_flops(s, pos: int) -> int:
    """2 flops per weight element of every projection, plus q.k and p.v per key."""
    d, F, hd = s.hidden, s.ffn, s.head_dim
    nq, nkv = s.n_q_heads * hd, s.n_kv_heads * hd
    mats = s.n_layers * ((nq + 2 * nkv) * d + d * nq + 3 * F * d) + s.vocab * d
    attn = s.n_layers * 4 * s.n_q_heads * hd * (pos + 1)
    return 2 * mats + attn


def forwards_per_second(bytes_per_forward: float, bandwidth_Bps: float,
                        n_kernels: int = 0, stall_s: float = 0.0) -> float:
    """The article's bubble model: time = bytes / bandwidth + kernels x stall."""
    return 1.0 / (bytes_per_forward / bandwidth_Bps + n_kernels * stall_s)
