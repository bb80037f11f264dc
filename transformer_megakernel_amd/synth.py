"""Seeded synthetic inputs for the batch-1 decode step.

This module only draws random numbers and shapes them into bf16 tensors; it holds
none of the decode arithmetic, so both the CPU oracle (through the tests) and the
HIP path consume exactly the same bits from here.

Recipe (matches the workload description of the Llama-3.2-1B megakernel article,
which measures a Llama-3.2-1B-shaped batch-1 forward; trained checkpoints are not
used, random weights of the same shape stand in for them):

* projection / embedding matrices: N(0, 0.02) drawn in fp32, rounded to bf16 (RNE);
* RMSNorm gains: 1 + N(0, 0.1), rounded to bf16;
* KV cache positions [0, ctx): N(0, 1), rounded to bf16; positions >= ctx hold a bf16
  quiet NaN (0x7FC0) by default, so that a read of a slot that is not attended shows up
  as a non-finite result instead of a small error;
* start token: uniform in [0, vocab).

Every tensor has its own generator seeded from (seed, tensor index), so tensors do
not depend on the order in which they are drawn.  On a CUDA/HIP device torch's
Philox generator is used, on the CPU torch's default generator: the bits therefore
depend on the device type, which is why callers hand the *same* tensors (copied
across devices when needed) to both sides.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List

import torch

# Shapes of the workloads (names describe what they are; sizes are the model shapes).
CONFIGS: Dict[str, dict] = {
    # Tiny Llama-style decoder used for exhaustive correctness checks.
    "tiny": dict(n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
                 ffn=1024, vocab=4096, rms_eps=1e-5, rope_theta=500000.0, tied=True),
    # Llama-3.2-1B shape (16 layers, d 2048, 32/8 heads, hd 64, F 8192, V 128256).
    "llama1b": dict(n_layers=16, hidden=2048, n_q_heads=32, n_kv_heads=8, head_dim=64,
                    ffn=8192, vocab=128256, rms_eps=1e-5, rope_theta=500000.0, tied=True),
    # Llama-3.1-8B shape (32 layers, d 4096, 32/8 heads, hd 128, F 14336, V 128256).
    "llama8b": dict(n_layers=32, hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128,
                    ffn=14336, vocab=128256, rms_eps=1e-5, rope_theta=500000.0, tied=False),
}

WEIGHT_STD = 0.02
GAIN_STD = 0.1


@dataclasses.dataclass
class ModelShape:
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    rms_eps: float
    rope_theta: float
    tied: bool = True

    @staticmethod
    def named(name: str) -> "ModelShape":
        return ModelShape(**CONFIGS[name])


def _gen(device: torch.device, seed: int, idx: int) -> torch.Generator:
    g = torch.Generator(device=device)
    # Distinct, order-independent stream per tensor.
    g.manual_seed((int(seed) * 1_000_003 + int(idx) * 7_919 + 12_345) & 0x7FFF_FFFF_FFFF)
    return g


def _normal_bf16(shape, std, mean, device, seed, idx) -> torch.Tensor:
    t = torch.empty(shape, dtype=torch.float32, device=device)
    t.normal_(mean=0.0, std=1.0, generator=_gen(device, seed, idx))
    if std != 1.0:
        t.mul_(std)
    if mean != 0.0:
        t.add_(mean)
    return t.to(torch.bfloat16)


@dataclasses.dataclass
class Weights:
    """bf16 weights, row-major [out][in] matrices, one list entry per layer."""
    embed: torch.Tensor
    lm_head: torch.Tensor          # the same tensor object as ``embed`` when tied
    final_norm: torch.Tensor
    attn_norm: List[torch.Tensor]
    wq: List[torch.Tensor]
    wk: List[torch.Tensor]
    wv: List[torch.Tensor]
    wo: List[torch.Tensor]
    mlp_norm: List[torch.Tensor]
    w_gate: List[torch.Tensor]
    w_up: List[torch.Tensor]
    w_down: List[torch.Tensor]

    def to(self, device) -> "Weights":
        def mv(x):
            return [t.to(device) for t in x] if isinstance(x, list) else x.to(device)
        emb = self.embed.to(device)
        lm = emb if self.lm_head is self.embed else self.lm_head.to(device)
        return Weights(emb, lm, mv(self.final_norm), mv(self.attn_norm), mv(self.wq),
                       mv(self.wk), mv(self.wv), mv(self.wo), mv(self.mlp_norm),
                       mv(self.w_gate), mv(self.w_up), mv(self.w_down))

    def as_numpy_bits(self) -> dict:
        """uint16 numpy views of every tensor (bf16 bit patterns), for the CPU oracle."""
        def b(t):
            return t.detach().cpu().contiguous().view(torch.int16).numpy().view("uint16")
        out = dict(embed=b(self.embed), final_norm=b(self.final_norm))
        out["lm_head"] = out["embed"] if self.lm_head is self.embed else b(self.lm_head)
        for k in ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down"):
            out[k] = [b(t) for t in getattr(self, k)]
        return out


def make_weights(shape: ModelShape, seed: int = 0, device="cpu") -> Weights:
    dev = torch.device(device)
    d, F, hd = shape.hidden, shape.ffn, shape.head_dim
    nq, nkv = shape.n_q_heads * hd, shape.n_kv_heads * hd
    idx = 0

    def nxt():
        nonlocal idx
        idx += 1
        return idx

    embed = _normal_bf16((shape.vocab, d), WEIGHT_STD, 0.0, dev, seed, nxt())
    lm_head = embed if shape.tied else _normal_bf16((shape.vocab, d), WEIGHT_STD, 0.0, dev, seed, nxt())
    final_norm = _normal_bf16((d,), GAIN_STD, 1.0, dev, seed, 1000)
    L = dict(attn_norm=[], wq=[], wk=[], wv=[], wo=[], mlp_norm=[], w_gate=[], w_up=[], w_down=[])
    for layer in range(shape.n_layers):
        base = 10_000 + 100 * layer
        L["attn_norm"].append(_normal_bf16((d,), GAIN_STD, 1.0, dev, seed, base + 0))
        L["wq"].append(_normal_bf16((nq, d), WEIGHT_STD, 0.0, dev, seed, base + 1))
        L["wk"].append(_normal_bf16((nkv, d), WEIGHT_STD, 0.0, dev, seed, base + 2))
        L["wv"].append(_normal_bf16((nkv, d), WEIGHT_STD, 0.0, dev, seed, base + 3))
        L["wo"].append(_normal_bf16((d, nq), WEIGHT_STD, 0.0, dev, seed, base + 4))
        L["mlp_norm"].append(_normal_bf16((d,), GAIN_STD, 1.0, dev, seed, base + 5))
        L["w_gate"].append(_normal_bf16((F, d), WEIGHT_STD, 0.0, dev, seed, base + 6))
        L["w_up"].append(_normal_bf16((F, d), WEIGHT_STD, 0.0, dev, seed, base + 7))
        L["w_down"].append(_normal_bf16((d, F), WEIGHT_STD, 0.0, dev, seed, base + 8))
    return Weights(embed, lm_head, final_norm, **L)


def make_kv_cache(shape: ModelShape, max_ctx: int, ctx: int, seed: int = 1, device="cpu",
                  unused: float = float("nan")) -> torch.Tensor:
    """bf16 cache laid out [layer][k|v][kv_head][max_ctx][head_dim]; [0, ctx) ~ N(0,1),
    the slots from ctx on filled with ``unused`` (a quiet NaN unless given)."""
    dev = torch.device(device)
    kv = torch.full((shape.n_layers, 2, shape.n_kv_heads, max_ctx, shape.head_dim), unused,
                    dtype=torch.bfloat16, device=dev)
    if ctx > 0:
        for layer in range(shape.n_layers):
            kv[layer, :, :, :ctx, :] = _normal_bf16(
                (2, shape.n_kv_heads, ctx, shape.head_dim), 1.0, 0.0, dev, seed, 50_000 + layer)
    return kv


def make_token(shape: ModelShape, seed: int = 2) -> int:
    g = _gen(torch.device("cpu"), seed, 99_999)
    return int(torch.randint(0, shape.vocab, (1,), generator=g).item())
