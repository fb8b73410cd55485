"""Seeded synthetic inputs for the batch-1 decode path.

This module is shared by the oracle's tests, the HIP path's tests and the
benchmark. It holds model shapes, run lengths and random draws only; none of
the decode arithmetic (norms, quantizers, GEMVs, attention) lives here.

Workloads follow the monolith project page (projects.dotslasha.me/p/monolith,
"Upstream facts": Qwen3-0.6B has hidden 1024, intermediate 3072, 28 layers,
16 query heads, 8 KV heads, head_dim 128, vocab 151,936, tied embeddings,
QK-norm and RoPE). The real checkpoint, prompt set and WikiText-2 are not
available, so random weights and uniform random prompts of the same shapes
stand in for them: decode speed depends only on shapes and positions.

Recipe (one bf16 master per shape; the quantized configs quantize it):
  * tensor order: embed; per layer (in_norm, q, k, v, q_norm, k_norm, o,
    post_norm, gate, up, down); final_norm.  Tensor i is drawn from
    numpy.random.default_rng([seed, i]).
  * linear and embedding tensors: float32 standard normal times 0.02,
    rounded to bfloat16 (round to nearest even, by torch's cast).
  * norm gains: 1 + 0.1 * standard normal, rounded the same way.
  * prompts: default_rng(prompt_seed).integers(0, vocab, P), uniform.
"""
from __future__ import annotations

import dataclasses
import os
from typing import Dict, List

import numpy as np

# Weight formats.  The integer values are the ones the C-ABI uses.
BF16 = 0
FP8_ROW = 1
FP4_MIX = 2
WFMT_NAMES = {BF16: "bf16", FP8_ROW: "fp8_row", FP4_MIX: "fp4_mix"}

LAYER_TENSORS = ("in_norm", "q", "k", "v", "q_norm", "k_norm", "o",
                 "post_norm", "gate", "up", "down")
NORM_TENSORS = ("in_norm", "q_norm", "k_norm", "post_norm")


@dataclasses.dataclass(frozen=True)
class Shape:
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    vocab: int
    rope_theta: float = 1.0e6
    rms_eps: float = 1.0e-6

    def tensor_shapes(self) -> Dict[str, tuple]:
        """[out, in] shapes of one layer's tensors (PyTorch Linear layout)."""
        H, hd, I = self.hidden, self.head_dim, self.intermediate
        return {
            "in_norm": (H,), "q": (self.n_q_heads * hd, H),
            "k": (self.n_kv_heads * hd, H), "v": (self.n_kv_heads * hd, H),
            "q_norm": (hd,), "k_norm": (hd,), "o": (H, self.n_q_heads * hd),
            "post_norm": (H,), "gate": (I, H), "up": (I, H), "down": (H, I),
        }


TINY = Shape(n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
             intermediate=768, vocab=4096)
QWEN3_0P6B = Shape(n_layers=28, hidden=1024, n_q_heads=16, n_kv_heads=8,
                   head_dim=128, intermediate=3072, vocab=151936)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    shape: Shape
    wfmt: int
    prompt_len: int
    decode_steps: int
    max_ctx: int
    weight_seed: int = 0
    prompt_seed: int = 1


WORKLOADS = {
    w.name: w for w in (
        Workload("tiny_bf16", TINY, BF16, 16, 32, 2048),
        Workload("qwen3_0p6b_bf16", QWEN3_0P6B, BF16, 128, 256, 2048),
        Workload("qwen3_0p6b_fp8", QWEN3_0P6B, FP8_ROW, 128, 256, 2048),
        Workload("qwen3_0p6b_fp4mix", QWEN3_0P6B, FP4_MIX, 512, 512, 2048),
        Workload("qwen3_0p6b_fp8_long", QWEN3_0P6B, FP8_ROW, 16384, 128, 16512),
    )
}


def _to_bf16_bits(x: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def _draw(seed: int, index: int, shape: tuple, is_norm: bool) -> np.ndarray:
    rng = np.random.default_rng([seed, index])
    z = rng.standard_normal(shape, dtype=np.float32)
    if is_norm:
        z = np.float32(1.0) + np.float32(0.1) * z
    else:
        z = np.float32(0.02) * z
    return _to_bf16_bits(z)


@dataclasses.dataclass
class MasterWeights:
    """bf16 master weights as uint16 bit patterns."""
    shape: Shape
    embed: np.ndarray                  # [V, H]
    layers: List[Dict[str, np.ndarray]]
    final_norm: np.ndarray             # [H]


def make_weights(shape: Shape, seed: int = 0, zero_linears: bool = False) -> MasterWeights:
    """Draw the bf16 master for `shape`.  `zero_linears` zeroes every layer
    linear (q, k, v, o, gate, up, down), a degenerate case used by tests.
    Tensors are drawn in parallel; each has its own generator, so the result
    does not depend on the order."""
    from concurrent.futures import ThreadPoolExecutor
    shapes = shape.tensor_shapes()
    jobs = [(0, (shape.vocab, shape.hidden), False)]
    for l in range(shape.n_layers):
        for j, name in enumerate(LAYER_TENSORS):
            jobs.append((1 + 11 * l + j, shapes[name], name in NORM_TENSORS))
    jobs.append((1 + 11 * shape.n_layers, (shape.hidden,), True))
    workers = min(16, len(os.sched_getaffinity(0)))
    with ThreadPoolExecutor(workers) as ex:
        out = list(ex.map(lambda j: _draw(seed, *j), jobs))
    embed, final_norm = out[0], out[-1]
    layers = []
    for l in range(shape.n_layers):
        layer = {}
        for j, name in enumerate(LAYER_TENSORS):
            t = out[1 + 11 * l + j]
            if zero_linears and name not in NORM_TENSORS:
                t[...] = 0
            layer[name] = t
        layers.append(layer)
    return MasterWeights(shape, embed, layers, final_norm)


def make_prompt(vocab: int, length: int, seed: int = 1) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return rng.integers(0, vocab, length).astype(np.int32)
