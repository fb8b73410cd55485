"""One batch-1 decode step of a Qwen3-style decoder (oracle; test
infrastructure only).

The model is the one the monolith project page describes ("Upstream facts":
Qwen3-0.6B, a pre-norm decoder with QK-norm, i.e. RMSNorm on q and k per
head, RoPE, grouped-query attention with 16 query and 8 KV heads, a SwiGLU
MLP, and a tied embedding used as the LM head), decoded greedily at batch 1.
Where the page is silent the plain readings are:
  * RMSNorm y = g * (x / sqrt(mean(x^2) + eps)), eps = 1e-6, gains multiply.
  * q/k-norm: one gain vector of head_dim per layer, shared by all heads,
    applied before RoPE.
  * RoPE: rotate-half pairs (i, i + hd/2) over the full head; angle
    p * theta^(-2i/hd) evaluated in float64, cos and sin rounded to float32.
  * attention: scores q.k / sqrt(hd) over positions 0..p, softmax, no bias,
    window or soft-cap; query head h reads KV head h // (nq / nkv).
  * MLP: down(silu(gate(x)) * up(x)), silu(z) = z / (1 + e^-z), no biases.
  * rounding points (the page keeps activations and the KV cache in bf16):
    the input of every GEMV, the K and V written to the cache, and the
    final-norm output are rounded to bf16.  The residual stream, q, GEMV
    outputs and logits stay float32.
  * argmax: the smallest index among the maximal logits.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

from .codecs import bf16_bits_to_f32, bf16_round
from .quant import Fp4Block, Fp8Row, quant_fp4, quant_fp8_row

BF16, FP8_ROW, FP4_MIX = 0, 1, 2
LINEARS = ("q", "k", "v", "o", "gate", "up", "down")
NORMS = ("in_norm", "q_norm", "k_norm", "post_norm")


def tensor_format(wfmt: int, name: str) -> str:
    """Which format a tensor is stored in.  FP8_ROW: every linear and the tied
    embedding in FP8.  FP4_MIX: q, k, v, o, gate, up in NVFP4; down and the
    embedding in FP8 (the page keeps sensitive matrices and the LM head in
    FP8).  Norm gains always stay bf16."""
    if name in NORMS or name == "final_norm" or wfmt == BF16:
        return "bf16"
    if wfmt == FP8_ROW:
        return "fp8"
    if wfmt == FP4_MIX:
        return "fp8" if name in ("down", "embed") else "fp4"
    raise ValueError(f"unknown weight format {wfmt}")


# ------------------------------------------------------------ primitives
def quantize_tensor(bits: np.ndarray, fmt: str, fp4_search: int = 0):
    """Store one bf16 master tensor in `fmt` ("bf16", "fp8" or "fp4") and
    return (the packed form, its float32 dequantization).  FP8 scales are per
    row, so rows of a tensor may be quantized on their own; FP4 needs the
    whole tensor (its tensor scale).  `fp4_search` is the NVFP4 block scale
    search radius (0: the absolute-maximum recipe)."""
    w = bf16_bits_to_f32(bits)
    if fmt == "fp8":
        p = quant_fp8_row(w)
        return p, p.dequant()
    if fmt == "fp4":
        p = quant_fp4(w, fp4_search)
        return p, p.dequant()
    return bits, w


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float, dt=np.float32) -> np.ndarray:
    """g * (x / sqrt(mean(x^2) + eps)) along the last axis."""
    x = x.astype(dt)
    ms = np.mean(x * x, axis=-1, keepdims=True, dtype=dt)
    r = dt(1.0) / np.sqrt(ms + dt(eps))
    return (g.astype(dt) * (x * r)).astype(dt)


def rope_table(n_pos: int, head_dim: int, theta: float) -> Tuple[np.ndarray, np.ndarray]:
    """cos and sin of p * theta^(-2i/hd), angle in float64, each rounded once
    to float32.  Shape [n_pos, hd/2]."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    omega = np.power(np.float64(theta), -2.0 * i / head_dim)
    ang = np.arange(n_pos, dtype=np.float64)[:, None] * omega[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def apply_rope(x: np.ndarray, cos: np.ndarray, sin: np.ndarray, dt=np.float32) -> np.ndarray:
    """Rotate pairs (x_i, x_{i+hd/2}) by the angle whose cos/sin are given:
    x'_i = x_i c - x_{i+hd/2} s ; x'_{i+hd/2} = x_{i+hd/2} c + x_i s."""
    half = x.shape[-1] // 2
    a, b = x[..., :half].astype(dt), x[..., half:].astype(dt)
    c, s = cos.astype(dt), sin.astype(dt)
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1).astype(dt)


def softmax(s: np.ndarray, dt=np.float32) -> np.ndarray:
    s = s.astype(dt)
    e = np.exp(s - np.max(s, axis=-1, keepdims=True))
    return (e / np.sum(e, axis=-1, keepdims=True, dtype=dt)).astype(dt)


def silu(z: np.ndarray, dt=np.float32) -> np.ndarray:
    z = z.astype(dt)
    return (z / (dt(1.0) + np.exp(-z))).astype(dt)


def gqa_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, dt=np.float32) -> np.ndarray:
    """q [nq, hd]; k, v [nkv, n, hd] (positions 0..n-1).  Query head h uses
    KV head h // (nq / nkv).  Returns o [nq, hd]."""
    nq, hd = q.shape
    nkv = k.shape[0]
    group = nq // nkv
    out = np.empty((nq, hd), dtype=dt)
    scale = dt(np.sqrt(dt(hd)))
    for h in range(nq):
        g = h // group
        s = (k[g].astype(dt) @ q[h].astype(dt)).astype(dt) / scale
        p = softmax(s, dt)
        out[h] = (p @ v[g].astype(dt)).astype(dt)
    return out


def argmax_lowest(logits: np.ndarray) -> int:
    """Smallest index i with logits[i] == max(logits)."""
    m = np.max(logits)
    return int(np.flatnonzero(logits == m)[0])


# ---------------------------------------------------------------- model
@dataclasses.dataclass
class KVCache:
    k: np.ndarray   # [L, nkv, max_ctx, hd] (bf16 values held as float)
    v: np.ndarray


class Oracle:
    """Quantizes a bf16 master per the weight format and runs decode steps.

    `dtype` is the arithmetic type (float32 by default); `round_bf16=False`
    removes the bf16 rounding points (used with float64 only, to bound the
    oracle's own rounding); `fp4_search` is the NVFP4 block scale search
    radius (0: the absolute-maximum recipe)."""

    def __init__(self, master, wfmt: int, max_ctx: int, dtype=np.float32,
                 round_bf16: bool = True, fp4_search: int = 0):
        sh = master.shape
        self.fp4_search = fp4_search
        self.shape, self.wfmt, self.max_ctx = sh, wfmt, max_ctx
        self.dt, self.round_bf16 = dtype, round_bf16
        self.eps = sh.rms_eps
        self.packed: Dict[Tuple[int, str], object] = {}
        # tensors are independent, so they are prepared on a thread pool
        from concurrent.futures import ThreadPoolExecutor
        import os
        jobs = [(-1, "embed", master.embed)]
        jobs += [(l, name, bits) for l, layer in enumerate(master.layers) for name, bits in layer.items()]
        with ThreadPoolExecutor(min(16, len(os.sched_getaffinity(0)))) as ex:
            done = list(ex.map(lambda j: self._prepare(*j), jobs))
        self.embed = done[0]
        self.w: List[Dict[str, np.ndarray]] = [dict() for _ in master.layers]
        for (l, name, _), w in zip(jobs[1:], done[1:]):
            self.w[l][name] = w
        self.final_norm = bf16_bits_to_f32(master.final_norm).astype(dtype)
        self.cos, self.sin = rope_table(max_ctx, sh.head_dim, sh.rope_theta)

    def _prepare(self, layer: int, name: str, bits: np.ndarray) -> np.ndarray:
        p, w = quantize_tensor(bits, tensor_format(self.wfmt, name), self.fp4_search)
        self.packed[(layer, name)] = p
        return w.astype(self.dt)

    def _r(self, x: np.ndarray) -> np.ndarray:
        """bf16 rounding point."""
        if not self.round_bf16:
            return x.astype(self.dt)
        return bf16_round(x.astype(np.float32)).astype(self.dt)

    def new_cache(self) -> KVCache:
        sh = self.shape
        z = np.zeros((sh.n_layers, sh.n_kv_heads, self.max_ctx, sh.head_dim), dtype=self.dt)
        return KVCache(z, z.copy())

    def step(self, cache: KVCache, token: int, pos: int, trace: Optional[dict] = None) -> np.ndarray:
        """One decode step at position `pos`; writes K/V at `pos` and returns
        float logits over the vocabulary.  With `trace`, also records each
        layer's intermediates under (layer, name): "qkv" the q, k, v GEMV
        outputs (concatenated, before the q/k norms), "attn" the attention
        output as the O-projection reads it, "x_o" the residual after the
        O-projection, "h" the SwiGLU output, "x_d" the residual after the
        down projection."""
        sh, dt = self.shape, self.dt
        if not (0 <= pos < self.max_ctx) or not (0 <= token < sh.vocab):
            raise ValueError("token or position out of range")
        nq, nkv, hd = sh.n_q_heads, sh.n_kv_heads, sh.head_dim
        x = self.embed[token].astype(dt).copy()
        cos, sin = self.cos[pos], self.sin[pos]
        for l, w in enumerate(self.w):
            xn = self._r(rmsnorm(x, w["in_norm"], self.eps, dt))
            q = (w["q"] @ xn).astype(dt).reshape(nq, hd)
            k = (w["k"] @ xn).astype(dt).reshape(nkv, hd)
            v = (w["v"] @ xn).astype(dt).reshape(nkv, hd)
            if trace is not None:
                trace[(l, "qkv")] = np.concatenate([q.reshape(-1), k.reshape(-1), v.reshape(-1)])
            q = apply_rope(rmsnorm(q, w["q_norm"], self.eps, dt), cos, sin, dt)
            k = apply_rope(rmsnorm(k, w["k_norm"], self.eps, dt), cos, sin, dt)
            cache.k[l, :, pos] = self._r(k)
            cache.v[l, :, pos] = self._r(v)
            o = gqa_attention(q, cache.k[l, :, :pos + 1], cache.v[l, :, :pos + 1], dt)
            o = self._r(o.reshape(-1))
            x = (x + (w["o"] @ o).astype(dt)).astype(dt)
            xn2 = self._r(rmsnorm(x, w["post_norm"], self.eps, dt))
            g = (w["gate"] @ xn2).astype(dt)
            u = (w["up"] @ xn2).astype(dt)
            h = self._r(silu(g, dt) * u)
            if trace is not None:
                trace[(l, "attn")], trace[(l, "x_o")], trace[(l, "h")] = o, x.copy(), h
            x = (x + (w["down"] @ h).astype(dt)).astype(dt)
            if trace is not None:
                trace[(l, "x_d")] = x.copy()
        xf = self._r(rmsnorm(x, self.final_norm, self.eps, dt))
        return (self.embed @ xf).astype(dt)

    def prefill(self, cache: KVCache, tokens: Sequence[int]) -> Tuple[int, np.ndarray]:
        """Decode steps at positions 0..P-1 with the prompt's tokens; returns
        the greedy token after the prompt and the last logits."""
        logits = None
        for p, t in enumerate(tokens):
            logits = self.step(cache, int(t), p)
        return argmax_lowest(logits), logits

    def prefill_batched(self, cache: KVCache, tokens: Sequence[int]) -> Tuple[int, np.ndarray]:
        """The same computation as `prefill`, all positions at once: each
        position's row goes through exactly the steps of `step`, with the
        products taken as matrix-matrix multiplies (only the summation order
        differs).  Used for long prompts."""
        sh, dt = self.shape, self.dt
        toks = np.asarray(tokens, dtype=np.int64)
        n = len(toks)
        nq, nkv, hd = sh.n_q_heads, sh.n_kv_heads, sh.head_dim
        group = nq // nkv
        x = self.embed[toks].astype(dt)
        cos, sin = self.cos[:n][:, None, :], self.sin[:n][:, None, :]
        causal = np.triu(np.ones((n, n), dtype=bool), 1)
        scale = dt(np.sqrt(dt(hd)))
        for l, w in enumerate(self.w):
            xn = self._r(rmsnorm(x, w["in_norm"], self.eps, dt))
            q = (xn @ w["q"].T).astype(dt).reshape(n, nq, hd)
            k = (xn @ w["k"].T).astype(dt).reshape(n, nkv, hd)
            v = (xn @ w["v"].T).astype(dt).reshape(n, nkv, hd)
            q = apply_rope(rmsnorm(q, w["q_norm"], self.eps, dt), cos, sin, dt)
            k = apply_rope(rmsnorm(k, w["k_norm"], self.eps, dt), cos, sin, dt)
            kr, vr = self._r(k), self._r(v)
            cache.k[l, :, :n] = kr.transpose(1, 0, 2)
            cache.v[l, :, :n] = vr.transpose(1, 0, 2)
            o = np.empty((n, nq, hd), dtype=dt)
            for h in range(nq):
                g = h // group
                s = (q[:, h, :] @ kr[:, g, :].T).astype(dt) / scale
                s = np.where(causal, -np.inf, s).astype(dt)
                o[:, h, :] = (softmax(s, dt) @ vr[:, g, :]).astype(dt)
            x = (x + (self._r(o.reshape(n, -1)) @ w["o"].T).astype(dt)).astype(dt)
            xn2 = self._r(rmsnorm(x, w["post_norm"], self.eps, dt))
            g_ = (xn2 @ w["gate"].T).astype(dt)
            u = (xn2 @ w["up"].T).astype(dt)
            h_ = self._r(silu(g_, dt) * u)
            x = (x + (h_ @ w["down"].T).astype(dt)).astype(dt)
        xf = self._r(rmsnorm(x[-1], self.final_norm, self.eps, dt))
        logits = (self.embed @ xf).astype(dt)
        return argmax_lowest(logits), logits

    def generate(self, prompt: Sequence[int], n_steps: int,
                 forced: Optional[Sequence[int]] = None, batched_prefill: bool = False):
        """Prefill the prompt, then `n_steps` greedy decode steps starting at
        position len(prompt).  With `forced`, step i consumes forced[i]
        (teacher forcing) instead of the previous argmax.  Returns the
        argmax of every step (the first is the prefill's) and the logits of
        every decode step."""
        cache = self.new_cache()
        fill = self.prefill_batched if batched_prefill else self.prefill
        nxt, _ = fill(cache, prompt)
        tokens, all_logits = [nxt], []
        pos = len(prompt)
        for i in range(n_steps):
            t = int(forced[i]) if forced is not None else tokens[-1]
            logits = self.step(cache, t, pos + i)
            all_logits.append(logits)
            tokens.append(argmax_lowest(logits))
        return tokens, all_logits
