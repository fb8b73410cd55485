"""Op-by-op checker: recompute each phase of a decode step with the
oracle's functions from the input that phase actually had.

Each comparison then sees only that phase's rounding, not the drift
accumulated over the layers before it, so the tolerances are tight:

* fp32 GEMV outputs (q/k/v, residuals): |got - ref| <= 1e-4 * sum_j |w_ij x_j|
  (+ the residual's magnitude), which admits another summation order and a
  few activation elements rounded to the neighbouring bf16 value, but not one
  missing or doubled product term;
* bf16 outputs (attention, SwiGLU): one bf16 step (2^-7 relative) plus the
  propagated fp32 error of their inputs;
* the V row appended to the cache is bit-exact (same fp32 value, same
  rounding), the K row within one bf16 step (norm and rotation in another
  order).

tests/test_opcheck.py pins these comparisons on the CPU (it accepts the oracle's
own intermediates and rejects planted mistakes); tests/test_gpu_ops.py
applies it to the GPU.
"""
import numpy as np

from oracle.codecs import bf16_bits_to_f32, bf16_round
from oracle.model import (apply_rope, argmax_lowest, gqa_attention, quantize_tensor, rmsnorm, rope_table, silu,
                          tensor_format)

GEMV_REL = 1e-4
BF16_STEP = 2.0 ** -7


class Weights:
    """The oracle's dequantized weights of one master in one format, made
    on demand (FP8 scales are per row, so sampled rows are quantized alone;
    an FP4 tensor is quantized whole for its tensor scale)."""

    def __init__(self, master, wfmt, fp4_search=0):
        self.m, self.wfmt, self.full, self.search = master, wfmt, {}, fp4_search

    def rows(self, l, name, rows):
        bits = self.m.embed if name == "embed" else self.m.layers[l][name]
        fmt = tensor_format(self.wfmt, name)
        if fmt == "fp4":
            key = (l, name)
            if key not in self.full:
                self.full[key] = quantize_tensor(bits, fmt, self.search)[1]
            return self.full[key][rows]
        return quantize_tensor(bits[rows], fmt)[1]

    def gain(self, l, name):
        return bf16_bits_to_f32(self.m.final_norm if name == "final_norm" else self.m.layers[l][name])


def _gemv(w, x):
    """w @ x in float64 and the bound sum_j |w_ij x_j|."""
    w64, x64 = w.astype(np.float64), x.astype(np.float64)
    return w64 @ x64, np.abs(w64) @ np.abs(x64)


def _close_fp32(got, ref, bound, what):
    err = np.abs(got.astype(np.float64) - ref)
    lim = GEMV_REL * bound + 1e-7
    bad = np.flatnonzero(err > lim)
    assert bad.size == 0, (what, bad[:8], err[bad[:8]], lim[bad[:8]])


def _close_bf16(got, ref, slack, what):
    """got is bf16-valued; ref is the unrounded reference.  got must be one
    of the bf16 neighbours of a value within `slack` of ref."""
    got, ref = np.ravel(got), np.ravel(ref)
    slack = np.broadcast_to(slack, ref.shape).ravel()
    assert np.array_equal(got, bf16_round(got.astype(np.float32))), (what, "not bf16 values")
    err = np.abs(got.astype(np.float64) - ref)
    lim = BF16_STEP * np.maximum(np.abs(ref), np.abs(got)) + slack + 1e-30
    bad = np.flatnonzero(err > lim)
    assert bad.size == 0, (what, bad[:8], got[bad[:8]], ref[bad[:8]], lim[bad[:8]])


def check_step(dec, W, sh, token, pos, logits, layers, rng, n_sample=None):
    """Recompute every phase of the step that just ran (token at pos) from
    the inputs it had; with n_sample, only that many rows of each matrix.
    `dec` gives the step's intermediates: read_exchange(layer, vec) with vec
    in qkv, attn, x_o, h, x_d, and kv_bits(), the bf16 KV cache as uint16
    [L][2][nkv][ctx][hd]."""
    nq, nkv, hd, H, I = sh.n_q_heads, sh.n_kv_heads, sh.head_dim, sh.hidden, sh.intermediate
    eps = sh.rms_eps

    def pick(n):
        if n_sample is None or n_sample >= n:
            return np.arange(n)
        r = rng.choice(n, n_sample, replace=False)
        return np.unique(np.concatenate([r, [0, n - 1]]))

    cos, sin = rope_table(pos + 1, hd, sh.rope_theta)
    cos, sin = cos[pos], sin[pos]
    kv = dec.kv_bits()
    for l in layers:
        x_prev = W.rows(0, "embed", [token])[0] if l == 0 else dec.read_exchange(l - 1, "x_d")
        # fused QKV GEMV on the normalised, bf16-rounded residual
        xn = bf16_round(rmsnorm(x_prev, W.gain(l, "in_norm"), eps))
        qkv = dec.read_exchange(l, "qkv")
        for name, base, n in (("q", 0, nq * hd), ("k", nq * hd, nkv * hd), ("v", (nq + nkv) * hd, nkv * hd)):
            r = pick(n)
            ref, bound = _gemv(W.rows(l, name, r), xn)
            _close_fp32(qkv[base + r], ref, bound, (l, name))
        # q/k norm + RoPE from the GPU's q/k/v; the rows appended to the cache
        q = apply_rope(rmsnorm(qkv[:nq * hd].reshape(nq, hd), W.gain(l, "q_norm"), eps), cos, sin)
        k = apply_rope(rmsnorm(qkv[nq * hd:(nq + nkv) * hd].reshape(nkv, hd), W.gain(l, "k_norm"), eps), cos, sin)
        v = qkv[(nq + nkv) * hd:].reshape(nkv, hd)
        k_row = bf16_bits_to_f32(kv[l, 0, :, pos])
        v_row = bf16_bits_to_f32(kv[l, 1, :, pos])
        assert np.array_equal(v_row, bf16_round(v)), (l, "V append")
        _close_bf16(k_row, k.astype(np.float64), 1e-6 * np.abs(k).max(), (l, "K append"))
        # attention over the GPU's cache (positions 0..pos, its own rows included)
        K = bf16_bits_to_f32(kv[l, 0, :, :pos + 1])
        V = bf16_bits_to_f32(kv[l, 1, :, :pos + 1])
        o_ref = gqa_attention(q.astype(np.float64), K.astype(np.float64), V.astype(np.float64),
                              dt=np.float64).reshape(-1)
        o = dec.read_exchange(l, "attn")
        _close_bf16(o, o_ref, 1e-4 * np.abs(V).max(), (l, "attention"))
        # O-projection + residual
        x_o = dec.read_exchange(l, "x_o")
        r = pick(H)
        ref, bound = _gemv(W.rows(l, "o", r), o)
        _close_fp32(x_o[r], x_prev[r] + ref, bound + np.abs(x_prev[r]), (l, "o_proj"))
        # gate/up + SwiGLU on the normalised residual
        xn2 = bf16_round(rmsnorm(x_o, W.gain(l, "post_norm"), eps))
        h = dec.read_exchange(l, "h")
        r = pick(I)
        g, gb = _gemv(W.rows(l, "gate", r), xn2)
        u, ub = _gemv(W.rows(l, "up", r), xn2)
        sg = silu(g, np.float64)
        slack = 1.1 * np.abs(u) * GEMV_REL * gb + np.abs(sg) * GEMV_REL * ub
        _close_bf16(h[r], sg * u, slack, (l, "swiglu"))
        # down + residual
        x_d = dec.read_exchange(l, "x_d")
        r = pick(H)
        ref, bound = _gemv(W.rows(l, "down", r), h)
        _close_fp32(x_d[r], x_o[r] + ref, bound + np.abs(x_o[r]), (l, "down"))
    # final norm + tied LM head on the last residual
    L = sh.n_layers
    xf = bf16_round(rmsnorm(dec.read_exchange(L - 1, "x_d"), W.gain(0, "final_norm"), eps))
    r = pick(sh.vocab)
    r = np.unique(np.concatenate([r, [argmax_lowest(logits)]]))
    ref, bound = _gemv(W.rows(0, "embed", r), xf)
    _close_fp32(logits[r], ref, bound, "lm_head")
