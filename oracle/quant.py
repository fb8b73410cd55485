"""Weight quantizers (oracle; test infrastructure only).

Both follow the monolith project page, "Design decisions":
  * FP8 format: E4M3 weights, one fp32 scale per output row, symmetric,
    round to nearest.  The scale is the row's absolute maximum over 448, the
    largest finite E4M3 magnitude, so the largest weight of every row lands
    on the top code.
  * NVFP4 format: E2M1 values, one E4M3 scale per 16 consecutive weights of
    a row, and one fp32 scale per tensor, round to nearest.  The page also
    names a per-block MSE scale search; the plain absolute-maximum recipe is
    taken here (the search is a later refinement).

Every arithmetic step is a single float32 operation (division, product),
written out so that another implementation can reproduce the bytes exactly.

Canonical packed forms (row-major, un-tiled):
  FP8 : codes uint8 [N, K]; scales float32 [N]
  FP4 : codes uint8 [N, K/2], element 2j in the low nibble of byte j;
        block scales uint8 [N, K/16] (E4M3, sign 0); tensor scale float32
"""
from __future__ import annotations

import dataclasses

import numpy as np

from .codecs import (E2M1_MAX, E4M3_MAX, e2m1_decode, e2m1_encode,
                     e4m3_decode, e4m3_encode)

F32 = np.float32


@dataclasses.dataclass
class Fp8Row:
    codes: np.ndarray      # uint8 [N, K]
    scales: np.ndarray     # float32 [N]

    def dequant(self) -> np.ndarray:
        """w_hat = fl32(e4m3(c) * s_r)."""
        return (e4m3_decode(self.codes) * self.scales[:, None]).astype(F32)


@dataclasses.dataclass
class Fp4Block:
    codes: np.ndarray          # uint8 [N, K/2] packed nibbles
    block_scales: np.ndarray   # uint8 [N, K/16]
    tensor_scale: np.float32

    def unpacked_codes(self) -> np.ndarray:
        lo = self.codes & 0x0F
        hi = self.codes >> 4
        return np.stack([lo, hi], axis=-1).reshape(self.codes.shape[0], -1)

    def effective_scales(self) -> np.ndarray:
        """eff = fl32(e4m3(bs) * ts), float32 [N, K/16]."""
        return (e4m3_decode(self.block_scales) * F32(self.tensor_scale)).astype(F32)

    def dequant(self) -> np.ndarray:
        """w_hat = fl32(e2m1(c) * eff)."""
        eff = np.repeat(self.effective_scales(), 16, axis=1)
        return (e2m1_decode(self.unpacked_codes()) * eff).astype(F32)


def quant_fp8_row(w: np.ndarray) -> Fp8Row:
    """Per output row r: a = max |w[r, :]|; s = fl32(a / 448), or 1 when a = 0;
    c = e4m3(fl32(w / s))."""
    w = np.asarray(w, dtype=F32)
    a = np.max(np.abs(w), axis=1)
    s = (a / F32(E4M3_MAX)).astype(F32)
    s = np.where(a == 0, F32(1.0), s).astype(F32)
    q = (w / s[:, None]).astype(F32)
    return Fp8Row(e4m3_encode(q), s)


def quant_fp4(w: np.ndarray) -> Fp4Block:
    """Per tensor: A = max |w|; ts = fl32(A / 2688) (2688 = 6 * 448), or 1 when
    A = 0.  Per row and 16-wide block: a_b = max |w_block|;
    bs = e4m3(fl32(a_b / fl32(6 * ts))); eff = fl32(e4m3(bs) * ts);
    c = e2m1(fl32(w / eff)), or code 0 for the whole block when eff = 0."""
    w = np.asarray(w, dtype=F32)
    n, k = w.shape
    if k % 16:
        raise ValueError("NVFP4 needs the input dimension to be a multiple of 16")
    big_a = F32(np.max(np.abs(w))) if w.size else F32(0)
    ts = F32(big_a / F32(E2M1_MAX * E4M3_MAX)) if big_a != 0 else F32(1.0)
    blocks = w.reshape(n, k // 16, 16)
    a_b = np.max(np.abs(blocks), axis=2)
    six_ts = F32(F32(E2M1_MAX) * ts)
    bs = e4m3_encode((a_b / six_ts).astype(F32))   # a_b >= 0, so the sign bit is 0
    eff = (e4m3_decode(bs) * ts).astype(F32)
    safe = np.where(eff == 0, F32(1.0), eff).astype(F32)
    q = (blocks / safe[:, :, None]).astype(F32)
    c = e2m1_encode(q).reshape(n, k // 16, 16)
    c = np.where((eff == 0)[:, :, None], np.uint8(0), c).astype(np.uint8)
    c = c.reshape(n, k)
    packed = (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)
    return Fp4Block(packed, bs.astype(np.uint8), ts)
