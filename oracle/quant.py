"""Weight quantizers (oracle; test infrastructure only).

Both follow the monolith project page, "Design decisions":
  * FP8 format: E4M3 weights, one fp32 scale per output row, symmetric,
    round to nearest.  The scale is the row's absolute maximum over 448, the
    largest finite E4M3 magnitude, so the largest weight of every row lands
    on the top code.
  * NVFP4 format: E2M1 values, one E4M3 scale per 16 consecutive weights of
    a row, and one fp32 scale per tensor, round to nearest, plus a per-block
    scale search that minimizes the squared error.  The page fixes neither the
    candidate set nor the error sum; the reading taken: the candidates are the
    E4M3 scale codes within +-k of the absolute-maximum recipe's code (k = 0
    is that recipe alone), the error of a candidate is the sum over the
    block's 16 weights of (w - w_hat)^2, each term and the running sum in
    float64 in index order, and the smallest error wins, ties to the smaller
    code.

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


def _fp4_codes(blocks: np.ndarray, eff: np.ndarray) -> np.ndarray:
    """e2m1(fl32(w / eff)) per weight; every code 0 where eff = 0."""
    safe = np.where(eff == 0, F32(1.0), eff).astype(F32)
    c = e2m1_encode((blocks / safe[..., None]).astype(F32))
    return np.where((eff == 0)[..., None], np.uint8(0), c).astype(np.uint8)


def fp4_block_sq_error(blocks: np.ndarray, eff: np.ndarray) -> np.ndarray:
    """Squared error of each 16-wide block stored with effective scale eff:
    sum_i (w_i - w_hat_i)^2 with w_hat_i = fl32(e2m1(c_i) * eff), each
    difference, square and partial sum a float64 operation, i = 0..15 in
    order."""
    q = (e2m1_decode(_fp4_codes(blocks, eff)) * eff[..., None]).astype(F32)
    err = np.zeros(blocks.shape[:-1], np.float64)
    for i in range(blocks.shape[-1]):
        d = blocks[..., i].astype(np.float64) - q[..., i].astype(np.float64)
        err = err + d * d
    return err


def quant_fp4(w: np.ndarray, search: int = 0) -> Fp4Block:
    """Per tensor: A = max |w|; ts = fl32(A / 2688) (2688 = 6 * 448), or 1 when
    A = 0.  Per row and 16-wide block: a_b = max |w_block|;
    b0 = e4m3(fl32(a_b / fl32(6 * ts))), the absolute-maximum scale code.
    With search = k > 0 the block's scale code bs is the code in
    [b0 - k, b0 + k] (within 0..0x7E, the finite non-negative codes) whose
    fp4_block_sq_error is least, the smaller code on a tie; with k = 0,
    bs = b0.  Then eff = fl32(e4m3(bs) * ts) and c = e2m1(fl32(w / eff)), or
    code 0 for the whole block when eff = 0."""
    w = np.asarray(w, dtype=F32)
    n, k = w.shape
    if k % 16:
        raise ValueError("NVFP4 needs the input dimension to be a multiple of 16")
    if not 0 <= search <= 0x7E:
        raise ValueError("the scale search radius is 0..126")
    big_a = F32(np.max(np.abs(w))) if w.size else F32(0)
    ts = F32(big_a / F32(E2M1_MAX * E4M3_MAX)) if big_a != 0 else F32(1.0)
    blocks = w.reshape(n, k // 16, 16)
    a_b = np.max(np.abs(blocks), axis=2)
    six_ts = F32(F32(E2M1_MAX) * ts)
    bs = e4m3_encode((a_b / six_ts).astype(F32)).astype(np.int64)   # a_b >= 0: sign bit 0
    if search:
        best, best_err = bs.copy(), np.full(bs.shape, np.inf)
        for off in range(-search, search + 1):          # ascending codes: a tie keeps the smaller
            cand = bs + off
            ok = (cand >= 0) & (cand <= 0x7E)
            cc = np.clip(cand, 0, 0x7E)
            err = fp4_block_sq_error(blocks, (e4m3_decode(cc) * ts).astype(F32))
            take = ok & (err < best_err)
            best = np.where(take, cand, best)
            best_err = np.where(take, err, best_err)
        bs = best
    eff = (e4m3_decode(bs) * ts).astype(F32)
    c = _fp4_codes(blocks, eff).reshape(n, k)
    packed = (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)
    return Fp4Block(packed, bs.astype(np.uint8), ts)
