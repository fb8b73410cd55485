"""Pins for the oracle's FP8 per-row and NVFP4 quantizers: hand-worked
examples, invariants that follow from the recipe, and error bounds (no GPU)."""
from fractions import Fraction

import numpy as np

from oracle.codecs import e2m1_decode, e4m3_decode
from oracle.quant import quant_fp4, quant_fp8_row


def _is_rounded_quotient(q, num, den) -> bool:
    """q is the float32 nearest to the real num / den (exact rationals)."""
    exact = Fraction(float(num)) / Fraction(float(den))
    qf = np.float32(q)
    up, dn = np.nextafter(qf, np.float32(np.inf)), np.nextafter(qf, np.float32(-np.inf))
    d = abs(Fraction(float(qf)) - exact)
    return d <= abs(Fraction(float(up)) - exact) and d <= abs(Fraction(float(dn)) - exact)


def _rand(shape, seed):
    return (np.random.default_rng(seed).standard_normal(shape) * 0.02).astype(np.float32)


# ------------------------------------------------------------------ FP8
def test_fp8_hand_worked_rows():
    w = np.array([[448.0, 1.0, -0.5, 100.0],   # s = 1; 100 is a tie between 96 and 104 -> 96
                  [0.0, 0.0, 0.0, 0.0],        # zero row: s = 1, codes 0
                  [2.0, -4.0, 1.0, 0.0]],      # s = 4/448; 2 -> ~224, 1 -> ~112
                 np.float32)
    p = quant_fp8_row(w)
    assert p.codes.tolist() == [[0x7E, 0x38, 0xB0, 0x6C], [0, 0, 0, 0], [0x76, 0xFE, 0x6E, 0x00]]
    assert p.scales[0] == 1.0 and p.scales[1] == 1.0
    assert _is_rounded_quotient(p.scales[2], 4.0, 448.0)
    # a row maximum of 3 is where a rounded reciprocal would differ
    assert _is_rounded_quotient(quant_fp8_row(np.array([[3.0, -1.0]], np.float32)).scales[0], 3.0, 448.0)


def test_fp8_row_invariants_and_error_bound():
    w = _rand((257, 384), 11)
    w[5] = 0.0
    p = quant_fp8_row(w)
    mag = p.codes & 0x7F
    nz = np.any(w != 0, axis=1)
    # the largest weight of every nonzero row lands on the top code 448
    assert np.all(mag[nz].max(axis=1) == 0x7E)
    assert np.all(p.codes[~nz] == 0) and np.all(p.scales[~nz] == 1.0)
    assert np.all(p.scales[nz] > 0)
    amax = np.abs(w).max(axis=1)
    assert all(_is_rounded_quotient(p.scales[r], amax[r], 448.0) for r in np.flatnonzero(nz))
    wh = p.dequant().astype(np.float64)
    s = p.scales.astype(np.float64)[:, None]
    bound = (2.0 ** -4 * np.abs(w) + 2.0 ** -10 * s) * (1 + 2.0 ** -20)
    assert np.all(np.abs(w - wh) <= bound)
    # signs survive (a weight never changes sign; tiny ones may become +-0)
    assert np.all(np.sign(wh) * np.sign(w) >= 0)
    assert np.array_equal(wh, (e4m3_decode(p.codes) * p.scales[:, None]).astype(np.float32))


# ------------------------------------------------------------------ FP4
def test_fp4_hand_worked_blocks():
    g = [6, 3, -1.5, 0.5, 0, 0.25, 0.75, 1.25, -6, 2, 4, 3.5, 1.75, 2.5, 5, 1]
    w = np.zeros((2, 32), np.float32)
    w[0, :16] = np.array(g, np.float32) * 448.0   # tensor max 2688 -> ts = 1, bs = 448
    w[0, 16] = 7.0                                 # a_b = 7 -> bs = e4m3(7/6) = 1.125
    w[1, 16:] = -0.001                             # bs rounds to 0 -> eff 0 -> codes 0
    p = quant_fp4(w)
    assert p.tensor_scale == 1.0
    assert p.block_scales.tolist() == [[0x7E, 0x39], [0x00, 0x00]]
    assert p.codes[0, :8].tolist() == [0x57, 0x1B, 0x00, 0x22, 0x4F, 0x66, 0x44, 0x26]
    assert p.codes[0, 8:].tolist() == [0x07, 0, 0, 0, 0, 0, 0, 0]
    assert np.all(p.codes[1] == 0)
    wh = p.dequant()
    assert wh[0, 16] == 6.0 * 1.125
    assert np.array_equal(wh[0, :16], e2m1_decode(np.array(
        [7, 5, 11, 1, 0, 0, 2, 2, 15, 4, 6, 6, 4, 4, 6, 2])) * 448.0)


def test_fp4_invariants_and_error_bound():
    w = _rand((96, 512), 12)
    w[3, 32:48] = 0.0                # one zero block
    w[7] *= 1e-4                     # a row of tiny blocks
    p = quant_fp4(w)
    amax = np.max(np.abs(w))
    assert _is_rounded_quotient(p.tensor_scale, amax, 2688.0)
    blocks = np.abs(w).reshape(96, 32, 16).max(axis=2)
    r, b = np.unravel_index(np.argmax(blocks), blocks.shape)
    assert p.block_scales[r, b] == 0x7E            # the block holding the tensor max
    assert np.all(p.block_scales < 0x80)
    codes = p.unpacked_codes().reshape(96, 32, 16)
    normal = p.block_scales >= 0x08                # normal e4m3 scale
    assert np.all((codes[normal] & 7).max(axis=1) == 7)
    eff = np.repeat(p.effective_scales(), 16, axis=1).astype(np.float64)
    assert np.all(np.abs(w - p.dequant()) <= eff * (1 + 2.0 ** -20) + (eff == 0) * np.abs(w))
    assert p.block_scales[3, 2] == 0 and np.all(codes[3, 2] == 0)


def test_fp4_zero_tensor_and_nibble_order():
    p = quant_fp4(np.zeros((2, 16), np.float32))
    assert p.tensor_scale == 1.0 and np.all(p.codes == 0) and np.all(p.block_scales == 0)
    w = np.zeros((1, 16), np.float32)
    w[0, 0], w[0, 1] = 2688.0, -448.0               # element 0 low nibble, element 1 high
    assert quant_fp4(w).codes[0, 0] == (0x7 | (0xA << 4))
