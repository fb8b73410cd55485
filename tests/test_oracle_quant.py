"""Pins for the oracle's FP8 per-row and NVFP4 quantizers (with and without
the NVFP4 block scale search): hand-worked examples, invariants that follow
from the recipe, an exhaustive search, and error bounds (no GPU)."""
from fractions import Fraction

import numpy as np
import pytest

from oracle.codecs import e2m1_decode, e2m1_encode, e4m3_decode
from oracle.quant import Fp4Block, fp4_block_sq_error, quant_fp4, quant_fp8_row


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


# -------------------------------------------------- NVFP4 block scale search
def _search_fixture():
    """Row 0: a block holding the tensor maximum 2.625 (so ts = 2.625/2688 =
    2^-10 exactly) and a block of u * [1.0 x 15, 1.25 at index 5], u = 2^-7."""
    w = np.zeros((1, 32), np.float32)
    w[0, 0] = 2.625
    w[0, 16:] = 2.0 ** -7
    w[0, 21] = 1.25 * 2.0 ** -7
    return w


@pytest.mark.parametrize("k,code,err_1024", [
    (0, 0x3D, None),   # a_b/(6 ts) = 5/3 -> e4m3 1.625
    (1, 0x3E, 244),    # 1.5: 256, 1.625: 541, 1.75: 240 + 4 = 244
    (2, 0x3B, 64),     # 1.375: 15 * 1 + 49 = 64 (1.875: 60 + 25 = 85)
    (3, 0x3B, 64),     # 2.0 also gives 64 (exact 4s, the 5 ties down to 4): the smaller code wins
    (6, 0x43, 31),     # 2.75: 15 * 1 (8/2.75 -> 3) + 16 (10/2.75 -> 4)
])
def test_fp4_search_hand_worked_block(k, code, err_1024):
    """Hand-worked block (errors in units of u^2 / 1024): the scale code the
    search picks at each radius, and its squared error."""
    p = quant_fp4(_search_fixture(), k)
    assert p.tensor_scale == np.float32(2.0 ** -10)
    assert p.block_scales[0, 0] == 0x7E
    assert p.block_scales[0, 1] == code
    if err_1024 is not None:
        blk = _search_fixture()[:, 16:].reshape(1, 1, 16)
        eff = (e4m3_decode(np.array([[code]])) * np.float32(2.0 ** -10)).astype(np.float32)
        assert fp4_block_sq_error(blk, eff)[0, 0] == err_1024 / 1024 * 2.0 ** -14
        wh = p.dequant()[0, 16:].astype(np.float64)
        assert np.sum((wh - _search_fixture()[0, 16:]) ** 2) == err_1024 / 1024 * 2.0 ** -14


def _block_errors_brute(w, p):
    """Squared error of every block of a packed tensor from its dequantization
    (numpy's own float64 sum)."""
    n, k = w.shape
    d = (p.dequant().astype(np.float64) - w.astype(np.float64)).reshape(n, k // 16, 16)
    return np.sum(d * d, axis=2)


def test_fp4_search_is_the_exhaustive_minimum():
    """With the radius covering every code, each block's scale is the global
    minimizer found by trying all 127 finite codes one by one (a uniform code
    planted in every block, error from the dequantized tensor)."""
    w = _rand((6, 128), 31)
    w[2] *= 1e-3                                      # small blocks: subnormal scale codes
    p = quant_fp4(w, 0x7E)
    n, k = w.shape
    blocks = w.reshape(n, k // 16, 16)
    errs = np.empty((0x7F,) + blocks.shape[:2])
    for c in range(0x7F):
        bs = np.full(blocks.shape[:2], c, np.uint8)
        eff = (e4m3_decode(bs) * p.tensor_scale).astype(np.float32)
        codes = np.zeros(blocks.shape, np.uint8)
        for r in range(n):
            for b in range(k // 16):
                if eff[r, b] != 0:
                    codes[r, b] = e2m1_encode((blocks[r, b] / eff[r, b]).astype(np.float32))
        flat = codes.reshape(n, k)
        trial = Fp4Block((flat[:, 0::2] | (flat[:, 1::2] << 4)).astype(np.uint8), bs, p.tensor_scale)
        errs[c] = _block_errors_brute(w, trial)
    best = errs.min(axis=0)
    got = np.take_along_axis(errs, p.block_scales.astype(np.int64)[None], 0)[0]
    assert np.all(got <= best * (1 + 1e-12))
    # where the minimum is clear of the runner-up, the code itself
    srt = np.sort(errs, axis=0)
    clear = srt[1] > srt[0] * (1 + 1e-9)
    assert clear.sum() > 0.8 * clear.size
    assert np.array_equal(p.block_scales[clear], errs.argmin(axis=0)[clear])


def test_fp4_search_never_worse_and_nested():
    """The candidate sets grow with the radius, so each block's error never
    increases with it; radius 0 is the absolute-maximum recipe."""
    w = _rand((64, 256), 32)
    base = quant_fp4(w)
    assert np.array_equal(quant_fp4(w, 0).block_scales, base.block_scales)
    prev = _block_errors_brute(w, base)
    for k in (1, 2, 4, 8):
        p = quant_fp4(w, k)
        assert p.tensor_scale == base.tensor_scale
        e = _block_errors_brute(w, p)
        assert np.all(e <= prev * (1 + 1e-12))
        assert np.all(np.abs(p.block_scales.astype(int) - base.block_scales.astype(int)) <= k)
        prev = e
    assert prev.sum() < 0.95 * _block_errors_brute(w, base).sum()


def test_fp4_search_sign_and_power_of_two_scaling():
    """Negating the tensor flips only the code sign bits; scaling it by 2^j
    scales ts by 2^j and keeps every code (all quotients are unchanged)."""
    w = _rand((8, 64), 33)
    p = quant_fp4(w, 4)
    n = quant_fp4(-w, 4)
    assert np.array_equal(n.block_scales, p.block_scales)
    assert np.all(w != 0)
    assert np.array_equal(n.unpacked_codes(), p.unpacked_codes() ^ 8)
    s = quant_fp4((w * np.float32(8.0)).astype(np.float32), 4)
    assert s.tensor_scale == p.tensor_scale * 8
    assert np.array_equal(s.codes, p.codes) and np.array_equal(s.block_scales, p.block_scales)


def test_fp4_search_radius_bounds():
    with pytest.raises(ValueError):
        quant_fp4(np.zeros((1, 16), np.float32), 127)
    z = quant_fp4(np.zeros((2, 32), np.float32), 5)
    assert np.all(z.block_scales == 0) and np.all(z.codes == 0)
