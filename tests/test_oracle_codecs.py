"""Pins for the oracle's number formats, against the format definitions,
brute force and library casts (no GPU)."""
import os

import numpy as np
import pytest
import torch

from oracle.codecs import (bf16_bits_to_f32, bf16_round, e2m1_decode,
                           e2m1_encode, e4m3_decode, e4m3_encode,
                           f32_to_bf16_bits)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f32(bits):
    return np.asarray(bits, dtype=np.uint32).view(np.float32)


# ------------------------------------------------------------------ bf16
def test_bf16_matches_torch_cast():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(200_000) * np.exp2(rng.integers(-60, 60, 200_000))).astype(np.float32)
    # exact halfway cases, both parities of the kept bit, and their neighbours
    hi = rng.integers(0, 1 << 15, 5000).astype(np.uint32) << 16
    ties = np.concatenate([hi | 0x8000, hi | 0x18000, hi | 0x7FFF, hi | 0x8001]).astype(np.uint32)
    x = np.concatenate([x, _f32(ties), np.array([0.0, -0.0, 1.0, -3.5], np.float32)])
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f32_to_bf16_bits(x), ref)


def test_bf16_exact_roundtrip_and_ties():
    assert bf16_bits_to_f32(np.array([0x3F80], np.uint16))[0] == 1.0
    assert bf16_bits_to_f32(np.array([0xC040], np.uint16))[0] == -3.0
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to even -> 1
    assert bf16_round(np.array([1.0 + 2.0 ** -8], np.float32))[0] == 1.0
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even)
    assert bf16_round(np.array([1.0 + 3 * 2.0 ** -8], np.float32))[0] == 1.0 + 2.0 ** -6
    with pytest.raises(ValueError):
        f32_to_bf16_bits(np.array([np.nan], np.float32))


# ------------------------------------------------------------------ e4m3
def _e4m3_closed_form(c: int) -> float:
    s = -1.0 if c & 0x80 else 1.0
    e, m = (c >> 3) & 0xF, c & 7
    if e == 0xF and m == 7:
        return float("nan")
    if e == 0:
        return s * m * 2.0 ** -9
    return s * 2.0 ** (e - 7) * (1 + m / 8)


def test_e4m3_decode_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    got = e4m3_decode(codes).astype(np.float64)
    ref = np.array([_e4m3_closed_form(int(c)) for c in codes])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])
    # library decode of the same bytes
    lib = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(lib), np.isnan(got))
    assert np.array_equal(lib[fin], got[fin])
    # spot values and structure
    assert got[0x38] == 1.0 and got[0x40] == 2.0 and got[0x7E] == 448.0
    assert got[0x08] == 2.0 ** -6 and got[0x01] == 2.0 ** -9
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF])
    assert int(fin.sum()) == 254
    assert np.all(np.diff(got[:0x7F]) > 0)


def _brute_encode(x, grid_codes, grid_vals, max_code, sign_bit):
    """Nearest finite value by exhaustive search; ties to the even code;
    saturation beyond the largest magnitude; sign kept."""
    out = np.empty(len(x), dtype=np.uint8)
    for i, v in enumerate(np.asarray(x, np.float64)):
        a = abs(v)
        d = np.abs(grid_vals - a)
        best = np.flatnonzero(d == d.min())
        if len(best) > 1:
            best = [b for b in best if grid_codes[b] % 2 == 0]
        c = int(grid_codes[best[0]])
        if a >= grid_vals[-1]:
            c = max_code
        out[i] = c | (sign_bit if np.signbit(v) else 0)
    return out


def _probe_points(grid: np.ndarray, rng, n_random: int, hi: float) -> np.ndarray:
    mids = (grid[1:] + grid[:-1]) / 2
    pts = np.concatenate([grid, mids]).astype(np.float32)
    nb = np.concatenate([np.nextafter(pts, np.float32(np.inf)), np.nextafter(pts, np.float32(0))])
    rnd = (rng.random(n_random) * hi).astype(np.float32)
    tiny = (rng.random(200) * grid[1] * 2).astype(np.float32)
    big = np.array([hi, hi * 1.01, hi * 10, 1e30, 3.4e38], np.float32)
    pos = np.concatenate([pts, nb, rnd, tiny, big, [0.0]]).astype(np.float32)
    return np.concatenate([pos, -pos]).astype(np.float32)


def test_e4m3_encode_brute_force():
    rng = np.random.default_rng(5)
    codes = np.arange(0x7F)
    vals = e4m3_decode(codes.astype(np.uint8)).astype(np.float64)
    x = _probe_points(vals, rng, 20000, 448.0)
    got = e4m3_encode(x)
    ref = _brute_encode(x, codes, vals, 0x7E, 0x80)
    assert np.array_equal(got, ref)


def test_e4m3_encode_matches_torch_below_464():
    rng = np.random.default_rng(6)
    x = (rng.standard_normal(100_000) * np.exp2(rng.integers(-12, 9, 100_000))).astype(np.float32)
    x = x[np.abs(x) < 464]
    lib = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3_encode(x), lib)
    assert e4m3_encode(np.array([1.0625], np.float32))[0] == 0x38
    assert e4m3_encode(np.array([2.0 ** -10], np.float32))[0] == 0x00
    assert e4m3_encode(np.array([-2.0 ** -10], np.float32))[0] == 0x80
    assert e4m3_encode(np.array([1000.0, -1e9], np.float32)).tolist() == [0x7E, 0xFE]


# ------------------------------------------------------------------ e2m1
def _golden_grid():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "e2m1_grid.txt"))
            if l.strip() and not l.startswith("#")]
    return np.array([int(r[0]) for r in rows]), np.array([float(r[1]) for r in rows])


def test_e2m1_decode_matches_printed_grid():
    codes, vals = _golden_grid()
    got = e2m1_decode(codes.astype(np.uint8)).astype(np.float64)
    assert np.array_equal(got, vals)
    assert np.array_equal(np.signbit(got), np.signbit(vals))


def test_e2m1_encode_brute_force_and_ties():
    codes, vals = _golden_grid()
    rng = np.random.default_rng(7)
    x = _probe_points(vals[:8], rng, 5000, 6.0)
    assert np.array_equal(e2m1_encode(x), _brute_encode(x, codes[:8], vals[:8], 7, 8))
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    assert e2m1_decode(e2m1_encode(ties)).tolist() == [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0]
    assert e2m1_encode(np.array([7.0, -100.0], np.float32)).tolist() == [7, 15]
