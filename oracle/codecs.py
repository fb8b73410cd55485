"""Number formats on the decode path (oracle; test infrastructure only).

* bfloat16: the upper 16 bits of an IEEE binary32, rounded to nearest even.
  Activations entering each GEMV, the KV cache and the bf16 weights use it
  (monolith page, "Design decisions": FP8 format, activations stay bf16;
  KV cache stays bf16).
* e4m3: the OCP E4M3FN byte (1 sign, 4 exponent bits with bias 7, 3 mantissa
  bits, no infinities, S.1111.111 is NaN, largest finite 448).  Used for FP8
  weights and for the NVFP4 block scales (monolith page, "Design decisions").
* e2m1: 1 sign, 2 exponent bits with bias 1, 1 mantissa bit; the magnitudes
  are {0, 0.5, 1, 1.5, 2, 3, 4, 6} (TSCT super-kernel note, section 3b).

Encoding is round to nearest, ties to even, with saturation to the largest
finite magnitude (the pages ask for "round to nearest"; saturation is the
reading taken for out-of-range inputs).  The sign of the input is kept, so a
negative value that rounds to zero encodes as negative zero.
"""
from __future__ import annotations

import numpy as np


# ----------------------------------------------------------------- bfloat16
def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even.  NaN is not
    expected on this path and is rejected."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if np.isnan(x).any():
        raise ValueError("NaN reached a bf16 rounding point")
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 value, returned as float32."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


# ------------------------------------------------------ generic minifloats
class MiniFloat:
    """A sign-magnitude binary float with `ebits` exponent bits, `mbits`
    mantissa bits and exponent bias `bias`.  Exponent field 0 holds the
    subnormals; `max_code` is the largest finite magnitude code."""

    def __init__(self, ebits: int, mbits: int, bias: int, max_code: int):
        self.ebits, self.mbits, self.bias, self.max_code = ebits, mbits, bias, max_code
        self.sign_bit = 1 << (ebits + mbits)

    def decode(self, codes: np.ndarray) -> np.ndarray:
        """Codes -> float32 values (exact).  Magnitude codes above max_code
        decode to NaN."""
        c = np.asarray(codes).astype(np.int64)
        mag = c & (self.sign_bit - 1)
        e = mag >> self.mbits
        m = mag & ((1 << self.mbits) - 1)
        frac = m.astype(np.float64) / float(1 << self.mbits)
        # exponent field 0: (m / 2^mbits) * 2^(1 - bias); else (1 + m/2^mbits) * 2^(e - bias)
        val = np.where(e == 0, frac * 2.0 ** (1 - self.bias),
                       (1.0 + frac) * np.exp2((e - self.bias).astype(np.float64)))
        val = np.where(mag > self.max_code, np.nan, val)
        val = np.where((c & self.sign_bit) != 0, -val, val)
        return val.astype(np.float32)

    def encode(self, x: np.ndarray) -> np.ndarray:
        """float32 -> codes: round to nearest, ties to the even code, magnitudes
        beyond the largest finite value saturate to it."""
        x = np.asarray(x, dtype=np.float32)
        if np.isnan(x).any():
            raise ValueError("NaN cannot be encoded")
        ax = np.abs(x).astype(np.float64)
        neg = np.signbit(x)
        max_val = float(self.decode(np.array([self.max_code]))[0])
        emin = 1 - self.bias                       # exponent of the smallest normal
        with np.errstate(divide="ignore"):
            e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
        e = np.maximum(e, emin)                    # subnormals share the emin quantum
        quantum = np.exp2(e - self.mbits)
        q = np.rint(ax / quantum)                  # exact scaling; rint ties to even
        # code = (biased exponent field of e) * 2^mbits + (q - 2^mbits); for a
        # subnormal the same formula gives q directly, and q == 2^(mbits+1)
        # (rounding up into the next binade) lands on the next exponent field.
        field = np.where(ax < 2.0 ** emin, 0.0, e + self.bias)
        code = np.where(ax < 2.0 ** emin, q, field * (1 << self.mbits) + q - (1 << self.mbits))
        code = np.where(ax >= max_val, self.max_code, code).astype(np.int64)
        code = np.minimum(code, self.max_code)
        code = np.where(neg, code | self.sign_bit, code)
        return code.astype(np.uint8)


E4M3 = MiniFloat(ebits=4, mbits=3, bias=7, max_code=0x7E)
E2M1 = MiniFloat(ebits=2, mbits=1, bias=1, max_code=0x7)

E4M3_MAX = 448.0
E2M1_MAX = 6.0


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    return E4M3.decode(codes)


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    return E4M3.encode(x)


def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    return E2M1.decode(np.asarray(codes) & 0xF)


def e2m1_encode(x: np.ndarray) -> np.ndarray:
    return E2M1.encode(x)
