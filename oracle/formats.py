"""Exact decoding of the storage formats the library consumes (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

* bfloat16: the upper 16 bits of an IEEE-754 binary32.  Decoding places the 16
  bits in the high half of a 32-bit word and reads it as binary32, which is
  exact, then widens to float64 (also exact).
* OCP FP8 E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa
  bits.  Exponent field 0 encodes subnormals (-1)^s * 2^-6 * m/8; other
  exponent fields encode (-1)^s * 2^(e-7) * (1 + m/8).  There are no
  infinities; the two codes S.1111.111 (0x7F, 0xFF) are NaN, so the largest
  finite magnitude is 1.75 * 2^8 = 448.  The pages only say "fp8" at one byte
  per parameter (shard planner, "The Shard Planner" section of the
  scalablesystem.dev page); the OCP E4M3 variant is the reading used here.

* int8 weight codes: two's complement, the byte b read as b for b < 128 and
  b - 256 otherwise (the planner's "int8" at one byte per parameter on the
  same page).

The e4m3 table is built from that definition with a direct loop over the 256
codes; it does not use any library fp8 type.
"""

import numpy as np

E4M3FN_MAX = 448.0


def bf16_bits_to_f64(bits):
    """Decode an array of bf16 bit patterns (uint16) to float64, exactly."""
    b = np.asarray(bits)
    if b.dtype != np.uint16:
        raise TypeError("bf16 storage must be uint16 bit patterns")
    u32 = b.astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):   # NaN payloads widen to NaN
        return u32.view(np.float32).astype(np.float64)


def _e4m3fn_value(code):
    sign = -1.0 if (code >> 7) & 1 else 1.0
    exp_field = (code >> 3) & 0xF
    mant = code & 0x7
    if exp_field == 0xF and mant == 0x7:
        return float("nan")
    if exp_field == 0:
        return sign * (2.0 ** -6) * (mant / 8.0)
    return sign * (2.0 ** (exp_field - 7)) * (1.0 + mant / 8.0)


_E4M3FN_TABLE = np.array([_e4m3fn_value(c) for c in range(256)], dtype=np.float64)


def e4m3fn_table():
    """The 256 code values, index = code (a copy)."""
    return _E4M3FN_TABLE.copy()


def int8_to_f64(codes):
    """Decode an array of int8 codes stored as uint8 bytes to float64."""
    c = np.asarray(codes)
    if c.dtype != np.uint8:
        raise TypeError("int8 storage must be uint8 bytes")
    v = c.astype(np.int64)
    return np.where(v >= 128, v - 256, v).astype(np.float64)


def e4m3fn_encode(v):
    """float32 values -> e4m3fn codes (uint8): the nearest finite code, ties to
    the even code (even mantissa), magnitudes of 448 and above saturating to
    448 (code 0x7E), the sign bit copied (so -0.0 -> 0x80).  Nearest is found
    by bisection in the increasing table of the non-negative codes 0x00-0x7E;
    every table value and midpoint is exact in float64."""
    v = np.asarray(v, dtype=np.float32)
    if np.isnan(v).any():
        raise ValueError("NaN has no code here")
    mags = _E4M3FN_TABLE[:0x7F]                      # codes 0x00 .. 0x7E, increasing
    a = np.abs(v.astype(np.float64))
    hi = np.clip(np.searchsorted(mags, a, side="left"), 1, 0x7E)   # mags[hi-1] < a <= mags[hi] (inside the range)
    lo = hi - 1
    dlo = a - mags[lo]
    dhi = mags[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a >= 448.0, 0x7E, code)
    code = np.where(a == 0.0, 0, code)
    sign = np.signbit(v).astype(np.int64) << 7
    return (code.astype(np.int64) | sign).astype(np.uint8)


def bf16_round_bits(v):
    """float32 values -> bf16 bit patterns (uint16), round to nearest even:
    the upper 16 bits of the binary32 word after adding half a bf16 unit
    (0x7FFF plus the kept low bit, for ties to even).  Finite inputs."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    u = v.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def e4m3fn_to_f64(codes):
    """Decode an array of e4m3fn codes (uint8) to float64, exactly."""
    c = np.asarray(codes)
    if c.dtype != np.uint8:
        raise TypeError("e4m3fn storage must be uint8 codes")
    return _E4M3FN_TABLE[c]
