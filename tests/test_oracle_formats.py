"""Pins for the oracle's format decoders and the input module's encoders.

The decoders are checked against values printed in the format definitions
(tests/golden), against torch's own bf16 / float8_e4m3fn types (an independent
library implementation) and against structural properties.  The encoders in
``workloads`` (used only to make inputs) are checked against brute-force
nearest-value search over the oracle's decode table and against torch's
conversions.
"""

import math

import numpy as np
import pytest
import torch

from conftest import read_golden
import oracle
from oracle.formats import e4m3fn_table
import workloads


def test_bf16_golden_codes():
    for bits, val in read_golden("bf16_codes.txt"):
        got = oracle.bf16_bits_to_f64(np.array([int(bits, 16)], dtype=np.uint16))[0]
        want = float(val)
        assert got == want or (math.isnan(got) and math.isnan(want)), (bits, got, want)
        assert math.copysign(1.0, got) == math.copysign(1.0, want), bits


def test_bf16_matches_torch_for_all_codes():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.bf16_bits_to_f64(codes)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_e4m3fn_golden_codes():
    for code, val in read_golden("e4m3fn_codes.txt"):
        got = oracle.e4m3fn_to_f64(np.array([int(code, 16)], dtype=np.uint8))[0]
        want = float(val)
        if math.isnan(want):
            assert math.isnan(got), code
        else:
            assert got == want, (code, got, want)
            assert math.copysign(1.0, got) == math.copysign(1.0, want), code


def test_e4m3fn_matches_torch_for_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3fn_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2
    assert np.array_equal(ours[~nan], ref[~nan])


def test_e4m3fn_structure():
    tab = e4m3fn_table()
    pos = tab[:0x7F]
    assert np.all(np.diff(pos) > 0), "positive codes must be strictly increasing"
    assert pos[-1] == oracle.E4M3FN_MAX == 448.0
    # sign bit negates
    assert np.array_equal(tab[0x80:0xFF], -tab[:0x7F])
    # the subnormal step equals the first normal step (no gap at 2^-6)
    assert tab[0x08] - tab[0x07] == tab[0x01] == 2.0 ** -9


def test_bf16_encoder_matches_torch():
    w = workloads.draw_f32(12345, (1 << 16,), 3.0)
    w = np.concatenate([w, np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8),
                                     2.0 ** -130, 0.0, -0.0], dtype=np.float32)])
    ours = workloads.f32_to_bf16_bits(w)
    ref = torch.from_numpy(w).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    # ties go to even: 1 + 2^-8 is halfway between 1 and 1 + 2^-7
    assert ours[-6] == 0x3F80 and ours[-5] == 0x3F82


def test_e4m3fn_encoder_is_nearest_even():
    tab = e4m3fn_table()
    finite_codes = np.array([c for c in range(256) if not np.isnan(tab[c])], dtype=np.int64)
    vals = tab[finite_codes]
    rng = np.random.Generator(np.random.PCG64(7))
    x = np.concatenate([
        rng.uniform(-448, 448, 4000), rng.normal(0, 1, 4000), rng.normal(0, 0.01, 2000),
        # exact midpoints between neighbouring positive codes (ties)
        (tab[1:0x7F] + tab[0:0x7E]) / 2.0,
    ]).astype(np.float32)
    x = x[np.abs(x) <= 448]
    codes = workloads.f32_to_e4m3fn(x).astype(np.int64)
    for xi, ci in zip(x.astype(np.float64), codes):
        d = np.abs(vals - xi)
        best = d.min()
        cands = finite_codes[d == best]
        # among equally near values prefer the even mantissa; +0 / -0 by sign
        even = [c for c in cands if (c & 1) == 0]
        assert tab[ci] == tab[even[0]] if even else tab[cands[0]], (xi, ci, cands)
        assert abs(tab[ci] - xi) == best


def test_e4m3fn_encoder_matches_torch():
    rng = np.random.Generator(np.random.PCG64(8))
    x = np.clip(rng.normal(0, 100, 20000), -448, 448).astype(np.float32)
    ours = workloads.f32_to_e4m3fn(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_quantise_rows_roundtrip_bound():
    w = workloads.draw_f32(99, (64, 512), 0.02)
    q, s = workloads.quantise_rows_e4m3fn(w)
    assert q.dtype == np.uint8 and s.dtype == np.float32 and s.shape == (64,)
    deq = oracle.e4m3fn_to_f64(q) * s.astype(np.float64)[:, None]
    # each row's largest magnitude maps to +-448 exactly (up to the fp32 scale rounding)
    assert np.all(np.max(np.abs(oracle.e4m3fn_to_f64(q)), axis=1) >= 447.0)
    # e4m3 relative spacing is 2^-3, so the rounding error is at most 2^-4 relative
    # for normal codes and half a subnormal step (2^-10 * s) below 2^-6 * s.
    err = np.abs(deq - w.astype(np.float64))
    bound = np.maximum(np.abs(w.astype(np.float64)) * 2.0 ** -4, 2.0 ** -10 * s[:, None]) * (1 + 1e-6)
    assert np.all(err <= bound)
    # an all-zero row gets scale 1 and zero codes
    q0, s0 = workloads.quantise_rows_e4m3fn(np.zeros((2, 8), np.float32))
    assert np.all(s0 == 1.0) and np.all(oracle.e4m3fn_to_f64(q0) == 0.0)


# ----------------------------------------------------------------- int8

def test_int8_golden_codes():
    for code, want in read_golden("int8_codes.txt"):
        got = oracle.int8_to_f64(np.array([int(code, 16)], dtype=np.uint8))[0]
        assert got == float(want), code


def test_int8_matches_numpy_view_for_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    assert np.array_equal(oracle.int8_to_f64(codes), codes.view(np.int8).astype(np.float64))
    with pytest.raises(TypeError):
        oracle.int8_to_f64(codes.view(np.int8))


def test_int8_quantiser_is_nearest_even_and_symmetric():
    rng = np.random.Generator(np.random.PCG64(12))
    w = rng.normal(0, 0.02, (16, 300)).astype(np.float32)
    w[3, 7] = 0.0
    w[5] = 0.0                                   # all-zero row
    q, s = workloads.quantise_rows_int8(w)
    assert q.dtype == np.uint8 and s.dtype == np.float32
    v = oracle.int8_to_f64(q)
    assert np.all(np.abs(v) <= 127)
    assert s[5] == 1.0 and np.all(v[5] == 0)
    for r in range(16):
        if r == 5:
            continue
        # the row's largest magnitude maps to +-127
        assert np.max(np.abs(v[r])) == 127
        scaled = (w[r] / s[r]).astype(np.float32).astype(np.float64)
        for j in range(300):
            cands = np.arange(-127, 128, dtype=np.float64)
            d = np.abs(cands - scaled[j])
            best = cands[d == d.min()]
            want = best[0] if len(best) == 1 else best[(best % 2) == 0][0]
            assert v[r, j] == want, (r, j)
    # crafted ties: 0.5 -> 0, 1.5 -> 2, 2.5 -> 2, -2.5 -> -2 (scale 1 from amax 127)
    t = np.array([[127.0, 0.5, 1.5, 2.5, -2.5, -0.5]], np.float32)
    qt, st = workloads.quantise_rows_int8(t)
    assert st[0] == 1.0
    assert oracle.int8_to_f64(qt)[0].tolist() == [127.0, 0.0, 2.0, 2.0, -2.0, -0.0]


def test_int8_roundtrip_bound():
    w = workloads.draw_f32(98, (32, 512), 0.02)
    q, s = workloads.quantise_rows_int8(w)
    deq = oracle.int8_to_f64(q) * s.astype(np.float64)[:, None]
    err = np.abs(deq - w.astype(np.float64))
    assert np.all(err <= 0.5 * s[:, None].astype(np.float64) * (1 + 1e-6))
