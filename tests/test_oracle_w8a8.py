"""Pins for the oracle's W8A8 pieces (``oracle/w8a8.py`` and the encoders in
``oracle/formats.py``): the e4m3fn and bf16 encoders against brute force and
against torch's casts, the per-row quantiser against closed forms, and the
forward against a lossless closed form and a pure-Python re-derivation on a
tiny case."""

import itertools

import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle.formats import e4m3fn_table


def _brute_e4m3(x):
    """Nearest of the 255 finite codes by exhaustive search, ties to the even
    code, saturation at 448, sign copied."""
    tab = e4m3fn_table()
    out = []
    for v in np.asarray(x, dtype=np.float32).tolist():
        a = abs(v)
        if a >= 448.0:
            c = 0x7E
        else:
            best, bd = None, None
            for code in range(0x7F):
                d = abs(tab[code] - a)
                if bd is None or d < bd or (d == bd and code % 2 == 0):
                    best, bd = code, d
            c = best
        if np.signbit(np.float32(v)):
            c |= 0x80
        out.append(c)
    return np.array(out, dtype=np.uint8)


def test_e4m3_encoder_brute_force():
    rng = np.random.Generator(np.random.PCG64(21))
    x = np.concatenate([rng.normal(0, 30, 400), rng.normal(0, 0.01, 200), rng.uniform(-500, 500, 100)])
    tab = e4m3fn_table()[:0x7F]
    mids = (tab[:-1] + tab[1:]) / 2                       # every tie, both signs
    x = np.concatenate([x, mids, -mids, [0.0, -0.0, 448.0, -448.0, 1e30, -1e30, 464.0, 447.9]]).astype(np.float32)
    assert np.array_equal(oracle.e4m3fn_encode(x), _brute_e4m3(x))


def test_e4m3_encoder_matches_torch_in_range():
    rng = np.random.Generator(np.random.PCG64(22))
    x = np.clip(rng.normal(0, 60, 50000), -447, 447).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3fn_encode(x), ref)


def test_bf16_rounding_matches_torch():
    rng = np.random.Generator(np.random.PCG64(23))
    x = (rng.normal(0, 1, 20000) * 10.0 ** rng.integers(-20, 20, 20000)).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bf16_round_bits(x), ref)


def test_row_quantiser_closed_forms():
    # amax 448 * 2^e makes s = 2^e exactly; codes of x / s are then exact for code values
    tab = e4m3fn_table()
    codes = np.array([0x38, 0x7E, 0x01, 0xB8, 0x45, 0x00], dtype=np.uint8)      # 1, 448, 2^-9, -1, 3.25?, 0
    vals = tab[codes]
    for e in (-8, 0, 5):
        row = (vals * 2.0 ** e).astype(np.float32)[None, :]
        q, s = oracle.quantise_rows_e4m3(row)
        assert s[0] == np.float32(2.0 ** e)
        assert np.array_equal(q[0], codes)
    # an all-zero row (with a negative zero) keeps scale 1
    q, s = oracle.quantise_rows_e4m3(np.array([[0.0, -0.0, 0.0]], np.float32))
    assert s[0] == 1.0 and q[0].tolist() == [0x00, 0x80, 0x00]
    # the largest magnitude of a row maps to +-448 and the dequantised row is within half a code step
    rng = np.random.Generator(np.random.PCG64(24))
    x = rng.normal(0, 3, (6, 256)).astype(np.float32)
    q, s = oracle.quantise_rows_e4m3(x)
    v = oracle.e4m3fn_to_f64(q)
    assert np.all(np.max(np.abs(v), axis=1) == 448.0)
    d = oracle.dequantise_rows(q, s)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * s[:, None]) * (1 + 1e-6)
    assert np.all(np.abs(d - x) <= bound)


def _bits(x32):
    return workloads.f32_to_bf16_bits(np.asarray(x32, np.float32))


def test_w8a8_lossless_single_channel_closed_form():
    """Inputs that the quantiser keeps exactly, one intermediate channel: the
    forward is the plain MLP on those values with A rounded to bf16."""
    tab = e4m3fn_table()
    h = 16
    x = np.stack([tab[[0x38, 0x40, 0x30, 0xB8] * 4] * 2.0 ** k for k in (0, 3)]).astype(np.float32)  # M=2
    x[:, 0] = 448.0 * np.array([1.0, 8.0], np.float32)          # row amax: s = 1 and 8
    wg = np.array([[0x38] * h], np.uint8)                        # gate row: all 1.0
    wu = np.array([[0x40] * h], np.uint8)                        # up row: all 2.0
    wd = np.array([[0x38], [0xB8], [0x30]], np.uint8)            # h_out = 3: 1, -1, 0.5
    one = lambda n: np.ones(n, np.float32)
    p = oracle.rank_partial_w8a8_from_storage(_bits(x), wg, wu, wd, one(1), one(1), one(3))
    xs = oracle.bf16_bits_to_f64(_bits(x))
    g = xs.sum(axis=1)
    u = 2.0 * xs.sum(axis=1)
    a = torch.tensor(g / (1 + np.exp(-g)) * u, dtype=torch.float32).to(torch.bfloat16).double().numpy()
    # A is a single value per row: it quantises to +-448 * float32(|a| / 448), equal to a up to float32
    want = np.outer(a, [1.0, -1.0, 0.5])
    np.testing.assert_allclose(p, want, rtol=2e-7, atol=0)


def test_w8a8_matches_a_scalar_rederivation():
    """Tiny case re-derived with Python scalars: per-element float32 quotients,
    the brute-force encoder, loops for the products."""
    rng = np.random.Generator(np.random.PCG64(25))
    M, h, I_s, t = 3, 16, 8, 1
    x = rng.normal(0, 2, (M, h)).astype(np.float32)
    x[1] = 0.0
    xb = _bits(x)
    ws = workloads.make_shard_weights(77, h, I_s, 0, "e4m3fn", 0.3, 0.3)
    p = oracle.rank_partial_w8a8_from_storage(xb, ws["w_gate"], ws["w_up"], ws["w_down"], ws["s_gate"],
                                              ws["s_up"], ws["s_down"])
    tab = e4m3fn_table()

    def quant_row(row32):
        amax = max(abs(float(v)) for v in row32)
        s = np.float32(1.0) if amax == 0 else np.float32(np.float32(amax) / np.float32(448.0))
        codes = _brute_e4m3([np.float32(np.float32(v) / s) for v in row32])
        return [tab[c] for c in codes], float(s)

    wgd = [[tab[c] * float(ws["s_gate"][j]) for c in ws["w_gate"][j]] for j in range(I_s)]
    wud = [[tab[c] * float(ws["s_up"][j]) for c in ws["w_up"][j]] for j in range(I_s)]
    wdd = [[tab[c] * float(ws["s_down"][n]) for c in ws["w_down"][n]] for n in range(h)]
    for m in range(M):
        xv = oracle.bf16_bits_to_f64(xb[m]).astype(np.float32)
        xq, sx = quant_row(xv)
        a = []
        for j in range(I_s):
            g = sum(xq[i] * sx * wgd[j][i] for i in range(h))
            u = sum(xq[i] * sx * wud[j][i] for i in range(h))
            val = g / (1.0 + np.exp(-g)) * u
            a.append(float(torch.tensor(val, dtype=torch.float32).to(torch.bfloat16)))
        aq, sa = quant_row(np.array(a, np.float32))
        for n in range(h):
            want = sum(aq[j] * sa * wdd[n][j] for j in range(I_s))
            assert p[m, n] == pytest.approx(want, rel=1e-10, abs=1e-12)
