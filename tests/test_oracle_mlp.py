"""Pins for the oracle's MLP shard, unsharded MLP and fixed-order fold.

Each check is independent of the oracle's own code path: a hand-worked
example, closed forms, pure-Python brute force, torch's silu as a library
special case, the Megatron split-equals-unsplit invariant (the equivalence
test the engineer-atlas.dev page asks for, "What must stay true after
deployment"), and hand-built float32 sums for the fold order.
"""

import math

import numpy as np
import pytest
import torch

from conftest import read_golden
import oracle
import workloads


# ----------------------------------------------------------------- SiLU

def test_silu_closed_forms():
    for z, want in read_golden("silu_values.txt"):
        got = oracle.silu(np.array([float(z)]))[0]
        assert got == pytest.approx(float(want), rel=1e-15, abs=1e-300)


def test_silu_odd_part_identity():
    # z*s(z) - (-z)*s(-z) = z (s(z) + s(-z)) = z: catches a sign slip in either term
    z = np.linspace(-30, 30, 1001)
    np.testing.assert_allclose(oracle.silu(z) - oracle.silu(-z), z, rtol=1e-13, atol=1e-13)


def test_silu_limits():
    assert oracle.silu(np.array([-1000.0]))[0] == 0.0
    assert oracle.silu(np.array([1000.0]))[0] == 1000.0
    assert oracle.silu(np.array([0.0]))[0] == 0.0


def test_silu_matches_torch():
    z = np.random.Generator(np.random.PCG64(3)).normal(0, 5, 10000)
    ref = torch.nn.functional.silu(torch.from_numpy(z)).numpy()
    np.testing.assert_allclose(oracle.silu(z), ref, rtol=1e-14, atol=1e-300)


# ----------------------------------------------------------------- MLP

def _golden_tiny():
    rows = {r[0]: [float(v) for v in r[1:]] for r in read_golden("tiny_mlp_worked.txt")}
    x = np.array(rows["X"]).reshape(1, 2)
    wg = np.array(rows["W_gate"]).reshape(2, 2)
    wu = np.array(rows["W_up"]).reshape(2, 2)
    wd = np.array(rows["W_down"]).reshape(2, 2)
    return x, wg, wu, wd, rows


def test_hand_worked_example():
    x, wg, wu, wd, rows = _golden_tiny()
    y = oracle.mlp_full(x, wg, wu, wd)
    np.testing.assert_allclose(y[0], rows["Y"], rtol=1e-15)
    for k in range(2):
        g, u, d = oracle.shard_of_full(wg, wu, wd, 2, k)
        p = oracle.mlp_partial(x, g, u, d)
        np.testing.assert_allclose(p[0], rows["P_%d" % k], rtol=1e-15, atol=0)


def _brute_partial(x, wg, wu, wd):
    M, h = len(x), len(x[0])
    I_s = len(wg)
    out = [[0.0] * len(wd) for _ in range(M)]
    for m in range(M):
        a = []
        for j in range(I_s):
            g = sum(x[m][i] * wg[j][i] for i in range(h))
            u = sum(x[m][i] * wu[j][i] for i in range(h))
            a.append(g / (1.0 + math.exp(-g)) * u)
        for n in range(len(wd)):
            out[m][n] = sum(a[j] * wd[n][j] for j in range(I_s))
    return out


@pytest.mark.parametrize("M,h,I_s", [(1, 3, 4), (2, 5, 3), (3, 4, 6)])
def test_brute_force_tiny(M, h, I_s):
    rng = np.random.Generator(np.random.PCG64(M * 100 + h * 10 + I_s))
    x = rng.normal(size=(M, h))
    wg = rng.normal(size=(I_s, h))
    wu = rng.normal(size=(I_s, h))
    wd = rng.normal(size=(h + 1, I_s))  # output width != h on purpose: shapes stay distinct
    ref = np.array(_brute_partial(x.tolist(), wg.tolist(), wu.tolist(), wd.tolist()))
    got = oracle.mlp_partial(x, wg, wu, wd)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_matches_torch_float64():
    rng = np.random.Generator(np.random.PCG64(11))
    x = rng.normal(size=(7, 24))
    wg, wu = rng.normal(size=(40, 24)) * 0.2, rng.normal(size=(40, 24)) * 0.2
    wd = rng.normal(size=(24, 40)) * 0.2
    tx, tg, tu, td = (torch.from_numpy(a) for a in (x, wg, wu, wd))
    ref = (torch.nn.functional.silu(tx @ tg.T) * (tx @ tu.T)) @ td.T
    np.testing.assert_allclose(oracle.mlp_full(x, wg, wu, wd), ref.numpy(), rtol=1e-13, atol=1e-13)


def test_gate_and_up_are_not_interchangeable():
    # one channel: y = c * (b x) * SiLU(a x); swapping gate/up gives c * (a x) * SiLU(b x)
    x = np.array([[1.5]])
    a, b, c = 0.7, -2.0, 3.0
    y = oracle.mlp_full(x, [[a]], [[b]], [[c]])[0, 0]
    assert y == pytest.approx(c * b * 1.5 * (a * 1.5) / (1 + math.exp(-a * 1.5)), rel=1e-15)
    swapped = c * a * 1.5 * (b * 1.5) / (1 + math.exp(-b * 1.5))
    assert abs(y - swapped) > 1e-3


def test_zero_up_gives_zero():
    rng = np.random.Generator(np.random.PCG64(5))
    x = rng.normal(size=(4, 8))
    y = oracle.mlp_full(x, rng.normal(size=(6, 8)), np.zeros((6, 8)), rng.normal(size=(8, 6)))
    assert np.all(y == 0.0)


@pytest.mark.parametrize("t", [1, 2, 4, 8])
def test_split_sums_to_unsplit(t):
    rng = np.random.Generator(np.random.PCG64(t))
    M, h, I = 5, 16, 32
    x = rng.normal(size=(M, h))
    wg, wu = rng.normal(size=(I, h)) / 4, rng.normal(size=(I, h)) / 4
    wd = rng.normal(size=(h, I)) / 6
    full = oracle.mlp_full(x, wg, wu, wd)
    parts = [oracle.mlp_partial(x, *oracle.shard_of_full(wg, wu, wd, t, k)) for k in range(t)]
    total = np.sum(parts, axis=0)
    np.testing.assert_allclose(total, full, rtol=1e-12, atol=1e-12 * np.abs(full).max())
    # the order of the ranks does not matter in exact arithmetic either
    np.testing.assert_allclose(np.sum(parts[::-1], axis=0), full, rtol=1e-12,
                               atol=1e-12 * np.abs(full).max())
    if t == 1:
        assert np.array_equal(parts[0], full)


def test_shard_is_contiguous_block():
    I, h, t = 16, 3, 4
    wg = np.arange(I * h, dtype=np.float64).reshape(I, h)
    wd = np.arange(h * I, dtype=np.float64).reshape(h, I)
    for k in range(t):
        g, u, d = oracle.shard_of_full(wg, wg, wd, t, k)
        assert np.array_equal(g, wg[4 * k:4 * k + 4])
        assert np.array_equal(d, wd[:, 4 * k:4 * k + 4])
    # P_k depends on rows S_k of W_gate only
    rng = np.random.Generator(np.random.PCG64(2))
    x = rng.normal(size=(2, h))
    wg, wu, wd = rng.normal(size=(I, h)), rng.normal(size=(I, h)), rng.normal(size=(h, I))
    p1 = oracle.mlp_partial(x, *oracle.shard_of_full(wg, wu, wd, t, 1))
    wg2 = wg.copy()
    wg2[0] += 1.0      # row of rank 0
    assert np.array_equal(p1, oracle.mlp_partial(x, *oracle.shard_of_full(wg2, wu, wd, t, 1)))
    wg2[5] += 1.0      # row of rank 1
    assert not np.array_equal(p1, oracle.mlp_partial(x, *oracle.shard_of_full(wg2, wu, wd, t, 1)))


def test_shard_slice_rejects_bad_args():
    with pytest.raises(ValueError):
        oracle.shard_slice(10, 4, 0)
    with pytest.raises(ValueError):
        oracle.shard_slice(8, 4, 4)
    with pytest.raises(ValueError):
        oracle.shard_slice(8, 0, 0)


def test_storage_decoding_paths():
    rng = np.random.Generator(np.random.PCG64(21))
    M, h, I_s = 3, 32, 16
    x32 = rng.normal(size=(M, h)).astype(np.float32)
    w = [rng.normal(0, 0.1, size=s).astype(np.float32) for s in ((I_s, h), (I_s, h), (h, I_s))]
    # bf16: the oracle must see exactly the rounded values
    xb = workloads.f32_to_bf16_bits(x32)
    wb = [workloads.f32_to_bf16_bits(a) for a in w]
    got = oracle.rank_partial_from_storage(xb, "bf16", *wb, "bf16")
    xr = torch.from_numpy(x32).to(torch.bfloat16).double().numpy()
    wr = [torch.from_numpy(a).to(torch.bfloat16).double().numpy() for a in w]
    np.testing.assert_allclose(got, oracle.mlp_full(xr, *wr), rtol=0, atol=0)
    # e4m3fn: dequantised weights are code value times the row scale
    qs = [workloads.quantise_rows_e4m3fn(a) for a in w]
    got = oracle.rank_partial_from_storage(xb, "bf16", qs[0][0], qs[1][0], qs[2][0], "e4m3fn",
                                           qs[0][1], qs[1][1], qs[2][1])
    deq = [torch.from_numpy(q).view(torch.float8_e4m3fn).double().numpy() * s.astype(np.float64)[:, None]
           for q, s in qs]
    np.testing.assert_allclose(got, oracle.mlp_full(xr, *deq), rtol=0, atol=0)
    with pytest.raises(ValueError):
        oracle.rank_partial_from_storage(xb, "bf16", qs[0][0], qs[1][0], qs[2][0], "e4m3fn")


# ----------------------------------------------------------------- fold

def test_fold_order_is_left_to_right():
    big = np.float32(1e8)
    p = [np.array([big], np.float32), np.array([1.0], np.float32), np.array([-big], np.float32)]
    # (1e8 + 1) rounds to 1e8 in binary32 (spacing 8 there), then - 1e8 = 0
    assert oracle.fold_fp32(p)[0] == 0.0
    # another order gives another answer: (1e8 - 1e8) + 1 = 1
    assert oracle.fold_fp32([p[0], p[2], p[1]])[0] == 1.0


def test_fold_single_buffer_is_copy():
    a = workloads.draw_f32(5, (1000,), 1.0)
    y = oracle.fold_fp32([a])
    assert y.dtype == np.float32 and np.array_equal(y.view(np.uint32), a.view(np.uint32))
    assert y is not a


def test_fold_matches_exact_rounding():
    # for two binary32 operands whose exponents differ by < 29 the float64 sum is
    # exact, so rounding it to binary32 is the correctly rounded binary32 sum
    a = workloads.draw_f32(6, (5000,), 1.0)
    b = workloads.draw_f32(7, (5000,), 1.0)
    keep = (np.abs(a) > 1e-6) & (np.abs(b) > 1e-6)
    a, b = a[keep], b[keep]
    want = (a.astype(np.float64) + b.astype(np.float64)).astype(np.float32)
    got = oracle.fold_fp32([a, b])
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    # three buffers: the third is added to the rounded sum of the first two
    c = workloads.draw_f32(8, (a.size,), 1.0)
    c = np.where(np.abs(c) > 1e-6, c, np.float32(1.0)).astype(np.float32)
    want3 = (want.astype(np.float64) + c.astype(np.float64)).astype(np.float32)
    assert np.array_equal(oracle.fold_fp32([a, b, c]).view(np.uint32), want3.view(np.uint32))


def test_fold_keeps_subnormals():
    tiny = np.array([2.0 ** -140], np.float32)
    assert oracle.fold_fp32([tiny, tiny])[0] == np.float32(2.0 ** -139)


def test_error_metric():
    ref = np.array([3.0, -4.0])          # rms = sqrt(12.5)
    out = np.array([3.5, -4.0])
    assert oracle.rms_normalised_max_error(out, ref) == pytest.approx(0.5 / math.sqrt(12.5))
    assert oracle.rms_normalised_max_error(ref, ref) == 0.0


# ------------------------------------------------------------ sequence-parallel forms (12.3.1)

def test_reduce_scatter_rows_closed_form():
    # partial j, row i holds i * 1000 + j (exact in float32): rank k's rows of the
    # sum are sum_j (i * 1000 + j) = t * i * 1000 + t (t - 1) / 2 for its rows i only
    t, rows, cols = 4, 12, 5
    parts = [np.repeat((np.arange(rows) * 1000.0 + j)[:, None], cols, axis=1).astype(np.float32)
             for j in range(t)]
    for k in range(t):
        got = oracle.reduce_scatter_fp32(parts, k)
        i = np.arange(k * rows // t, (k + 1) * rows // t)
        want = (t * i * 1000.0 + t * (t - 1) / 2)[:, None] * np.ones(cols)
        assert got.shape == (rows // t, cols)
        assert np.array_equal(got, want.astype(np.float32))


def test_reduce_scatter_tiles_the_full_fold():
    # the t ranks' reduce-scatter outputs, stacked in rank order, are the full fold, bit for bit
    rng = np.random.Generator(np.random.PCG64(17))
    t = 8
    parts = [(rng.standard_normal((16, 24)) * 10.0 ** rng.integers(-3, 4)).astype(np.float32) for _ in range(t)]
    full = oracle.fold_fp32(parts)
    stacked = np.concatenate([oracle.reduce_scatter_fp32(parts, k) for k in range(t)], axis=0)
    assert np.array_equal(stacked.view(np.uint32), full.view(np.uint32))
    with pytest.raises(ValueError):
        oracle.reduce_scatter_fp32([p[:15] for p in parts], 0)


def test_gather_rows_then_shard_is_the_unsplit_input():
    # row blocks of a sequence, gathered, give back the sequence; the MLP of the
    # gathered rows equals, row block by row block, the MLP of each block
    rng = np.random.Generator(np.random.PCG64(18))
    t, s, h, I = 4, 8, 6, 10
    x = rng.standard_normal((s, h))
    blocks = [x[j * s // t:(j + 1) * s // t] for j in range(t)]
    assert np.array_equal(oracle.gather_rows(blocks), x)
    wg, wu, wd = rng.standard_normal((I, h)), rng.standard_normal((I, h)), rng.standard_normal((h, I))
    y = oracle.mlp_full(oracle.gather_rows(blocks), wg, wu, wd)
    for j in range(t):
        np.testing.assert_allclose(y[j * s // t:(j + 1) * s // t], oracle.mlp_full(blocks[j], wg, wu, wd),
                                   rtol=1e-13, atol=1e-13)
