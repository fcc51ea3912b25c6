"""GPU parity of tp_partial_reduce: bit-exact against the oracle's float32 left fold."""

import numpy as np
import pytest
import torch

import oracle
import workloads
import tensor_transformer_mlp_tp_amd as tp

pytestmark = pytest.mark.gpu


def _run(parts_np, in_place=False):
    parts = [torch.from_numpy(p).cuda() for p in parts_np]
    out = parts[0] if in_place else None
    y = tp.partial_reduce(parts, out=out)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def _bits_equal(a, b):
    return np.array_equal(np.asarray(a, np.float32).view(np.uint32), np.asarray(b, np.float32).view(np.uint32))


@pytest.mark.parametrize("t", [1, 2, 3, 4, 5, 8, 13, 64])
@pytest.mark.parametrize("n", [1, 3, 4, 5, 1023, 4 * 512 * 3 + 7, 1 << 20])
def test_reduce_bit_exact(t, n):
    print("reduce t=%d n=%d" % (t, n), flush=True)
    parts = workloads.make_partials(3, t, n, weight_set=n % 97)
    assert _bits_equal(_run(parts), oracle.fold_fp32(parts))


@pytest.mark.parametrize("t", [2, 8])
def test_reduce_in_place(t):
    parts = workloads.make_partials(3, t, 100003)
    assert _bits_equal(_run(parts, in_place=True), oracle.fold_fp32(parts))


def test_reduce_order_is_fixed():
    # (1e8 + 1) - 1e8 = 0 in the left fold; another order would give 1
    n = 4099
    a = np.full(n, 1e8, np.float32)
    b = np.ones(n, np.float32)
    c = np.full(n, -1e8, np.float32)
    assert np.all(_run([a, b, c]) == 0.0)
    assert np.all(_run([a, c, b]) == 1.0)


def test_reduce_subnormals_kept():
    n = 1000
    tiny = np.full(n, 2.0 ** -140, np.float32)
    y = _run([tiny, tiny, -tiny * 0.5])
    assert _bits_equal(y, oracle.fold_fp32([tiny, tiny, -tiny * 0.5]))
    assert np.all(y > 0)


def test_reduce_empty():
    parts = [torch.empty(0, device="cuda") for _ in range(3)]
    y = tp.partial_reduce(parts)
    torch.cuda.synchronize()
    assert y.numel() == 0


def test_reduce_special_values():
    vals = np.array([np.inf, -np.inf, np.nan, 0.0, -0.0, 3.4e38, -3.4e38, 1e-45], np.float32)
    a = np.tile(vals, 8)
    b = np.repeat(vals, 8)
    y = _run([a, b])
    ref = oracle.fold_fp32([a, b])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(y), nan)
    assert _bits_equal(y[~nan], ref[~nan])


@pytest.mark.parametrize("cfg", [3, 5])
def test_reduce_full_size(cfg):
    """The configurations' reduces: 8 x (4096 x 8192) and 8 x (8192 x 16384) fp32."""
    c = workloads.CONFIGS[cfg]
    n, t = c["reduce_n"], c["t"]
    print("reduce full-size config %d: t=%d n=%d" % (cfg, t, n), flush=True)
    parts = workloads.make_partials(cfg, t, n)
    ref = oracle.fold_fp32(parts)
    dev = [torch.from_numpy(p).cuda() for p in parts]
    del parts
    y = tp.partial_reduce(dev)
    torch.cuda.synchronize()
    assert _bits_equal(y.cpu().numpy(), ref)
    # in place over partials[0], as the all-reduce it stands in for would
    tp.partial_reduce(dev, out=dev[0])
    torch.cuda.synchronize()
    assert _bits_equal(dev[0].cpu().numpy(), ref)
