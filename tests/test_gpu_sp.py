"""Sequence-parallel forms on the GPU: the forward over t row blocks of X
(tp_mlp_shard_forward_sp) against the forward on the gathered X and the
oracle, and the reduce-scatter (tp_partial_reduce_scatter) against the
oracle's fixed-order fold, bit for bit ("Chapter 12 Parallelism Strategies",
arunshar.com, section 12.3.1)."""

import numpy as np
import pytest
import torch

import oracle
import tensor_transformer_mlp_tp_amd as tp
from helpers import TOL_BF16, TOL_FP8, make_case, upload_case, oracle_partial

pytestmark = pytest.mark.gpu


def _blocks(xdev, t, pad=0):
    """The t row blocks of X as separate allocations (optionally with a padded
    leading dimension), filled from the gathered X."""
    M, h = xdev.shape
    r = M // t
    out = []
    for j in range(t):
        buf = torch.zeros((r, h + pad), dtype=xdev.dtype, device=xdev.device)
        buf[:, :h] = xdev[j * r:(j + 1) * r]
        out.append(buf[:, :h] if pad else buf)
    return out


@pytest.mark.parametrize("M,t,h,I_s,w", [
    (8, 8, 512, 640, "bf16"),       # one token per block (decode, register-fragment path)
    (16, 4, 512, 640, "bf16"),
    (64, 8, 512, 640, "bf16"),      # decode, activation-staged path
    (32, 4, 1024, 1280, "e4m3fn"),
    (48, 8, 320, 192, "bf16"),      # decode shapes off the streaming grid (register-batch kernels)
    (520, 8, 320, 192, "bf16"),     # prefill, 65-row blocks: block edges inside MFMA tiles
    (1024, 4, 512, 384, "e4m3fn"),
    (520, 8, 2112, 2112, "bf16"),   # prefill with stream-K tails in both GEMMs (every tile in 2 pieces)
])
def test_forward_sp_matches_gathered(M, t, h, I_s, w):
    print("forward_sp M=%d t=%d h=%d I_s=%d w=%s" % (M, t, h, I_s, w), flush=True)
    x, ws = make_case(47, M, h, I_s, "bf16", w, 0.05, 0.05, weight_set=M + t)
    d = upload_case(x, ws, "bf16", w)
    kw = dict(t=t, k=0, s_gate=d["s_gate"], s_up=d["s_up"], s_down=d["s_down"])
    ref_gpu = tp.shard_forward(d["x"], d["w_gate"], d["w_up"], d["w_down"], **kw)
    for pad in (0, 64):
        got = tp.shard_forward_sp(_blocks(d["x"], t, pad), d["w_gate"], d["w_up"], d["w_down"], **kw)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int32), ref_gpu.view(torch.int32)), pad
    # and against the oracle on the gathered rows
    xb = [x[j * (M // t):(j + 1) * (M // t)] for j in range(t)]
    ref = oracle_partial(oracle.gather_rows(xb), ws, "bf16", w)
    err = oracle.rms_normalised_max_error(got.cpu().numpy(), ref)
    assert err <= (TOL_FP8 if w == "e4m3fn" else TOL_BF16), err


def test_forward_sp_fp32_tiny():
    M, t, h, I_s = 16, 4, 256, 256
    x, ws = make_case(1, M, h, I_s, "f32", "f32", 1 / 16, 1 / 32)
    d = upload_case(x, ws, "f32", "f32")
    ref_gpu = tp.shard_forward(d["x"], d["w_gate"], d["w_up"], d["w_down"], t=t, k=0)
    got = tp.shard_forward_sp(_blocks(d["x"], t), d["w_gate"], d["w_up"], d["w_down"], t=t, k=0)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int32), ref_gpu.view(torch.int32))


@pytest.mark.parametrize("rows,cols,t", [(8, 16, 8), (64, 8192, 8), (4096, 8192, 8), (24, 20, 3), (4, 4, 1)])
def test_reduce_scatter_bit_exact(rows, cols, t):
    print("reduce_scatter rows=%d cols=%d t=%d" % (rows, cols, t), flush=True)
    rng = np.random.Generator(np.random.PCG64(rows * 7 + t))
    parts = [(rng.standard_normal((rows, cols)) * 10.0 ** rng.integers(-2, 3)).astype(np.float32)
             for _ in range(t)]
    dev = [torch.from_numpy(p).cuda() for p in parts]
    for k in range(t):
        got = tp.partial_reduce_scatter(dev, k)
        want = oracle.reduce_scatter_fp32(parts, k)
        assert np.array_equal(got.cpu().numpy().view(np.uint32), want.view(np.uint32)), k


def test_reduce_scatter_in_place():
    rows, cols, t, k = 64, 256, 4, 2
    rng = np.random.Generator(np.random.PCG64(5))
    parts = [rng.standard_normal((rows, cols)).astype(np.float32) for _ in range(t)]
    dev = [torch.from_numpy(p).cuda() for p in parts]
    r = rows // t
    out = dev[0][k * r:(k + 1) * r]          # rank k's slice of its own partial
    tp.partial_reduce_scatter(dev, k, out=out)
    want = oracle.reduce_scatter_fp32(parts, k)
    assert np.array_equal(dev[0][k * r:(k + 1) * r].cpu().numpy().view(np.uint32), want.view(np.uint32))
    # rows outside the slice are untouched
    assert np.array_equal(dev[0][:k * r].cpu().numpy(), parts[0][:k * r])
