"""Every finite e4m3fn code reaches the products exactly (fp8 weights, W8A16).

The kernels widen e4m3fn codes to bf16 (every e4m3fn value is a bf16 value)
before the bf16 matrix instructions.  A tolerance test would let a wrong
conversion of a few codes (subnormals, the largest exponent, negative zero)
pass, so these tests pick single weights out with one-hot activations and
require the outputs bit for bit:

* the row GEMM (the down projection's kernels, here through the attention
  output projection): token m selects input column c_m, so output n is the
  code in row n, column c_m, times a unit scale;
* the MLP forward: with W_gate all 256 (e4m3fn 0x78) and unit gate scales,
  G = 256 exactly and SiLU(256) = 256 in fp32; with up scales 1/256, A_j is the
  up code W_up[j, c_m] exactly; W_down is the identity, so P = A.

The two NaN codes (0x7F, 0xFF) are left out (a zero activation times NaN is
NaN); their places hold +0 and -0.  The oracle decodes the codes from the
OCP E4M3FN field definitions (``oracle/formats.py``).
"""

import numpy as np
import pytest
import torch

import oracle
import tensor_transformer_mlp_tp_amd as tp

pytestmark = pytest.mark.gpu

FINITE = np.array([c for c in range(256) if c not in (0x7F, 0xFF)] + [0x00, 0x80], dtype=np.uint8)   # 256 entries
assert len(FINITE) == 256 and len(set(FINITE.tolist())) == 254


def _fp8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).view(torch.float8_e4m3fn).cuda()


def _one_hot_bf16(M, K, cols):
    o = np.zeros((M, K), np.uint16)
    o[np.arange(M), cols] = 0x3F80                      # bf16 1.0
    return torch.from_numpy(o.view(np.int16)).view(torch.bfloat16).cuda()


def _code_matrix(rows):
    # rows x 256, every finite code in every row and in every column
    return np.stack([np.roll(FINITE, 5 * n) for n in range(rows)])


@pytest.mark.parametrize("M", [1, 32, 64, 256])
def test_fp8_codes_widen_exactly_row_gemm(M):
    """Output projection (K = 256 input columns, h = 512 output rows; decode
    streams up to 64 tokens, the MFMA GEMM at 256)."""
    print("fp8 every code, row GEMM M=%d" % M, flush=True)
    nh, d, t, h = 4, 64, 1, 512
    K = nh // t * d
    w = _code_matrix(h)
    cols = (np.arange(M) * 37) % K
    p = tp.attn_out_forward(_one_hot_bf16(M, K, cols), _fp8(w), n_heads=nh, head_dim=d, t=t, k=0,
                            s_o=torch.ones(h, dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    want = oracle.e4m3fn_to_f64(w)[:, cols].T        # M x h
    assert np.array_equal(p.cpu().numpy().astype(np.float64), want)


@pytest.mark.parametrize("M", [1, 8, 32, 200])
def test_fp8_codes_widen_exactly_mlp(M):
    """MLP forward with h = I_s = 256 (gate/up and down decode streams up to
    32 tokens, the MFMA GEMMs at 200): P[m, n] is the up code W_up[n, c_m]."""
    print("fp8 every code, MLP M=%d" % M, flush=True)
    h = I_s = 256
    t = 2
    cols = (np.arange(M) * 37) % h
    w_gate = np.full((I_s, h), 0x78, np.uint8)          # e4m3fn 256.0
    w_up = _code_matrix(I_s)
    w_down = np.zeros((h, I_s), np.uint8)
    w_down[np.arange(h), np.arange(h)] = 0x38           # e4m3fn 1.0
    assert oracle.e4m3fn_to_f64(np.array([0x78, 0x38], np.uint8)).tolist() == [256.0, 1.0]
    ones = torch.ones(I_s, dtype=torch.float32, device="cuda")
    p = tp.shard_forward(_one_hot_bf16(M, h, cols), _fp8(w_gate), _fp8(w_up), _fp8(w_down), t=t, k=0,
                         s_gate=ones, s_up=torch.full((I_s,), 1.0 / 256.0, dtype=torch.float32, device="cuda"),
                         s_down=torch.ones(h, dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    want = oracle.e4m3fn_to_f64(w_up)[:, cols].T        # M x 256
    got = p.cpu().numpy().astype(np.float64)
    assert np.array_equal(got, want), np.argwhere(got != want)[:8]
