"""fp8 x fp8 (W8A8) on the GPU: the per-token activation quantiser bit for
bit against the oracle's, and the W8A8 rank forward against the oracle's
W8A8 steps (``oracle/w8a8.py``) within the fp8 bound."""

import numpy as np
import pytest
import torch

import oracle
import tensor_transformer_mlp_tp_amd as tp
import workloads
from helpers import TOL_FP8, make_case, upload_case

# How the W8A8 forward is judged.  The codes of X are decisions on exact
# bf16 inputs taken in the kernels' own (fp32) precision, so they and their
# scales must equal the oracle's bit for bit.  The codes of A are decisions on
# the GPU's A, which comes from fp32 sums of fp8 products (not exact fp32)
# where the oracle has fp64: an element of A near a bf16 rounding boundary can
# round to the neighbouring bf16 value, and a row maximum that moves by one
# bf16 step rescales every code of its row.  Each of those outputs is still a
# correct one, so the check is made in steps, none with a fitted bound:
#   1. X's codes and scales equal the oracle's (bit for bit);
#   2. the GPU's A is within one bf16 step of the oracle's A (near zero, where
#      the gate sums cancel, within A_ABS_FLOOR of the RMS of A);
#   3. A's codes and scales are the oracle's quantiser applied to the GPU's own
#      A (bit for bit): each code that differs from the oracle's is the e4m3
#      round-to-nearest-even of a correctly rounded A;
#   4. the partial equals the down projection of the GPU's own A codes, within
#      the fp8 bound TOL_FP8 (this isolates the down GEMM);
#   5. rows whose A codes all equal the oracle's meet TOL_FP8 against the
#      oracle's partial end to end, and every other row is within the bound
#      that follows from 4 and the triangle inequality: its step-4 error plus
#      |deq(Aq_gpu) - deq(Aq_ref)| . |W_down|^T, the exact effect of its
#      differing codes.
A_DIFF_FRACTION = 0.05  # elements of A that differ from the oracle's at all
A_ABS_FLOOR = 1e-3      # x RMS(A): absolute error of the fp8 sums near zero

pytestmark = pytest.mark.gpu


def _bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


# rows of 1 to 8 chunks of 8 per thread held in registers, and (20480) the two-pass loop
@pytest.mark.parametrize("rows,cols,scale", [(1, 8, 1.0), (7, 136, 3.0), (64, 8192, 1.0), (300, 3584, 1e-3),
                                              (5, 1024, 1e4), (3, 16384, 1.0), (2, 20480, 2.0)])
def test_quantiser_bit_exact(rows, cols, scale):
    print("quant rows=%d cols=%d" % (rows, cols), flush=True)
    rng = np.random.Generator(np.random.PCG64(rows * 7 + cols))
    x = (rng.normal(0, scale, (rows, cols)) * np.where(rng.random((rows, cols)) < 0.05, 30.0, 1.0)).astype(np.float32)
    if rows > 2:
        x[1] = 0.0                       # an all-zero row
        x[2, ::3] = -0.0
    xb = workloads.f32_to_bf16_bits(x)
    q, s = tp.quantize_rows_e4m3(_bf16_dev(xb))
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantise_rows_e4m3(oracle.bf16_bits_to_f64(xb).astype(np.float32))
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), q_ref)


def test_quantiser_row_scales_across_the_range():
    """Rows whose magnitudes run from bf16 subnormals (the scale an fp32
    subnormal) to 1e37: every code and scale bit-exact."""
    print("quant scales across the range", flush=True)
    rng = np.random.Generator(np.random.PCG64(77))
    rows, cols = 80, 1024
    exps = np.linspace(-40.0, 37.0, rows)
    x = (rng.normal(0, 1, (rows, cols)) * 10.0 ** exps[:, None]).astype(np.float32)
    x[:, 5] = -0.0
    xb = workloads.f32_to_bf16_bits(x)
    q, s = tp.quantize_rows_e4m3(_bf16_dev(xb))
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantise_rows_e4m3(oracle.bf16_bits_to_f64(xb).astype(np.float32))
    assert s_ref[0] < np.finfo(np.float32).tiny        # the first rows' scales are fp32 subnormals
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), q_ref)


def test_quantiser_ties_and_saturation():
    """Rows whose scale is a power of two (amax = 448 * 2^e), so x / s lands
    exactly on code midpoints: ties must go to the even code; and values at
    the top of the range."""
    tab = oracle.formats.e4m3fn_table()[:0x7F]
    mids = ((tab[:-1] + tab[1:]) / 2)[:120]
    row = np.concatenate([[448.0], mids, -mids, [444.0, 440.0, 432.0, 416.0, 0.0]]).astype(np.float32)
    cols = (len(row) + 7) // 8 * 8
    x = np.zeros((4, cols), np.float32)
    for e in range(4):
        x[e, :len(row)] = row * np.float32(2.0 ** (e - 2))
    xb = workloads.f32_to_bf16_bits(x)
    assert np.array_equal(oracle.bf16_bits_to_f64(xb), x.astype(np.float64))   # exact in bf16
    q, s = tp.quantize_rows_e4m3(_bf16_dev(xb))
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantise_rows_e4m3(x)
    assert np.array_equal(s.cpu().numpy(), s_ref)
    assert np.array_equal(q.cpu().numpy(), q_ref)


def _w8a8_layout(M, h, I_s):
    """Byte offsets of what tp_mlp_shard_forward_w8a8 leaves in its workspace
    (include/tp_mlp.h): A (bf16), X's codes, X's scales, A's codes, A's
    scales, each at a 256-byte boundary."""
    def r(n):
        return (n + 255) // 256 * 256
    a = 0
    xq = a + r(M * I_s * 2)
    sx = xq + r(M * h)
    aq = sx + r(M * 4)
    sa = aq + r(M * I_s)
    return a, xq, sx, aq, sa


def _w8a8_check(x, ws, M, h, I_s, t):
    """Run the W8A8 forward and check it in the five steps above; returns the
    partial and a summary."""
    d = upload_case(x, ws, "bf16", "e4m3fn")
    scratch = tp.alloc_workspace(tp.w8a8_workspace_bytes(M, h, I_s * t, t), "cuda")
    p = tp.shard_forward_w8a8(d["x"], d["w_gate"], d["w_up"], d["w_down"], t=t, k=0, s_gate=d["s_gate"],
                              s_up=d["s_up"], s_down=d["s_down"], workspace=scratch)
    torch.cuda.synchronize()
    o_a, o_xq, o_sx, o_aq, o_sa = _w8a8_layout(M, h, I_s)
    wsb = scratch.cpu().numpy()
    a_gpu = wsb[o_a:o_a + M * I_s * 2].view(np.uint16).reshape(M, I_s)
    xq_gpu = wsb[o_xq:o_xq + M * h].reshape(M, h)
    sx_gpu = wsb[o_sx:o_sx + M * 4].view(np.float32)
    aq_gpu = wsb[o_aq:o_aq + M * I_s].reshape(M, I_s)
    sa_gpu = wsb[o_sa:o_sa + M * 4].view(np.float32)
    pg = p.cpu().numpy().astype(np.float64)
    ref, steps = oracle.rank_partial_w8a8_from_storage(x, ws["w_gate"], ws["w_up"], ws["w_down"], ws["s_gate"],
                                                       ws["s_up"], ws["s_down"], return_codes=True)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    # 1. X's codes and scales
    assert np.array_equal(sx_gpu.view(np.uint32), steps["sx"].view(np.uint32)), "X scales"
    assert np.array_equal(xq_gpu, steps["xq"]), "X codes"
    # 2. A within one bf16 step
    ag, ar = oracle.bf16_bits_to_f64(a_gpu), oracle.bf16_bits_to_f64(steps["a_bits"])
    mag = np.maximum(np.abs(ag), np.abs(ar))
    ulp = np.where(mag > 0, 2.0 ** (np.floor(np.log2(np.where(mag > 0, mag, 1.0))) - 7), 0.0)
    floor = A_ABS_FLOOR * np.sqrt(np.mean(ar ** 2))
    assert np.all(np.abs(ag - ar) <= np.maximum(ulp, floor)), "A differs by more than one bf16 step"
    e_a = float(np.mean(ag != ar))
    assert e_a <= A_DIFF_FRACTION, e_a
    # 3. A's codes: the oracle's quantiser of the GPU's A
    aq_own, sa_own = oracle.quantise_rows_e4m3(ag.astype(np.float32))
    assert np.array_equal(sa_gpu.view(np.uint32), sa_own.view(np.uint32)), "A scales"
    assert np.array_equal(aq_gpu, aq_own), "A codes"
    # 4. the down GEMM on the GPU's own codes
    wd = oracle.dequantise_rows(ws["w_down"], ws["s_down"])
    p_own = oracle.dequantise_rows(aq_gpu, sa_gpu) @ wd.T
    e_down = oracle.rms_normalised_max_error(pg, p_own)
    assert e_down <= TOL_FP8, e_down
    # 5. end to end against the oracle
    same = np.all(aq_gpu == steps["aq"], axis=1) & (sa_gpu.view(np.uint32) == steps["sa"].view(np.uint32))
    err = np.abs(pg - ref)
    e_same = float(err[same].max() / rms) if same.any() else 0.0
    assert e_same <= TOL_FP8, e_same
    flips = ~same
    e_flip = 0.0
    if flips.any():
        delta = np.abs(oracle.dequantise_rows(aq_gpu[flips], sa_gpu[flips]) -
                       oracle.dequantise_rows(steps["aq"][flips], steps["sa"][flips]))
        bound = e_down * float(np.sqrt(np.mean(p_own ** 2))) + delta @ np.abs(wd).T
        assert np.all(err[flips] <= bound * (1 + 1e-12)), "rows with differing A codes exceed their bound"
        e_flip = float(err[flips].max() / rms)
    print("w8a8 M=%d h=%d I_s=%d: A differing %.2e; down on own codes %.2e; rows with equal codes %d, max %.2e; "
          "rows with differing codes %d, max %.2e" % (M, h, I_s, e_a, e_down, int(same.sum()), e_same,
                                                     int(flips.sum()), e_flip), flush=True)
    return p, dict(e_a=e_a, e_down=e_down, e_same=e_same, e_flip=e_flip, flips=int(flips.sum()))


@pytest.mark.parametrize("M,h,I_s", [
    (1, 512, 384),
    (37, 1024, 768),
    (256, 512, 384),
    (300, 1024, 640),
    (1024, 2048, 1536),
    (300, 4096, 2048),     # gate/up tiles cut along K in 2 stream-K pieces (32 k-tiles of 128)
    (2304, 7424, 4096),    # 256-token tiles (eight-wave kernel) with stream-K tails in both GEMMs:
                           # gate/up 288 tiles (32 in 3 pieces), down 261 tiles (5 in 2 pieces)
    (2200, 4096, 4096),    # ... ragged: the last 256-token tile holds 152 tokens (gate/up 288 tiles,
                           # 32 in 2 pieces)
])
def test_w8a8_forward_shapes(M, h, I_s):
    x, ws = make_case(93, M, h, I_s, "bf16", "e4m3fn", 0.05, 0.05, weight_set=M)
    _w8a8_check(x, ws, M, h, I_s, 2)


def test_w8a8_config4_prefill_full():
    """70B-shaped TP=4 rank with fp8 weights at 2048 tokens, every element."""
    c = workloads.CONFIGS[4]
    h, I_s, M = c["h"], c["I"] // c["t"], 2048
    print("w8a8 config 4 M=%d" % M, flush=True)
    x, ws = make_case(4, M, h, I_s, "bf16", "e4m3fn", c["std_gu"], c["std_down"])
    p, _ = _w8a8_check(x, ws, M, h, I_s, c["t"])
    # against the fp8-weight (bf16 activation) forward: the activation quantisation's own effect
    d = upload_case(x, ws, "bf16", "e4m3fn")
    p16 = tp.shard_forward(d["x"], d["w_gate"], d["w_up"], d["w_down"], t=c["t"], k=0, s_gate=d["s_gate"],
                           s_up=d["s_up"], s_down=d["s_down"])
    torch.cuda.synchronize()
    print("w8a8 vs w8a16 rms-normalised max difference: %.4f" % oracle.rms_normalised_max_error(
        p.cpu().numpy(), p16.cpu().numpy().astype(np.float64)), flush=True)


def test_w8a8_deterministic_and_k_independent():
    M, h, I_s = 300, 1024, 640
    x, ws = make_case(94, M, h, I_s, "bf16", "e4m3fn", 0.05, 0.05)
    d = upload_case(x, ws, "bf16", "e4m3fn")
    kw = dict(s_gate=d["s_gate"], s_up=d["s_up"], s_down=d["s_down"], t=2)
    a = tp.shard_forward_w8a8(d["x"], d["w_gate"], d["w_up"], d["w_down"], k=0, **kw)
    b = tp.shard_forward_w8a8(d["x"], d["w_gate"], d["w_up"], d["w_down"], k=1, **kw)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
