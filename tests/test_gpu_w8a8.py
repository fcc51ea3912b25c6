"""fp8 x fp8 (W8A8) on the GPU: the per-token activation quantiser bit for
bit against the oracle's, and the W8A8 rank forward against the oracle's
W8A8 steps (``oracle/w8a8.py``) within the fp8 bound."""

import numpy as np
import pytest
import torch

import oracle
import tensor_transformer_mlp_tp_amd as tp
import workloads
from helpers import make_case, upload_case

# Bounds (RMS-normalised, against the oracle's W8A8 steps).  The activation
# codes are decisions on floating-point values: X's are taken in the same
# fp32 arithmetic and match bit for bit (tested below), but A's come from
# fp32 sums (fp8 MFMA partial sums are not exact fp32) against the oracle's
# fp64, so an A element near a bf16 or e4m3 rounding boundary, or a row
# maximum that moves by one bf16 step (which rescales every code of the
# row), can round differently: one e4m3 step is 1/8 to 1/16 of the value.
# A before its quantisation: every element equals the oracle's bf16 value or
# a neighbour (one bf16 step), and few of them differ at all.
A_DIFF_FRACTION = 0.05
A_ABS_FLOOR = 1e-3     # x RMS(A): the fp32 (fp8 MFMA) sums' absolute error near zero
TOL_W8A8_P = 0.15      # max over the partial: rows whose A codes moved
TOL_W8A8_RMS = 1.5e-2  # RMS over the partial: a systematic error would be O(1)

pytestmark = pytest.mark.gpu


def _bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


@pytest.mark.parametrize("rows,cols,scale", [(1, 8, 1.0), (7, 136, 3.0), (64, 8192, 1.0), (300, 3584, 1e-3),
                                              (5, 1024, 1e4)])
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


def _w8a8_errors(x, ws, M, h, I_s, t, rows=None):
    """Run the W8A8 forward; return (fraction of A elements that differ from
    the oracle's, P max error, P rms error), the errors normalised by the
    reference's RMS.  A is read back from the workspace,
    where the forward leaves it (bf16, M x I_s at the start)."""
    d = upload_case(x, ws, "bf16", "e4m3fn")
    scratch = tp.alloc_workspace(tp.w8a8_workspace_bytes(M, h, I_s * t, t), "cuda")
    p = tp.shard_forward_w8a8(d["x"], d["w_gate"], d["w_up"], d["w_down"], t=t, k=0, s_gate=d["s_gate"],
                              s_up=d["s_up"], s_down=d["s_down"], workspace=scratch)
    torch.cuda.synchronize()
    rows = np.arange(M) if rows is None else rows
    a_gpu = scratch[:M * I_s * 2].view(torch.int16).cpu().numpy().view(np.uint16).reshape(M, I_s)[rows]
    ref, steps = oracle.rank_partial_w8a8_from_storage(x[rows], ws["w_gate"], ws["w_up"], ws["w_down"],
                                                       ws["s_gate"], ws["s_up"], ws["s_down"], return_codes=True)
    ag, ar = oracle.bf16_bits_to_f64(a_gpu), oracle.bf16_bits_to_f64(steps["a_bits"])
    mag = np.maximum(np.abs(ag), np.abs(ar))
    ulp = np.where(mag > 0, 2.0 ** (np.floor(np.log2(np.where(mag > 0, mag, 1.0))) - 7), 0.0)
    # near-zero elements (gate sums that cancel) carry the sums' absolute error instead
    floor = A_ABS_FLOOR * np.sqrt(np.mean(ar ** 2))
    assert np.all(np.abs(ag - ar) <= np.maximum(ulp, floor)), "A differs by more than one bf16 step"
    e_a = float(np.mean(ag != ar))
    pg = p.cpu().numpy()[rows].astype(np.float64)
    e_p = oracle.rms_normalised_max_error(pg, ref)
    r_p = float(np.sqrt(np.mean((pg - ref) ** 2)) / np.sqrt(np.mean(ref ** 2)))
    print("w8a8 M=%d h=%d I_s=%d: A differing %.2e, P max %.3e, P rms %.2e" % (M, h, I_s, e_a, e_p, r_p),
          flush=True)
    return e_a, e_p, r_p, p


@pytest.mark.parametrize("M,h,I_s", [
    (1, 512, 384),
    (37, 1024, 768),
    (256, 512, 384),
    (300, 1024, 640),
    (1024, 2048, 1536),
    (300, 4096, 2048),     # gate/up tiles cut along K in 2 stream-K pieces (32 k-tiles of 128)
])
def test_w8a8_forward_shapes(M, h, I_s):
    x, ws = make_case(93, M, h, I_s, "bf16", "e4m3fn", 0.05, 0.05, weight_set=M)
    e_a, e_p, r_p, _ = _w8a8_errors(x, ws, M, h, I_s, 2)
    assert e_a <= A_DIFF_FRACTION, e_a
    assert e_p <= TOL_W8A8_P and r_p <= TOL_W8A8_RMS, (e_p, r_p)


def test_w8a8_config4_prefill_sampled():
    """70B-shaped TP=4 rank with fp8 weights at 2048 tokens, sampled rows (the
    per-token steps make rows independent)."""
    c = workloads.CONFIGS[4]
    h, I_s, M = c["h"], c["I"] // c["t"], 2048
    x, ws = make_case(4, M, h, I_s, "bf16", "e4m3fn", c["std_gu"], c["std_down"])
    rows = np.sort(np.concatenate([[0, M - 1], np.random.Generator(np.random.PCG64(5)).choice(M - 2, 30,
                                                                                               replace=False) + 1]))
    e_a, e_p, r_p, p = _w8a8_errors(x, ws, M, h, I_s, c["t"], rows)
    assert e_a <= A_DIFF_FRACTION, e_a
    assert e_p <= TOL_W8A8_P and r_p <= TOL_W8A8_RMS, (e_p, r_p)
    # against the fp8-weight (bf16 activation) forward: the activation quantisation's own effect
    d = upload_case(x, ws, "bf16", "e4m3fn")
    p16 = tp.shard_forward(d["x"], d["w_gate"], d["w_up"], d["w_down"], t=c["t"], k=0, s_gate=d["s_gate"],
                           s_up=d["s_up"], s_down=d["s_down"])
    torch.cuda.synchronize()
    print("w8a8 vs w8a16 rms-normalised max difference: %.4f" % oracle.rms_normalised_max_error(
        p.cpu().numpy()[rows], p16.cpu().numpy()[rows].astype(np.float64)), flush=True)


def test_w8a8_deterministic_and_k_independent():
    M, h, I_s = 300, 1024, 640
    x, ws = make_case(94, M, h, I_s, "bf16", "e4m3fn", 0.05, 0.05)
    d = upload_case(x, ws, "bf16", "e4m3fn")
    kw = dict(s_gate=d["s_gate"], s_up=d["s_up"], s_down=d["s_down"], t=2)
    a = tp.shard_forward_w8a8(d["x"], d["w_gate"], d["w_up"], d["w_down"], k=0, **kw)
    b = tp.shard_forward_w8a8(d["x"], d["w_gate"], d["w_up"], d["w_down"], k=1, **kw)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
