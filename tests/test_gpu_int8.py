"""int8 weights (W8A16) on the GPU: the MLP shard forward and the attention
projections with int8 codes and fp32 per-row scales, against the oracle on
the dequantised weights (the planner's int8 mode at one byte per parameter,
"Build a model sharding system for serving 70B+ parameter models",
scalablesystem.dev)."""

import numpy as np
import pytest
import torch

import oracle
import tensor_transformer_mlp_tp_amd as tp
import workloads
from helpers import TOL_INT8, make_case, upload_case, oracle_partial, to_device

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,h,I_s", [
    (1, 512, 512),      # decode, streaming kernels (K multiple of 256)
    (9, 1024, 768),
    (16, 512, 1280),
    (30, 512, 512),     # activation-staged path
    (64, 1024, 512),
    (5, 320, 192),      # K not a multiple of 256: register-batch kernels
    (40, 320, 448),
    (65, 512, 320),     # prefill, ragged tiles
    (300, 1024, 768),
])
def test_int8_forward_shapes(M, h, I_s):
    print("int8 forward M=%d h=%d I_s=%d" % (M, h, I_s), flush=True)
    x, ws = make_case(91, M, h, I_s, "bf16", "int8", 0.05, 0.05, weight_set=M)
    d = upload_case(x, ws, "bf16", "int8")
    assert d["w_gate"].dtype == torch.int8
    p = tp.shard_forward(d["x"], d["w_gate"], d["w_up"], d["w_down"], t=2, k=1, s_gate=d["s_gate"],
                         s_up=d["s_up"], s_down=d["s_down"])
    torch.cuda.synchronize()
    err = oracle.rms_normalised_max_error(p.cpu().numpy(), oracle_partial(x, ws, "bf16", "int8"))
    assert err <= TOL_INT8, err


@pytest.mark.parametrize("M", [1, 8, 2048])
def test_llama70b_tp2_int8(M):
    """70B-shaped TP=2 rank with int8 weights (I_s = 14336): decode and
    prefill, every element."""
    c = workloads.CONFIGS[9]
    h, I_s = c["h"], c["I"] // c["t"]
    print("int8 70B TP=2 M=%d" % M, flush=True)
    x, ws = make_case(9, M, h, I_s, "bf16", "int8", c["std_gu"], c["std_down"])
    d = upload_case(x, ws, "bf16", "int8")
    p = tp.shard_forward(d["x"], d["w_gate"], d["w_up"], d["w_down"], t=c["t"], k=0, s_gate=d["s_gate"],
                         s_up=d["s_up"], s_down=d["s_down"])
    torch.cuda.synchronize()
    err = oracle.rms_normalised_max_error(p.cpu().numpy(), oracle_partial(x, ws, "bf16", "int8"))
    assert err <= TOL_INT8, err


@pytest.mark.parametrize("M", [1, 24, 64, 200])
def test_int8_attention_projections(M):
    h, nh, nkv, d, t = 2048, 16, 4, 64, 2
    n_loc, k_o = workloads.attn_widths(nh, nkv, d, t)
    print("int8 attention M=%d" % M, flush=True)
    ws = workloads.make_attn_weights(92, h, n_loc, k_o, 0, "int8", 0.05, weight_set=M)
    x = workloads.make_x(92, M, h, "bf16", weight_set=M)
    o = workloads.make_attn_out_input(92, M, k_o, "bf16", weight_set=M)
    q = tp.attn_qkv_forward(to_device(x, "bf16"), to_device(ws["w_qkv"], "int8"), n_heads=nh, n_kv_heads=nkv,
                            head_dim=d, t=t, k=0, s_qkv=torch.from_numpy(ws["s_qkv"]).cuda())
    p = tp.attn_out_forward(to_device(o, "bf16"), to_device(ws["w_o"], "int8"), n_heads=nh, head_dim=d, t=t, k=0,
                            s_o=torch.from_numpy(ws["s_o"]).cuda())
    torch.cuda.synchronize()
    q_bits = q.view(torch.int16).cpu().numpy().view(np.uint16)
    e_q = oracle.rms_normalised_max_error(oracle.bf16_bits_to_f64(q_bits),
                                          oracle.linear_from_storage(x, "bf16", ws["w_qkv"], "int8", ws["s_qkv"]))
    e_p = oracle.rms_normalised_max_error(p.cpu().numpy(),
                                          oracle.linear_from_storage(o, "bf16", ws["w_o"], "int8", ws["s_o"]))
    assert e_q <= TOL_INT8, e_q
    assert e_p <= TOL_INT8, e_p


@pytest.mark.parametrize("M", [1, 64, 256])
def test_int8_codes_widen_exactly(M):
    """Every int8 code reaches the products exactly: the output projection of
    one-hot token rows (token m selects input column c_m) against a weight
    whose 256 columns hold every code, unit scales: each output is the code
    itself, bit for bit (decode and prefill kernels)."""
    nh, d, t, h = 4, 64, 1, 64                        # K = 256 input columns, 64 output rows
    K = nh // t * d
    codes = np.arange(256, dtype=np.uint8)
    w = np.stack([np.roll(codes, 5 * n) for n in range(h)])            # h x K, every code in every row
    cols = (np.arange(M) * 37) % K
    o = np.zeros((M, K), np.uint16)
    o[np.arange(M), cols] = 0x3F80                                     # bf16 1.0
    p = tp.attn_out_forward(torch.from_numpy(o.view(np.int16)).view(torch.bfloat16).cuda(),
                            torch.from_numpy(w).view(torch.int8).cuda(), n_heads=nh, head_dim=d, t=t, k=0,
                            s_o=torch.ones(h, dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    want = oracle.int8_to_f64(w)[:, cols].T                            # M x h
    assert np.array_equal(p.cpu().numpy().astype(np.float64), want)
