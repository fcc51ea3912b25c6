"""Attention-block projections on the GPU (tp_attn_qkv_forward,
tp_attn_out_forward) against the oracle: the column-parallel QKV projection
of a rank's heads and the row-parallel output projection's fp32 partial
(TPAttentionBlock, "The Tensor-Parallel Shard Group", scalablesystem.dev)."""

import numpy as np
import pytest
import torch

import oracle
import tensor_transformer_mlp_tp_amd as tp
import workloads
from helpers import TOL_BF16, TOL_FP8, to_device

pytestmark = pytest.mark.gpu


def _bits(t):
    """bf16 device tensor -> numpy uint16 bits."""
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _out_f64(t):
    if t.dtype == torch.bfloat16:
        return oracle.bf16_bits_to_f64(_bits(t))
    return t.cpu().numpy().astype(np.float64)


def _scales(s):
    return None if s is None else torch.from_numpy(s).cuda()


def _tol(w):
    return TOL_FP8 if w == "e4m3fn" else TOL_BF16


def test_tiny_t4_ranks_reassemble_unsplit():
    """Config tiny_attn_t4 (fp32): every rank's QKV columns reassemble the
    unsharded Q, K, V (KV heads replicated over two ranks each), and the
    ranks' output-projection partials, summed by the library's fixed-order
    reduce, give the unsharded O W_o^T."""
    c = workloads.ATTN_CONFIGS[8]
    M, h, nh, nkv, d, t = c["M"][0], c["h"], c["n_heads"], c["n_kv_heads"], c["head_dim"], c["t"]
    full = workloads.make_attn_full_weights(8, h, nh, nkv, d, "f32", c["std_w"])
    x = workloads.make_x(8, M, h, "f32")
    o = workloads.make_attn_out_input(8, M, nh * d, "f32")
    xd, od = to_device(x, "f32"), to_device(o, "f32")
    q_loc = nh // t
    qs, ks, vs, parts = [], [], [], []
    for k in range(t):
        wq = np.ascontiguousarray(oracle.qkv_rank_weight(full["w_q"], full["w_k"], full["w_v"], nh, nkv, d, t, k))
        out = tp.attn_qkv_forward(xd, to_device(wq, "f32"), n_heads=nh, n_kv_heads=nkv, head_dim=d, t=t, k=k)
        out = out.cpu().numpy().astype(np.float64)
        qs.append(out[:, :q_loc * d])
        ks.append(out[:, q_loc * d:(q_loc + 1) * d])
        vs.append(out[:, (q_loc + 1) * d:])
        wo = np.ascontiguousarray(oracle.o_proj_rank_weight(full["w_o"], nh, d, t, k))
        parts.append(tp.attn_out_forward(od[:, k * q_loc * d:(k + 1) * q_loc * d].contiguous(),
                                         to_device(wo, "f32"), n_heads=nh, head_dim=d, t=t, k=k))
    q_ref = oracle.linear(x, full["w_q"])
    k_ref = oracle.linear(x, full["w_k"])
    v_ref = oracle.linear(x, full["w_v"])
    assert oracle.rms_normalised_max_error(np.concatenate(qs, 1), q_ref) <= 1e-5
    rep = t // nkv
    for k in range(t):
        j = k // rep
        assert oracle.rms_normalised_max_error(ks[k], k_ref[:, j * d:(j + 1) * d]) <= 1e-5
        assert oracle.rms_normalised_max_error(vs[k], v_ref[:, j * d:(j + 1) * d]) <= 1e-5
    y = tp.partial_reduce(parts)
    torch.cuda.synchronize()
    err = oracle.rms_normalised_max_error(y.cpu().numpy(), oracle.linear(o, full["w_o"]))
    assert err <= 1e-5, err


# (M, h, n_heads, n_kv_heads, head_dim, t, w): decode sizes (register and
# streaming kernels), prefill sizes with ragged tiles, replicated KV heads.
QKV_CASES = [
    (1, 512, 8, 2, 64, 2, "bf16"),
    (5, 512, 8, 2, 64, 2, "bf16"),
    (17, 512, 8, 8, 64, 4, "bf16"),
    (33, 320, 8, 2, 64, 4, "bf16"),       # h % 128 != 0: register-batch kernels; KV replicated
    (64, 1024, 16, 4, 32, 2, "bf16"),
    (300, 512, 8, 2, 64, 2, "bf16"),      # prefill, ragged M and N tiles (K too short to split)
    (1000, 4096, 8, 2, 64, 2, "bf16"),    # prefill, 8 tiles, each cut along K in 4 stream-K pieces
    (130, 2048, 16, 4, 64, 4, "e4m3fn"),  # prefill with fp8 weights, 2 tiles in 2 pieces: the row scale after the sum
    (520, 384, 12, 4, 64, 4, "bf16"),
    (3, 1024, 8, 2, 64, 2, "e4m3fn"),
    (40, 320, 8, 2, 64, 2, "e4m3fn"),     # fp8 register-batch path
    (257, 1024, 8, 2, 64, 2, "e4m3fn"),
    (4, 4096, 8, 2, 64, 2, "bf16"),       # narrow output, long h: h split in 4 ranges, the last one adds them
    (9, 4096, 8, 2, 64, 2, "bf16"),
    (12, 8192, 64, 8, 128, 8, "bf16"),    # 70B TP=8 QKV width at 12 tokens: split, one token block
    (2, 8192, 4, 4, 32, 4, "bf16"),       # n_loc = 96: h split in 8 ranges
    (40, 4096, 8, 2, 64, 2, "bf16"),      # activation-staged kernels, h split in 8 ranges
    (16, 4096, 8, 2, 64, 2, "e4m3fn"),    # fp8, h split in 2 ranges
    (64, 2048, 4, 4, 32, 4, "bf16"),      # n_loc = 96, h split in 4 ranges
    (1, 4096, 8, 2, 64, 2, "bf16"),       # one or two tokens, a narrow output the streams would split:
    (2, 16384, 32, 8, 128, 4, "bf16"),    # the row-streaming kernel (whole rows per wave, no split);
    (1, 2048, 16, 4, 64, 4, "bf16"),      # K = 16384 is its largest
    (3, 8192, 64, 8, 128, 8, "bf16"),     # 3, 5, 8 tokens of the 70B TP=8 QKV: split streams
    (5, 8192, 64, 8, 128, 8, "bf16"),
    (8, 8192, 64, 8, 128, 8, "bf16"),
    (8, 16384, 32, 8, 128, 4, "bf16"),
]


@pytest.mark.parametrize("M,h,nh,nkv,d,t,w", QKV_CASES)
def test_qkv_shapes(M, h, nh, nkv, d, t, w):
    print("qkv M=%d h=%d heads=%d/%d d=%d t=%d w=%s workspace=%d" % (
        M, h, nh, nkv, d, t, w, tp.attn_qkv_workspace_bytes(M, h, nh, nkv, d, t, torch.bfloat16,
                                                            torch.float8_e4m3fn if w == "e4m3fn" else torch.bfloat16)),
        flush=True)
    n_loc, _ = workloads.attn_widths(nh, nkv, d, t)
    ws = workloads.make_attn_weights(61, h, n_loc, 64, 1, w, 0.05, weight_set=M)
    x = workloads.make_x(61, M, h, "bf16", weight_set=M)
    out = tp.attn_qkv_forward(to_device(x, "bf16"), to_device(ws["w_qkv"], w), n_heads=nh, n_kv_heads=nkv,
                              head_dim=d, t=t, k=1, s_qkv=_scales(ws["s_qkv"]))
    torch.cuda.synchronize()
    assert out.shape == (M, n_loc) and out.dtype == torch.bfloat16
    ref = oracle.linear_from_storage(x, "bf16", ws["w_qkv"], w, ws["s_qkv"])
    err = oracle.rms_normalised_max_error(_out_f64(out), ref)
    assert err <= _tol(w), err


# (M, h, n_heads, head_dim, t, w)
OUT_CASES = [
    (1, 512, 8, 64, 2, "bf16"),
    (9, 256, 8, 32, 4, "bf16"),           # K = 64: one register step
    (64, 512, 16, 64, 4, "bf16"),
    (48, 320, 12, 32, 2, "bf16"),         # K = 192: register-batch kernels
    (130, 512, 8, 64, 2, "bf16"),
    (700, 640, 16, 64, 8, "bf16"),
    (2, 512, 8, 64, 2, "e4m3fn"),
    (200, 1024, 8, 64, 2, "e4m3fn"),
]


@pytest.mark.parametrize("M,h,nh,d,t,w", OUT_CASES)
def test_out_proj_shapes(M, h, nh, d, t, w):
    print("o_proj M=%d h=%d heads=%d d=%d t=%d w=%s" % (M, h, nh, d, t, w), flush=True)
    k_o = nh // t * d
    ws = workloads.make_attn_weights(62, h, 16, k_o, 0, w, 0.05, weight_set=M)
    o = workloads.make_attn_out_input(62, M, k_o, "bf16", weight_set=M)
    p = tp.attn_out_forward(to_device(o, "bf16"), to_device(ws["w_o"], w), n_heads=nh, head_dim=d, t=t, k=0,
                            s_o=_scales(ws["s_o"]))
    torch.cuda.synchronize()
    assert p.shape == (M, h) and p.dtype == torch.float32
    ref = oracle.linear_from_storage(o, "bf16", ws["w_o"], w, ws["s_o"])
    err = oracle.rms_normalised_max_error(p.cpu().numpy(), ref)
    assert err <= _tol(w), err


@pytest.mark.parametrize("cid,M", [(6, 1), (6, 8), (6, 64), (6, 4096), (7, 32), (7, 2048)])
def test_llama70b_attention_projections(cid, M):
    """Full 70B-shaped rank (TP=8 bf16, TP=4 fp8): QKV and output projection
    against the oracle on every element."""
    c = workloads.ATTN_CONFIGS[cid]
    h, nh, nkv, d, t, w = c["h"], c["n_heads"], c["n_kv_heads"], c["head_dim"], c["t"], c["w"]
    print("attn70b config %d M=%d" % (cid, M), flush=True)
    n_loc, k_o = workloads.attn_widths(nh, nkv, d, t)
    ws = workloads.make_attn_weights(cid, h, n_loc, k_o, 0, w, c["std_w"])
    x = workloads.make_x(cid, M, h, "bf16")
    o = workloads.make_attn_out_input(cid, M, k_o, "bf16")
    qkv = tp.attn_qkv_forward(to_device(x, "bf16"), to_device(ws["w_qkv"], w), n_heads=nh, n_kv_heads=nkv,
                              head_dim=d, t=t, k=0, s_qkv=_scales(ws["s_qkv"]))
    p = tp.attn_out_forward(to_device(o, "bf16"), to_device(ws["w_o"], w), n_heads=nh, head_dim=d, t=t, k=0,
                            s_o=_scales(ws["s_o"]))
    torch.cuda.synchronize()
    ref_q = oracle.linear_from_storage(x, "bf16", ws["w_qkv"], w, ws["s_qkv"])
    ref_p = oracle.linear_from_storage(o, "bf16", ws["w_o"], w, ws["s_o"])
    e_q = oracle.rms_normalised_max_error(_out_f64(qkv), ref_q)
    e_p = oracle.rms_normalised_max_error(p.cpu().numpy(), ref_p)
    assert e_q <= _tol(w), e_q
    assert e_p <= _tol(w), e_p


def test_k_independence_determinism_and_strided_weight():
    """The rank index selects no data; repeated calls give the same bits; the
    output projection reading its column block out of the full W_o (ldw =
    n_heads * head_dim) gives the same bits as a contiguous copy."""
    M, h, nh, nkv, d, t = 24, 512, 8, 2, 64, 2
    n_loc, k_o = workloads.attn_widths(nh, nkv, d, t)
    ws = workloads.make_attn_weights(63, h, n_loc, k_o, 0, "bf16", 0.05)
    x = to_device(workloads.make_x(63, M, h, "bf16"), "bf16")
    wq = to_device(ws["w_qkv"], "bf16")
    a = tp.attn_qkv_forward(x, wq, n_heads=nh, n_kv_heads=nkv, head_dim=d, t=t, k=0)
    b = tp.attn_qkv_forward(x, wq, n_heads=nh, n_kv_heads=nkv, head_dim=d, t=t, k=1)
    c = tp.attn_qkv_forward(x, wq, n_heads=nh, n_kv_heads=nkv, head_dim=d, t=t, k=0)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(a.view(torch.int16), c.view(torch.int16))

    full_o = torch.randn((h, nh * d), device="cuda").to(torch.bfloat16)
    o = torch.randn((M, k_o), device="cuda").to(torch.bfloat16)
    for k in range(t):
        view = full_o[:, k * k_o:(k + 1) * k_o]
        assert view.stride(0) == nh * d
        p_view = tp.attn_out_forward(o, view, n_heads=nh, head_dim=d, t=t, k=k)
        p_copy = tp.attn_out_forward(o, view.contiguous(), n_heads=nh, head_dim=d, t=t, k=k)
        torch.cuda.synchronize()
        assert torch.equal(p_view.view(torch.int32), p_copy.view(torch.int32))


def test_prepared_calls_in_a_graph():
    """Prepared projection calls replayed from a captured HIP graph give the
    eager result on every replay."""
    M, h, nh, nkv, d, t = 8, 1024, 16, 4, 64, 4
    n_loc, k_o = workloads.attn_widths(nh, nkv, d, t)
    ws = workloads.make_attn_weights(64, h, n_loc, k_o, 0, "bf16", 0.05)
    x = to_device(workloads.make_x(64, M, h, "bf16"), "bf16")
    o = to_device(workloads.make_attn_out_input(64, M, k_o, "bf16"), "bf16")
    wq, wo = to_device(ws["w_qkv"], "bf16"), to_device(ws["w_o"], "bf16")
    eager_q = tp.attn_qkv_forward(x, wq, n_heads=nh, n_kv_heads=nkv, head_dim=d, t=t, k=0)
    eager_p = tp.attn_out_forward(o, wo, n_heads=nh, head_dim=d, t=t, k=0)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        cq = tp.prepare_attn_qkv_forward(x, wq, n_heads=nh, n_kv_heads=nkv, head_dim=d, t=t, k=0, stream=s)
        cp = tp.prepare_attn_out_forward(o, wo, n_heads=nh, head_dim=d, t=t, k=0, stream=s)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            cq()
            cp()
    for _ in range(3):
        cq.out.zero_()
        cp.partial.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(cq.out.view(torch.int16), eager_q.view(torch.int16))
        assert torch.equal(cp.partial.view(torch.int32), eager_p.view(torch.int32))


def test_split_workspace_reuse_and_dirty_contents():
    """One workspace serves calls of different sizes; what it holds on entry
    does not change the result (decode: the split sums overwrite it; prefill:
    the stream-K counters are cleared by the call)."""
    h, nh, nkv, d, t = 8192, 64, 8, 128, 8
    n_loc, _ = workloads.attn_widths(nh, nkv, d, t)
    ws = workloads.make_attn_weights(65, h, n_loc, 64, 0, "bf16", 0.02)
    wq = to_device(ws["w_qkv"], "bf16")
    need = max(tp.attn_qkv_workspace_bytes(M, h, nh, nkv, d, t) for M in (1, 8, 64, 1000))
    assert need > 0
    scratch = tp.alloc_workspace(need, "cuda")
    for M in (64, 1, 1000, 8):
        x = to_device(workloads.make_x(65, M, h, "bf16", weight_set=M), "bf16")
        kw = dict(n_heads=nh, n_kv_heads=nkv, head_dim=d, t=t, k=0)
        scratch.fill_(0x7F)                      # fp32 words of 3.4e38
        a = tp.attn_qkv_forward(x, wq, workspace=scratch, **kw)
        scratch.fill_(0)
        b = tp.attn_qkv_forward(x, wq, workspace=scratch, **kw)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), M
        ref = oracle.linear_from_storage(workloads.make_x(65, M, h, "bf16", weight_set=M), "bf16", ws["w_qkv"], "bf16")
        assert oracle.rms_normalised_max_error(_out_f64(a), ref) <= TOL_BF16
