"""Packed weights: the layout, and the packed forward (decode streams, and
the packed-weight MFMA GEMMs above the decode sizes) against the row-major
forward (bit-identical where both sum in the same order) and the oracle."""
import numpy as np
import pytest
import torch

import oracle
import tensor_transformer_mlp_tp_amd as tp
from tensor_transformer_mlp_tp_amd import _lib
from helpers import TOL_BF16, TOL_FP8, TOL_INT8, make_case, upload_case, oracle_partial

pytestmark = pytest.mark.gpu

TOL = {"bf16": TOL_BF16, "e4m3fn": TOL_FP8, "int8": TOL_INT8}


def host_packed(ws, I_s, h):
    """The packed array written out from its documented layout: each 16-row
    block is a run of 1 KB MFMA A fragments, fragment st giving lane l the
    16 bytes [64 st + 16 (l // 16), +16) of row l % 16; gate/up blocks of 8
    gate then 8 up rows, then down blocks of 16 rows; rows past the end
    repeat the last one."""
    def rows_bytes(a):
        a = np.ascontiguousarray(a)
        return a.view(np.uint8).reshape(a.shape[0], -1)

    g, u, d = rows_bytes(ws["w_gate"]), rows_bytes(ws["w_up"]), rows_bytes(ws["w_down"])
    lane = np.arange(64)

    def blocks(src_of_row, nblk):
        parts = []
        for b in range(nblk):
            src = src_of_row(b)                  # (16, row bytes)
            nfrag = src.shape[1] // 64
            seg = src.reshape(16, nfrag, 4, 16)  # row, fragment, 16-byte chunk, byte
            parts.append(seg[lane % 16, :, lane // 16, :].transpose(1, 0, 2).reshape(-1))
        return np.concatenate(parts)

    gu = blocks(lambda b: np.concatenate([g[np.minimum(8 * b + np.arange(8), I_s - 1)],
                                          u[np.minimum(8 * b + np.arange(8), I_s - 1)]]), (I_s + 7) // 8)
    dn = blocks(lambda b: d[np.minimum(16 * b + np.arange(16), h - 1)], (h + 15) // 16)
    return np.concatenate([gu, dn])


@pytest.mark.parametrize("w,h,I_s", [("bf16", 256, 384), ("e4m3fn", 512, 256), ("int8", 256, 512)])
def test_pack_layout(w, h, I_s):
    t = 2
    print("pack layout w=%s h=%d I_s=%d" % (w, h, I_s), flush=True)
    x, ws = make_case(60, 1, h, I_s, "bf16", w, 0.05, 0.05)
    d = upload_case(x, ws, "bf16", w)
    pk = tp.pack_weights(d["w_gate"], d["w_up"], d["w_down"], t=t)
    torch.cuda.synchronize()
    assert pk.data.numel() == tp.packed_weights_bytes(h, I_s * t, t, d["w_gate"].dtype)
    assert np.array_equal(pk.data.cpu().numpy(), host_packed(ws, I_s, h))


CASES = [(M, w) for w in ("bf16", "e4m3fn", "int8") for M in (1, 2, 5, 16, 17, 32, 33, 48, 64)]


@pytest.mark.parametrize("M,w", CASES)
def test_packed_forward_small(M, w):
    # h = 512, I_s = 512: 64 gate/up blocks, 32 down blocks, 2 to 4 slots per wave
    h, I_s, t, k = 512, 512, 2, 1
    print("packed forward M=%d w=%s" % (M, w), flush=True)
    x, ws = make_case(61, M, h, I_s, "bf16", w, 0.05, 0.05, k=k, weight_set=M)
    d = upload_case(x, ws, "bf16", w)
    pk = tp.pack_weights(d["w_gate"], d["w_up"], d["w_down"], t=t)
    p = tp.shard_forward_packed(d["x"], pk, k=k, s_gate=d["s_gate"], s_up=d["s_up"], s_down=d["s_down"])
    ref = tp.shard_forward(d["x"], d["w_gate"], d["w_up"], d["w_down"], t=t, k=k, s_gate=d["s_gate"],
                           s_up=d["s_up"], s_down=d["s_down"])
    torch.cuda.synchronize()
    if w == "bf16" or M <= 32:     # the decode streams, on either layout
        assert torch.equal(p.view(torch.int32), ref.view(torch.int32))
    err = oracle.rms_normalised_max_error(p.cpu().numpy(), oracle_partial(x, ws, "bf16", w))
    print("  err=%.3e" % err, flush=True)
    assert err <= TOL[w]


@pytest.mark.parametrize("M", [1, 8, 64])
def test_packed_forward_70b(M):
    """70B TP = 8 shard (h = 8192, I_s = 3584), the decode sizes of the bench."""
    h, I_s, t = 8192, 3584, 8
    print("packed forward 70B M=%d" % M, flush=True)
    x, ws = make_case(2, M, h, I_s, "bf16", "bf16", 0.02, 0.02, weight_set=M)
    d = upload_case(x, ws, "bf16", "bf16")
    pk = tp.pack_weights(d["w_gate"], d["w_up"], d["w_down"], t=t)
    p = tp.shard_forward_packed(d["x"], pk, k=0)
    ref = tp.shard_forward(d["x"], d["w_gate"], d["w_up"], d["w_down"], t=t, k=0)
    torch.cuda.synchronize()
    assert torch.equal(p.view(torch.int32), ref.view(torch.int32))
    err = oracle.rms_normalised_max_error(p.cpu().numpy(), oracle_partial(x, ws, "bf16", "bf16"))
    assert err <= TOL_BF16


def test_packed_rejects():
    h, I_s, t = 256, 512, 2
    x, ws = make_case(62, 33, h, I_s, "bf16", "e4m3fn", 0.05, 0.05)
    d = upload_case(x, ws, "bf16", "e4m3fn")
    pk = tp.pack_weights(d["w_gate"], d["w_up"], d["w_down"], t=t)
    with pytest.raises(_lib.TPError, match="s_gate"):      # one-byte weights need their scales
        tp.shard_forward_packed(d["x"], pk, k=0)
    small = tp.alloc_workspace(1024, "cuda")
    lib = _lib.load()
    st = lib.tp_mlp_pack_weights(h, I_s * t, t, _lib.TP_BF16, d["w_gate"].data_ptr(), d["w_up"].data_ptr(), h,
                                 d["w_down"].data_ptr(), I_s, small.data_ptr(), 1024, None)
    assert st == _lib.TP_ERR_INVALID_ARG                  # too small


# Packed prefill (bf16 weights above 64 tokens): 256 x 256 tiles with the
# weights read from the packed array straight into registers.  Shapes: ragged
# token tiles (M not a multiple of 256), a down GEMM whose last tile has only
# 8 of its 16 row blocks (h = 384), a single k-stage pair (h = 128), odd
# stage counts, and stream-K tails.
PREFILL_CASES = [(65, 256, 128), (300, 384, 256), (513, 512, 384), (257, 128, 128), (1024, 640, 640),
                 (600, 1024, 1152)]


@pytest.mark.parametrize("M,h,I_s", PREFILL_CASES)
def test_packed_prefill_shapes(M, h, I_s):
    t, k = 2, 1
    print("packed prefill M=%d h=%d I_s=%d" % (M, h, I_s), flush=True)
    x, ws = make_case(63, M, h, I_s, "bf16", "bf16", 0.05, 0.05, k=k, weight_set=M)
    d = upload_case(x, ws, "bf16", "bf16")
    pk = tp.pack_weights(d["w_gate"], d["w_up"], d["w_down"], t=t)
    p = tp.shard_forward_packed(d["x"], pk, k=k)
    p2 = tp.shard_forward_packed(d["x"], pk, k=k)
    torch.cuda.synchronize()
    assert torch.equal(p.view(torch.int32), p2.view(torch.int32))       # deterministic
    err = oracle.rms_normalised_max_error(p.cpu().numpy(), oracle_partial(x, ws, "bf16", "bf16"))
    print("  err=%.3e" % err, flush=True)
    assert err <= TOL_BF16


@pytest.mark.parametrize("M,h,I_s", [(2304, 2048, 3712), (4096, 8192, 3584)])
def test_packed_prefill_matches_row_major(M, h, I_s):
    """Where both forwards use 256-token tiles and the same stream-K plan they
    add the same products in the same order: the partials are bit-identical.
    2304 x 2048 x 3712 has stream-K tails in both GEMMs (gate/up 261 tiles,
    down 72 tiles in 3 pieces); 4096 x 8192 x 3584 is the 70B TP = 8 prefill.
    Every element is also checked against the oracle on a third of the rows
    of every 256-token tile."""
    t = 8
    print("packed prefill vs row-major M=%d h=%d I_s=%d" % (M, h, I_s), flush=True)
    x, ws = make_case(3, M, h, I_s, "bf16", "bf16", 0.02, 0.02, weight_set=M)
    d = upload_case(x, ws, "bf16", "bf16")
    pk = tp.pack_weights(d["w_gate"], d["w_up"], d["w_down"], t=t)
    nb = tp.packed_workspace_bytes(M, h, I_s * t, t)
    wsp = tp.alloc_workspace(nb, "cuda")
    wsp.fill_(0x7F)                                                     # a dirty workspace
    p = tp.shard_forward_packed(d["x"], pk, k=0, workspace=wsp)
    ref = tp.shard_forward(d["x"], d["w_gate"], d["w_up"], d["w_down"], t=t, k=0)
    torch.cuda.synchronize()
    assert torch.equal(p.view(torch.int32), ref.view(torch.int32))
    rows = np.concatenate([np.arange(m0, min(m0 + 256, M), 3) for m0 in range(0, M, 256)])
    err = oracle.rms_normalised_max_error(p.cpu().numpy()[rows], oracle_partial(x, ws, "bf16", "bf16", rows=rows))
    print("  err=%.3e" % err, flush=True)
    assert err <= TOL_BF16


# One-byte packed weights above 32 tokens: the packed-weight GEMMs widen each
# lane's 16 codes to bf16 in registers (k order differs from the row-major
# kernels', so the comparison with those is to the tolerance, not bitwise).
ONEBYTE_PREFILL_CASES = [(w, M, h, I_s) for w in ("e4m3fn", "int8")
                         for (M, h, I_s) in ((33, 256, 256), (300, 512, 768), (513, 768, 512), (1024, 256, 1280))]


@pytest.mark.parametrize("w,M,h,I_s", ONEBYTE_PREFILL_CASES)
def test_packed_prefill_onebyte(w, M, h, I_s):
    t, k = 4, 3
    print("packed prefill w=%s M=%d h=%d I_s=%d" % (w, M, h, I_s), flush=True)
    x, ws = make_case(64, M, h, I_s, "bf16", w, 0.05, 0.05, k=k, weight_set=M)
    d = upload_case(x, ws, "bf16", w)
    pk = tp.pack_weights(d["w_gate"], d["w_up"], d["w_down"], t=t)
    sc = dict(s_gate=d["s_gate"], s_up=d["s_up"], s_down=d["s_down"])
    p = tp.shard_forward_packed(d["x"], pk, k=k, **sc)
    p2 = tp.shard_forward_packed(d["x"], pk, k=k, **sc)
    torch.cuda.synchronize()
    assert torch.equal(p.view(torch.int32), p2.view(torch.int32))       # deterministic
    err = oracle.rms_normalised_max_error(p.cpu().numpy(), oracle_partial(x, ws, "bf16", w))
    print("  err=%.3e" % err, flush=True)
    assert err <= TOL[w]


def test_packed_prefill_fp8_config4():
    """70B TP = 4 shard with fp8 e4m3fn weights at M = 2048 (the fp8 prefill config):
    448 gate/up tiles and 256 down tiles on the packed-weight GEMMs; every row of
    every 256-token tile sampled (a third of the rows) against the oracle."""
    M, h, I_s, t = 2048, 8192, 7168, 4
    print("packed prefill fp8 M=%d h=%d I_s=%d" % (M, h, I_s), flush=True)
    x, ws = make_case(4, M, h, I_s, "bf16", "e4m3fn", 0.02, 0.02, weight_set=M)
    d = upload_case(x, ws, "bf16", "e4m3fn")
    pk = tp.pack_weights(d["w_gate"], d["w_up"], d["w_down"], t=t)
    wsp = tp.alloc_workspace(tp.packed_workspace_bytes(M, h, I_s * t, t, torch.float8_e4m3fn), "cuda")
    wsp.fill_(0x5A)                                                     # a dirty workspace
    p = tp.shard_forward_packed(d["x"], pk, k=0, s_gate=d["s_gate"], s_up=d["s_up"], s_down=d["s_down"],
                                workspace=wsp)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(p).all())
    rows = np.concatenate([np.arange(m0 + 1, min(m0 + 256, M), 3) for m0 in range(0, M, 256)])
    err = oracle.rms_normalised_max_error(p.cpu().numpy()[rows],
                                          oracle_partial(x, ws, "bf16", "e4m3fn", rows=rows))
    print("  err=%.3e" % err, flush=True)
    assert err <= TOL_FP8
