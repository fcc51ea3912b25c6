"""Host-only checks of the C ABI: the library loads, exports every declared
symbol, and rejects invalid arguments before enqueuing anything.

Every forward / reduce call in this file is invalid by construction (the
pointer values are never dereferenced because validation fails first), so it
is safe on a machine with or without a GPU.
"""

import ctypes
import os
import re

import pytest

import tensor_transformer_mlp_tp_amd as tp
from tensor_transformer_mlp_tp_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    txt = open(os.path.join(ROOT, "include", "tp_mlp.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(tp_[a-z0-9_]+)\s*\(", txt)))


def test_header_declares_expected_api():
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTED_SYMBOLS), names


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    for name in declared_functions():
        assert hasattr(lib, name), name
    # and the dynamic symbol table has nothing else public from us
    out = os.popen("nm -D --defined-only %s" % _lib.LIB_PATH).read()
    ours = sorted(set(re.findall(r"\b(tp_[a-z0-9_]+)\b", out)))
    assert ours == declared_functions()


def test_status_strings_and_kinds():
    lib = _lib.load()
    for s in range(5):
        assert lib.tp_status_string(s).startswith(b"TP_")
    assert lib.tp_status_string(99) == b"unknown status"
    kinds = tp.kernel_kinds()
    assert "gateup_decode" in kinds and "partial_reduce" in kinds
    assert lib.tp_kernel_kind_name(-1) is None
    assert lib.tp_kernel_kind_name(len(kinds)) is None


BF16, F32, FP8 = _lib.TP_BF16, _lib.TP_F32, _lib.TP_FP8_E4M3FN


SLOT = 256 * 256 * 4   # one stream-K piece's fp32 sums of a 256 x 256 tile
SLOT64 = 64 * 256 * 4  # ... of a 64-token tile
SLOT128 = 128 * 256 * 4


def test_workspace_bytes():
    lib = _lib.load()
    # A = M x I_s bf16, rounded up to 256 bytes
    assert lib.tp_mlp_workspace_bytes(1, 8192, 28672, 8, BF16, BF16) == 3584 * 2
    assert lib.tp_mlp_workspace_bytes(3, 64, 128, 2, BF16, FP8) == 512          # 3*64*2 = 384 -> 512
    assert lib.tp_mlp_workspace_bytes(5, 64, 128, 2, BF16, BF16) == 768         # 5*64*2 = 640 -> 768
    assert lib.tp_mlp_workspace_bytes(16, 256, 1024, 4, F32, F32) == 16 * 256 * 4
    # bf16 prefill adds the stream-K scratch of its GEMMs (pieces in one round of 256 CUs).
    # 405B TP=8 at 8192 tokens: gate/up 32 x 52 = 1664 tiles, the last 128 in 2 pieces of 128
    # k-tiles (counters: 512 bytes); down 32 x 64 = 2048 tiles, whole rounds
    assert lib.tp_mlp_workspace_bytes(8192, 16384, 53248, 8, BF16, BF16) == 8192 * 6656 * 2 + 512 + 256 * SLOT
    # 70B TP=8 at 4096 tokens: 448 gate/up tiles, 192 past the first round (2 pieces each would
    # take two rounds); at 2048 tokens 224 tiles (one round, a split saves under an eighth of it)
    assert lib.tp_mlp_workspace_bytes(4096, 8192, 28672, 8, BF16, BF16) == 4096 * 3584 * 2
    assert lib.tp_mlp_workspace_bytes(2048, 8192, 28672, 8, BF16, BF16) == 2048 * 3584 * 2
    # just above the decode range the tiles are 64 tokens high: 2 x 28 gate/up tiles of 128
    # k-tiles cut in 4 pieces (counters: 256 bytes), the larger of the two GEMMs' scratch
    assert lib.tp_mlp_workspace_bytes(65, 8192, 28672, 8, BF16, BF16) == 65 * 3584 * 2 + 256 + 224 * SLOT64
    # one-byte weights leave the decode kernels above 32 tokens: at 48, 28 gate/up tiles in 5
    # pieces; bf16 weights stay on them (A only up to 48 tokens)
    assert lib.tp_mlp_workspace_bytes(48, 8192, 28672, 8, BF16, FP8) == 48 * 3584 * 2 + 256 + 140 * SLOT64
    assert lib.tp_mlp_workspace_bytes(48, 8192, 28672, 8, BF16, _lib.TP_INT8) == 48 * 3584 * 2 + 256 + 140 * SLOT64
    assert lib.tp_mlp_workspace_bytes(48, 8192, 28672, 8, BF16, BF16) == 48 * 3584 * 2
    assert lib.tp_mlp_workspace_bytes(16, 8192, 28672, 8, BF16, FP8) == 16 * 3584 * 2
    # decode split-K streams (bf16 at 49-64 tokens, one-byte weights at 17-32): arrival counters
    # (one per tile, 256-byte rounded) and a slot of fp32 fragments (1 KB each) per tile and K
    # range, the larger of the two GEMMs: gate/up tiles of 7 waves x 1 block (112 rows), down of
    # 4 waves x 2 blocks (128 rows).  70B TP = 8, 64 tokens: gate/up 64 tiles x 4 ranges of 28 KB,
    # down 64 tiles x 4 ranges of 32 KB
    assert lib.tp_mlp_workspace_bytes(64, 8192, 28672, 8, BF16, BF16) == 64 * 3584 * 2 + 256 + 64 * 4 * 32768
    # fp8 TP = 4, 32 tokens: gate/up 128 tiles x 2 ranges of 14 KB, down 64 tiles x 4 ranges of 16 KB
    assert lib.tp_mlp_workspace_bytes(32, 8192, 28672, 4, BF16, FP8) == 32 * 7168 * 2 + 512 + 64 * 4 * 16384
    assert lib.tp_mlp_workspace_bytes(32, 8192, 28672, 4, BF16, _lib.TP_INT8) == 32 * 7168 * 2 + 512 + 64 * 4 * 16384
    # fp8 TP = 8, 32 tokens: gate/up 64 tiles x 4 ranges, down 64 x 4
    assert lib.tp_mlp_workspace_bytes(32, 8192, 28672, 8, BF16, FP8) == 32 * 3584 * 2 + 256 + 64 * 4 * 16384
    # 600 tokens, h = I_s = 2048: gate/up in 128-token tiles (5 x 16, 2 pieces each: counters 512
    # bytes, slots of 128 x 256 fp32), down in 64-token tiles (10 x 8, 2 pieces each)
    assert lib.tp_mlp_workspace_bytes(600, 2048, 4096, 2, BF16, BF16) == 600 * 2048 * 2 + 512 + 160 * SLOT128
    # invalid arguments give 0
    assert lib.tp_mlp_workspace_bytes(1, 8192, 28672, 5, BF16, BF16) == 0       # I % t
    assert lib.tp_mlp_workspace_bytes(0, 8192, 28672, 8, BF16, BF16) == 0
    assert lib.tp_mlp_workspace_bytes(1, 8192, 28672, 8, F32, BF16) == 0        # unsupported pair
    assert lib.tp_mlp_workspace_bytes(1, 100, 28672, 8, BF16, BF16) == 0        # h % 64
    assert lib.tp_mlp_workspace_bytes(3, 64, 128, 2, BF16, _lib.TP_INT8) == 512
    assert lib.tp_mlp_workspace_bytes(3, 64, 128, 2, _lib.TP_INT8, _lib.TP_INT8) == 0
    assert lib.tp_mlp_workspace_bytes(3, 64, 128, 2, BF16, 9) == 0              # unknown code


P = 0x10000  # a 256-byte aligned fake address; never dereferenced (every call fails validation)


def fwd(M=1, h=128, I=256, t=2, k=0, act=BF16, w=BF16, x=P, wg=P * 2, wu=P * 3, wd=P * 4,
        ldx=None, ldgu=None, ldd=None, sg=None, su=None, sd=None, p=P * 8, ldp=None, ws=P * 16,
        wsb=1 << 20):
    lib = _lib.load()
    I_s = I // t if t else 1
    return lib.tp_mlp_shard_forward(M, h, I, t, k, act, w, x, ldx if ldx is not None else h,
                                    wg, wu, ldgu if ldgu is not None else h, wd,
                                    ldd if ldd is not None else I_s, sg, su, sd, p,
                                    ldp if ldp is not None else h, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(I=255), _lib.TP_ERR_INVALID_ARG),                 # I_full % t != 0
    (dict(k=2), _lib.TP_ERR_INVALID_ARG),                   # k >= t
    (dict(k=-1), _lib.TP_ERR_INVALID_ARG),
    (dict(t=0), _lib.TP_ERR_INVALID_ARG),
    (dict(t=65, I=65 * 64), _lib.TP_ERR_INVALID_ARG),
    (dict(M=0), _lib.TP_ERR_INVALID_ARG),
    (dict(h=0), _lib.TP_ERR_INVALID_ARG),
    (dict(x=None), _lib.TP_ERR_INVALID_ARG),
    (dict(wd=None), _lib.TP_ERR_INVALID_ARG),
    (dict(p=None), _lib.TP_ERR_INVALID_ARG),
    (dict(act=7), _lib.TP_ERR_INVALID_ARG),
    (dict(act=F32, w=BF16), _lib.TP_ERR_UNSUPPORTED),
    (dict(act=FP8, w=FP8), _lib.TP_ERR_UNSUPPORTED),
    (dict(w=FP8), _lib.TP_ERR_INVALID_ARG),                 # fp8 without scales
    (dict(w=_lib.TP_INT8), _lib.TP_ERR_INVALID_ARG),        # int8 without scales
    (dict(act=_lib.TP_INT8, w=_lib.TP_INT8), _lib.TP_ERR_UNSUPPORTED),
    (dict(act=F32, w=_lib.TP_INT8), _lib.TP_ERR_UNSUPPORTED),
    (dict(sg=P, su=P, sd=P), _lib.TP_ERR_INVALID_ARG),      # scales with bf16 weights
    (dict(ldx=64), _lib.TP_ERR_INVALID_ARG),                # ld < row length
    (dict(ldd=64), _lib.TP_ERR_INVALID_ARG),
    (dict(ldp=100), _lib.TP_ERR_INVALID_ARG),
    (dict(h=96), _lib.TP_ERR_UNSUPPORTED),                  # h % 64
    (dict(I=2 * 96), _lib.TP_ERR_UNSUPPORTED),              # I_s % 64
    (dict(wsb=10), _lib.TP_ERR_WORKSPACE),
    (dict(ws=None), _lib.TP_ERR_WORKSPACE),
    (dict(M=300, h=2112, I=4224, wsb=300 * 2112 * 2), _lib.TP_ERR_WORKSPACE),   # A only: the prefill's
                                                                                # stream-K scratch is missing
    (dict(x=P + 2), _lib.TP_ERR_UNSUPPORTED),               # misaligned
    (dict(ldx=132), _lib.TP_ERR_UNSUPPORTED),               # rows not 16-byte aligned
    (dict(ws=P * 16 + 16), _lib.TP_ERR_UNSUPPORTED),        # workspace not 256-aligned
    (dict(p=P * 2), _lib.TP_ERR_INVALID_ARG),               # partial aliases w_gate
    (dict(ws=P * 8), _lib.TP_ERR_INVALID_ARG),              # workspace aliases partial
    (dict(ws=P), _lib.TP_ERR_INVALID_ARG),                  # workspace aliases x
])
def test_forward_rejects(kw, status):
    lib = _lib.load()
    assert fwd(**kw) == status
    assert lib.tp_last_error() not in (b"", None)


def reduce_call(n, t, ptrs, out):
    lib = _lib.load()
    arr = None if ptrs is None else (ctypes.c_void_p * len(ptrs))(*ptrs)
    return lib.tp_partial_reduce(n, t, arr, out, None)


@pytest.mark.parametrize("n,t,ptrs,out,status", [
    (-1, 2, [P, P * 2], P * 4, _lib.TP_ERR_INVALID_ARG),
    (16, 0, [P], P * 4, _lib.TP_ERR_INVALID_ARG),
    (16, 65, [P] * 65, P * 4, _lib.TP_ERR_INVALID_ARG),
    (16, 2, None, P * 4, _lib.TP_ERR_INVALID_ARG),
    (16, 2, [P, P * 2], None, _lib.TP_ERR_INVALID_ARG),
    (16, 2, [P, None], P * 4, _lib.TP_ERR_INVALID_ARG),
    (16, 2, [P + 4, P * 2], P * 4, _lib.TP_ERR_UNSUPPORTED),
    (16, 2, [P, P * 2], P * 4 + 4, _lib.TP_ERR_UNSUPPORTED),
    (16, 2, [P, P * 2], P * 2, _lib.TP_ERR_INVALID_ARG),        # out aliases partials[1]
    (16, 2, [P, P * 2], P + 16, _lib.TP_ERR_INVALID_ARG),       # partial overlap with partials[0]
])
def test_reduce_rejects(n, t, ptrs, out, status):
    assert reduce_call(n, t, ptrs, out) == status


def test_reduce_empty_is_noop():
    # n == 0 passes validation and launches nothing
    assert reduce_call(0, 2, [P, P * 2], P * 4) == _lib.TP_OK
    assert reduce_call(0, 1, [P], P) == _lib.TP_OK
    assert reduce_call(0, 3, None, None) == _lib.TP_OK
    # t is still validated
    assert reduce_call(0, 0, None, None) == _lib.TP_ERR_INVALID_ARG


def fwd_sp(blocks, M=4, h=128, I=256, t=2, k=0, ldx=None, **kw):
    lib = _lib.load()
    I_s = I // t if t else 1
    arr = None if blocks is None else (ctypes.c_void_p * len(blocks))(*blocks)
    return lib.tp_mlp_shard_forward_sp(M, h, I, t, k, BF16, BF16, arr, ldx if ldx is not None else h,
                                       P * 2, P * 3, h, P * 4, I_s, None, None, None, kw.get("p", P * 8), h,
                                       kw.get("ws", P * 16), 1 << 20, None)


@pytest.mark.parametrize("blocks,kw,status", [
    (None, {}, _lib.TP_ERR_INVALID_ARG),                           # no block array
    ([P, None], {}, _lib.TP_ERR_INVALID_ARG),                      # a null block
    ([P, P * 32], dict(M=5), _lib.TP_ERR_INVALID_ARG),             # M % t
    ([P, P * 32], dict(t=0), _lib.TP_ERR_INVALID_ARG),
    ([P, P * 32], dict(k=2), _lib.TP_ERR_INVALID_ARG),
    ([P, P * 32 + 4], {}, _lib.TP_ERR_UNSUPPORTED),                # misaligned block
    ([P, P * 8], {}, _lib.TP_ERR_INVALID_ARG),                     # block overlaps the partial
    ([P, P * 16], {}, _lib.TP_ERR_INVALID_ARG),                    # block overlaps the workspace
])
def test_forward_sp_rejects(blocks, kw, status):
    assert fwd_sp(blocks, **kw) == status


def rs_call(rows, row_len, t, k, ptrs, out):
    lib = _lib.load()
    arr = None if ptrs is None else (ctypes.c_void_p * len(ptrs))(*ptrs)
    return lib.tp_partial_reduce_scatter(rows, row_len, t, k, arr, out, None)


@pytest.mark.parametrize("rows,row_len,t,k,ptrs,out,status", [
    (8, 16, 0, 0, [P], P * 4, _lib.TP_ERR_INVALID_ARG),
    (8, 16, 2, 2, [P, P * 2], P * 4, _lib.TP_ERR_INVALID_ARG),         # k >= t
    (8, 16, 2, -1, [P, P * 2], P * 4, _lib.TP_ERR_INVALID_ARG),
    (9, 16, 2, 0, [P, P * 2], P * 4, _lib.TP_ERR_INVALID_ARG),         # rows % t
    (8, 16, 2, 0, None, P * 4, _lib.TP_ERR_INVALID_ARG),
    (8, 16, 2, 0, [P, None], P * 4, _lib.TP_ERR_INVALID_ARG),
    (4, 3, 2, 0, [P, P * 2], P * 4, _lib.TP_ERR_UNSUPPORTED),          # rows/t * row_len % 4
    (8, 16, 2, 1, [P, P * 2], P * 2 + 64 * 4, _lib.TP_ERR_INVALID_ARG),  # out = rank 1's slice of partials[1]
])
def test_reduce_scatter_rejects(rows, row_len, t, k, ptrs, out, status):
    assert rs_call(rows, row_len, t, k, ptrs, out) == status


def test_reduce_scatter_empty_is_noop():
    assert rs_call(0, 16, 2, 1, [P, P * 2], P * 4) == _lib.TP_OK
    assert rs_call(8, 0, 2, 1, None, None) == _lib.TP_ERR_INVALID_ARG   # the array is checked first


# ------------------------------------------------------------- attention

def test_attn_qkv_width():
    lib = _lib.load()
    assert lib.tp_attn_qkv_width(64, 8, 128, 8) == (8 + 2) * 128       # 70B at TP = 8
    assert lib.tp_attn_qkv_width(64, 8, 128, 16) == (4 + 2) * 128      # KV heads replicated
    assert lib.tp_attn_qkv_width(64, 8, 128, 1) == (64 + 16) * 128
    assert lib.tp_attn_qkv_width(64, 8, 128, 3) == -1                  # 64 % 3
    assert lib.tp_attn_qkv_width(64, 8, 128, 128) == -1                # t above 64 / above the heads
    assert lib.tp_attn_qkv_width(48, 6, 128, 4) == -1                  # 6 KV heads, t = 4: neither divides
    assert lib.tp_attn_qkv_width(64, 6, 128, 2) == -1                  # 64 % 6: groups not whole
    assert lib.tp_attn_qkv_width(64, 8, 0, 8) == -1


def qkv_call(M=1, h=128, nh=8, nkv=2, d=32, t=2, k=0, act=BF16, w=BF16, x=P, ldx=None, wq=P * 2, ldw=None,
             s=None, out=P * 8, ldq=None, ws=None, wsb=0):
    lib = _lib.load()
    n_loc = lib.tp_attn_qkv_width(nh, nkv, d, t) if t > 0 else 16
    n_loc = max(int(n_loc), 16)
    return lib.tp_attn_qkv_forward(M, h, nh, nkv, d, t, k, act, w, x, ldx if ldx is not None else h, wq,
                                   ldw if ldw is not None else h, s, out, ldq if ldq is not None else n_loc,
                                   ws, wsb, None)


def test_attn_qkv_workspace_bytes():
    lib = _lib.load()
    # 70B TP=8 decode: at one or two tokens the row-streaming kernel needs no scratch
    for M in (1, 2):
        assert lib.tp_attn_qkv_workspace_bytes(M, 8192, 64, 8, 128, 8, BF16, BF16) == 0
    # above, the 1280-wide output over h = 8192 is split along h: one arrival counter per tile
    # of 16 RB rows (256-byte rounded), then a 1 KB fp32 fragment per 16-row block, 16-token
    # block, tile and range
    for M in (3, 8, 9, 16, 32, 64):
        b = lib.tp_attn_qkv_workspace_bytes(M, 8192, 64, 8, 128, 8, BF16, BF16)
        nt = (M + 15) // 16
        assert b % 256 == 0
        assert b >= 256 + 1280 // 16 * nt * 1024 * 2          # at least two ranges of every block
    # M = 8: tiles of one 16-row block (80 tiles: 512 bytes of counters), 4 ranges of h
    assert lib.tp_attn_qkv_workspace_bytes(8, 8192, 64, 8, 128, 8, BF16, BF16) == 512 + 80 * 4 * 1024
    # fp8 weights keep the split at M = 1
    assert lib.tp_attn_qkv_workspace_bytes(1, 8192, 64, 8, 128, 8, BF16, FP8) > 0
    # prefill: 80 tiles of 256 x 256 for 4096 tokens, fewer than the 256 CUs: every tile is cut
    # along K into 3 stream-K pieces (128 k-tiles of 64), each with a 256 x 256 fp32 slot, plus
    # 80 arrival counters rounded to 512 bytes
    assert lib.tp_attn_qkv_workspace_bytes(4096, 8192, 64, 8, 128, 8, BF16, BF16) == 512 + 240 * SLOT
    assert lib.tp_attn_qkv_workspace_bytes(16, 256, 8, 2, 32, 4, F32, F32) == 0          # fp32 path
    assert lib.tp_attn_qkv_workspace_bytes(1, 8192, 64, 8, 128, 3, BF16, BF16) == 0      # invalid split
    assert lib.tp_attn_qkv_workspace_bytes(0, 8192, 64, 8, 128, 8, BF16, BF16) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(nh=6, nkv=4), _lib.TP_ERR_INVALID_ARG),   # 6 % 4: KV groups not whole
    (dict(nh=9, nkv=3, t=2), _lib.TP_ERR_INVALID_ARG),  # 9 % 2
    (dict(nkv=3, nh=9, t=6), _lib.TP_ERR_INVALID_ARG),
    (dict(t=0), _lib.TP_ERR_INVALID_ARG),
    (dict(k=2), _lib.TP_ERR_INVALID_ARG),
    (dict(M=0), _lib.TP_ERR_INVALID_ARG),
    (dict(d=0), _lib.TP_ERR_INVALID_ARG),
    (dict(x=None), _lib.TP_ERR_INVALID_ARG),
    (dict(out=None), _lib.TP_ERR_INVALID_ARG),
    (dict(w=FP8), _lib.TP_ERR_INVALID_ARG),         # fp8 without scales
    (dict(s=P * 4), _lib.TP_ERR_INVALID_ARG),       # scales with bf16 weights
    (dict(act=F32, w=BF16), _lib.TP_ERR_UNSUPPORTED),
    (dict(w=_lib.TP_INT8), _lib.TP_ERR_INVALID_ARG),  # int8 without scales
    (dict(h=96), _lib.TP_ERR_UNSUPPORTED),          # h % 64
    (dict(d=36), _lib.TP_ERR_UNSUPPORTED),          # n_loc = 216, not a multiple of 16
    (dict(ldx=64), _lib.TP_ERR_INVALID_ARG),
    (dict(ldq=100), _lib.TP_ERR_INVALID_ARG),
    (dict(x=P + 2), _lib.TP_ERR_UNSUPPORTED),
    (dict(ldw=132), _lib.TP_ERR_UNSUPPORTED),
    (dict(out=P * 2 + 64), _lib.TP_ERR_INVALID_ARG),   # output overlaps the weight
    (dict(out=P), _lib.TP_ERR_INVALID_ARG),            # output overlaps x
    (dict(M=64, h=8192, nh=64, nkv=8, d=128, t=8, wq=P * 1024, out=P * 4096), _lib.TP_ERR_WORKSPACE),
    (dict(M=64, h=8192, nh=64, nkv=8, d=128, t=8, wq=P * 1024, out=P * 4096, ws=P * 8192, wsb=256),
     _lib.TP_ERR_WORKSPACE),                           # too small
    (dict(M=64, h=8192, nh=64, nkv=8, d=128, t=8, wq=P * 1024, out=P * 4096, ws=P * 8192 + 16, wsb=1 << 26),
     _lib.TP_ERR_UNSUPPORTED),                         # workspace not 256-aligned
    (dict(M=64, h=8192, nh=64, nkv=8, d=128, t=8, wq=P * 1024, out=P * 4096, ws=P * 1024, wsb=1 << 26),
     _lib.TP_ERR_INVALID_ARG),                         # workspace overlaps the weight
])
def test_attn_qkv_rejects(kw, status):
    lib = _lib.load()
    # every case must fail validation: a valid one would launch on fake addresses
    assert status != _lib.TP_OK
    assert qkv_call(**kw) == status
    assert lib.tp_last_error() not in (b"", None)


def oproj_call(M=1, h=128, nh=8, d=32, t=2, k=0, act=BF16, w=BF16, a=P, lda=None, wo=P * 2, ldw=None,
               s=None, p=P * 8, ldp=None):
    lib = _lib.load()
    K = nh // t * d if t > 0 and nh % t == 0 else 64
    return lib.tp_attn_out_forward(M, h, nh, d, t, k, act, w, a, lda if lda is not None else K, wo,
                                   ldw if ldw is not None else K, s, p, ldp if ldp is not None else h, None)


@pytest.mark.parametrize("kw,status", [
    (dict(nh=6, t=4), _lib.TP_ERR_INVALID_ARG),     # 6 % 4
    (dict(t=0), _lib.TP_ERR_INVALID_ARG),
    (dict(k=-1), _lib.TP_ERR_INVALID_ARG),
    (dict(h=0), _lib.TP_ERR_INVALID_ARG),
    (dict(a=None), _lib.TP_ERR_INVALID_ARG),
    (dict(w=FP8), _lib.TP_ERR_INVALID_ARG),
    (dict(d=24), _lib.TP_ERR_UNSUPPORTED),          # K = 96, not a multiple of 64
    (dict(h=120), _lib.TP_ERR_UNSUPPORTED),         # h % 16
    (dict(lda=64 + 32, d=48), _lib.TP_ERR_INVALID_ARG),  # lda < K = 192
    (dict(ldp=64), _lib.TP_ERR_INVALID_ARG),
    (dict(p=P * 8 + 4), _lib.TP_ERR_UNSUPPORTED),
    (dict(p=P), _lib.TP_ERR_INVALID_ARG),           # partial overlaps the input
])
def test_attn_out_rejects(kw, status):
    assert oproj_call(**kw) == status


# ------------------------------------------------------------- W8A8

def w8a8_call(M=256, h=128, I=256, t=2, k=0, x=P, wg=P * 2, wu=P * 3, wd=P * 4, sg=P * 5, su=P * 5 + 1024,
              sd=P * 5 + 2048, p=P * 8, ws=P * 16, wsb=1 << 22, ldx=None):
    lib = _lib.load()
    I_s = I // t if t else 1
    return lib.tp_mlp_shard_forward_w8a8(M, h, I, t, k, x, ldx if ldx is not None else h, wg, wu, h, wd, I_s,
                                         sg, su, sd, p, h, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(h=192), _lib.TP_ERR_UNSUPPORTED),            # h % 128
    (dict(I=2 * 192), _lib.TP_ERR_UNSUPPORTED),        # I_s % 128
    (dict(I=255), _lib.TP_ERR_INVALID_ARG),
    (dict(k=2), _lib.TP_ERR_INVALID_ARG),
    (dict(sg=None), _lib.TP_ERR_INVALID_ARG),
    (dict(x=None), _lib.TP_ERR_INVALID_ARG),
    (dict(wsb=100), _lib.TP_ERR_WORKSPACE),
    (dict(ws=P * 16 + 16), _lib.TP_ERR_UNSUPPORTED),
    (dict(x=P + 2), _lib.TP_ERR_UNSUPPORTED),
    (dict(ldx=64), _lib.TP_ERR_INVALID_ARG),
    (dict(p=P * 2), _lib.TP_ERR_INVALID_ARG),          # partial overlaps a weight
    (dict(ws=P), _lib.TP_ERR_INVALID_ARG),             # workspace overlaps x
])
def test_w8a8_rejects(kw, status):
    assert status != _lib.TP_OK
    assert w8a8_call(**kw) == status


def test_w8a8_workspace_bytes():
    lib = _lib.load()
    # A bf16 + X codes + scales + A codes + scales, each rounded to 256 bytes, then the stream-K
    # scratch: gate/up has 16 x 56 = 896 tiles of 64 k-tiles (128 wide), the last 128 cut in 2
    M, h, I_s = 4096, 8192, 7168
    want = M * I_s * 2 + M * h + M * 4 + M * I_s + M * 4 + 512 + 256 * SLOT
    assert lib.tp_mlp_w8a8_workspace_bytes(M, h, I_s * 4, 4) == want
    assert lib.tp_mlp_w8a8_workspace_bytes(M, 192, 1024, 4) == 0


@pytest.mark.parametrize("args,status", [
    ((4, 12, P, 12, P * 2, 16, P * 3), _lib.TP_ERR_UNSUPPORTED),    # cols % 8
    ((4, 16, P, 8, P * 2, 16, P * 3), _lib.TP_ERR_INVALID_ARG),     # ldx < cols
    ((4, 16, None, 16, P * 2, 16, P * 3), _lib.TP_ERR_INVALID_ARG),
    ((4, 16, P + 2, 16, P * 2, 16, P * 3), _lib.TP_ERR_UNSUPPORTED),
    ((4, 16, P, 16, P + 8, 16, P * 3), _lib.TP_ERR_INVALID_ARG),    # codes overlap x
    ((-1, 16, P, 16, P * 2, 16, P * 3), _lib.TP_ERR_INVALID_ARG),
])
def test_quantize_rows_rejects(args, status):
    lib = _lib.load()
    assert lib.tp_quantize_rows_e4m3(*args, None) == status


def test_quantize_rows_empty_is_noop():
    assert _lib.load().tp_quantize_rows_e4m3(0, 16, None, 16, None, 16, None, None) == _lib.TP_OK


def test_packed_workspace_bytes():
    lib = _lib.load()
    pw = lib.tp_mlp_packed_workspace_bytes
    # decode sizes: the same workspace as the row-major forward
    for M, w in ((1, BF16), (8, BF16), (64, BF16), (32, FP8), (16, _lib.TP_INT8)):
        assert pw(M, 8192, 28672, 8, w) == lib.tp_mlp_workspace_bytes(M, 8192, 28672, 8, BF16, w)
    # above them (bf16 only) 256-token tiles: at 65 tokens of the 70B TP = 8 shard, 28 gate/up
    # tiles of 128 k-tiles cut in 5 pieces (counters: 256 bytes) of 256 x 256 fp32 slots
    assert pw(65, 8192, 28672, 8, BF16) == 65 * 3584 * 2 + 256 + 28 * 5 * SLOT
    # 4096 tokens: 448 gate/up tiles (192 past the first round, kept whole), 512 down tiles
    assert pw(4096, 8192, 28672, 8, BF16) == 4096 * 3584 * 2
    assert pw(8192, 16384, 53248, 8, BF16) == lib.tp_mlp_workspace_bytes(8192, 16384, 53248, 8, BF16, BF16)
    # one-byte weights above 32 tokens: the packed-weight GEMMs (4096 x 7168 fp8: 448 gate/up tiles,
    # 192 past the first round, kept whole; 256 down tiles)
    assert pw(2048, 8192, 28672, 4, FP8) == 2048 * 7168 * 2
    assert pw(33, 8192, 28672, 4, FP8) > pw(32, 8192, 28672, 4, FP8) > 0
    assert pw(1, 320, 640, 2, BF16) == 0               # h % 128: not packable
    assert pw(0, 512, 1024, 2, BF16) == 0


def test_packed_weights_bytes_and_validation():
    lib = _lib.load()
    # the three matrices' bytes: 70B TP=8 bf16, TP=4 fp8
    assert lib.tp_mlp_packed_weights_bytes(8192, 28672, 8, BF16) == 3 * 3584 * 8192 * 2
    assert lib.tp_mlp_packed_weights_bytes(8192, 28672, 4, FP8) == 3 * 7168 * 8192
    assert lib.tp_mlp_packed_weights_bytes(512, 1024, 2, _lib.TP_INT8) == 3 * 512 * 512
    assert lib.tp_mlp_packed_weights_bytes(320, 512, 2, BF16) == 0          # h % 128
    assert lib.tp_mlp_packed_weights_bytes(512, 768, 2, FP8) == 0           # I_s = 384: % 256
    assert lib.tp_mlp_packed_weights_bytes(512, 1024, 2, F32) == 0          # fp32 weights
    # forward: bf16 activations; one-byte weights at decode sizes only; checked before any HIP call
    def fwdp(M=1, h=512, I=1024, t=2, act=BF16, w=BF16, packed=P, nbytes=1 << 24, sc=None, wsb=1 << 20):
        return lib.tp_mlp_shard_forward_packed(M, h, I, t, 0, act, w, P, h, packed, nbytes, sc, sc, sc, P * 8, h,
                                               P * 16, wsb, None)
    # bf16 weights above the decode sizes take the packed prefill kernels, which need the
    # workspace of tp_mlp_packed_workspace_bytes (A and the stream-K scratch)
    need = lib.tp_mlp_packed_workspace_bytes(65, 512, 1024, 2, BF16)
    assert need >= 65 * 512 * 2
    assert fwdp(M=65, wsb=need - 1) == _lib.TP_ERR_WORKSPACE
    need8 = lib.tp_mlp_packed_workspace_bytes(33, 512, 1024, 2, FP8)
    assert fwdp(M=33, w=FP8, sc=P, wsb=need8 - 1) == _lib.TP_ERR_WORKSPACE
    assert fwdp(act=F32, w=F32) == _lib.TP_ERR_UNSUPPORTED
    assert fwdp(packed=None) == _lib.TP_ERR_INVALID_ARG
    assert fwdp(w=FP8) == _lib.TP_ERR_INVALID_ARG                            # scales missing
    assert fwdp(h=320) == _lib.TP_ERR_UNSUPPORTED
    # an array packed for smaller shapes (3 * 512 * 512 bf16 bytes needed)
    assert fwdp(nbytes=3 * 512 * 512 * 2 - 16) == _lib.TP_ERR_INVALID_ARG
    # pack: invalid shapes, null pointers, short leading dimensions, a short array
    assert lib.tp_mlp_pack_weights(512, 1024, 0, BF16, P, P * 2, 512, P * 3, 512, P * 8, 1 << 22, None) == \
        _lib.TP_ERR_INVALID_ARG
    assert lib.tp_mlp_pack_weights(320, 640, 2, BF16, P, P * 2, 320, P * 3, 320, P * 8, 1 << 22, None) == \
        _lib.TP_ERR_UNSUPPORTED
    assert lib.tp_mlp_pack_weights(512, 1024, 2, BF16, None, P, 512, P, 512, P * 8, 1 << 22, None) == \
        _lib.TP_ERR_INVALID_ARG
    assert lib.tp_mlp_pack_weights(512, 1024, 2, BF16, P, P * 2, 256, P * 3, 512, P * 8, 1 << 22, None) == \
        _lib.TP_ERR_INVALID_ARG
    assert lib.tp_mlp_pack_weights(512, 1024, 2, BF16, P, P * 2, 512, P * 3, 512, P * 64, 1024, None) == \
        _lib.TP_ERR_INVALID_ARG


# ---- binding: scale vectors must have one element per output row (the C ABI
# takes no length, so the binding is the only place a short vector is caught)

def _cpu_fp8_shard(M=4, h=256, I_s=128):
    import torch
    x = torch.zeros((M, h), dtype=torch.bfloat16)
    wg = torch.zeros((I_s, h), dtype=torch.float8_e4m3fn)
    wu = torch.zeros((I_s, h), dtype=torch.float8_e4m3fn)
    wd = torch.zeros((h, I_s), dtype=torch.float8_e4m3fn)
    return x, wg, wu, wd


@pytest.mark.parametrize("which,n", [("s_gate", 127), ("s_up", 129), ("s_down", 255), ("s_down", 128)])
def test_binding_rejects_scale_lengths(which, n):
    import torch
    import tensor_transformer_mlp_tp_amd as tp
    x, wg, wu, wd = _cpu_fp8_shard()
    sc = {"s_gate": torch.ones(128), "s_up": torch.ones(128), "s_down": torch.ones(256)}
    sc[which] = torch.ones(n)
    with pytest.raises(ValueError, match=which):
        tp.prepare_shard_forward(x, wg, wu, wd, t=2, k=0, **sc)
    with pytest.raises(ValueError, match=which):
        tp.prepare_shard_forward_w8a8(x, wg, wu, wd, t=2, k=0, **sc)


def test_binding_rejects_packed_scale_lengths():
    import torch
    import tensor_transformer_mlp_tp_amd as tp
    x = torch.zeros((4, 512), dtype=torch.bfloat16)
    pk = tp.PackedWeights(torch.zeros(3 * 512 * 256, dtype=torch.uint8), 512, 256, 2, _lib.TP_FP8_E4M3FN)
    with pytest.raises(ValueError, match="s_down"):
        tp.prepare_shard_forward_packed(x, pk, k=0, s_gate=torch.ones(256), s_up=torch.ones(256),
                                        s_down=torch.ones(256))
    with pytest.raises(ValueError, match="s_gate"):
        tp.prepare_shard_forward_packed(x, pk, k=0, s_gate=torch.ones(512), s_up=torch.ones(256),
                                        s_down=torch.ones(512))


def test_binding_rejects_attention_scale_lengths():
    import torch
    import tensor_transformer_mlp_tp_amd as tp
    n_loc = tp.attn_qkv_width(8, 2, 32, 2)          # (4 + 2*1) * 32 = 192
    x = torch.zeros((4, 256), dtype=torch.bfloat16)
    w = torch.zeros((n_loc, 256), dtype=torch.float8_e4m3fn)
    with pytest.raises(ValueError, match="s_qkv"):
        tp.prepare_attn_qkv_forward(x, w, n_heads=8, n_kv_heads=2, head_dim=32, t=2, k=0,
                                    s_qkv=torch.ones(n_loc - 1))
    o = torch.zeros((4, 128), dtype=torch.bfloat16)
    wo = torch.zeros((256, 128), dtype=torch.float8_e4m3fn)
    with pytest.raises(ValueError, match="s_o"):
        tp.prepare_attn_out_forward(o, wo, n_heads=8, head_dim=32, t=2, k=0, s_o=torch.ones(128))
