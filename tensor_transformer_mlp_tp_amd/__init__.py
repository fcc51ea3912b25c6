"""MI355X-native tensor-parallel MLP shard (Python binding of libtp_mlp.so).

One TP rank's share of a Llama-style MLP under the Megatron split and the
local fixed-order sum of the ranks' partials.  The functions below only
marshal torch tensors (device memory) and the current HIP stream into the C
ABI declared in ``include/tp_mlp.h``; the computation is entirely in the
library's HIP kernels.

    P_k = (SiLU(X W_gate_k^T) * (X W_up_k^T)) W_down_k^T      (shard_forward)
    Y   = (((P_0 + P_1) + P_2) + ...) + P_{t-1}              (partial_reduce)

and the attention block's two projections of the same rank:

    QKV_k = X W_qkv_k^T                                        (attn_qkv_forward)
    P_k   = O_k W_o_k^T                                        (attn_out_forward)
"""

import ctypes

import torch

from . import _lib
from ._lib import (TPError, TP_F32, TP_BF16, TP_FP8_E4M3FN, TP_INT8, EXPORTED_SYMBOLS,  # noqa: F401
                   LIB_PATH, load)

__all__ = ["shard_forward", "shard_forward_noalloc", "partial_reduce", "prepare_shard_forward", "prepare_partial_reduce",
           "shard_forward_sp", "prepare_shard_forward_sp", "partial_reduce_scatter",
           "prepare_partial_reduce_scatter", "attn_qkv_width", "attn_qkv_workspace_bytes", "attn_qkv_forward",
           "w8a8_workspace_bytes", "shard_forward_w8a8", "prepare_shard_forward_w8a8", "quantize_rows_e4m3", "prepare_attn_qkv_forward",
           "attn_out_forward", "prepare_attn_out_forward", "profile_reserve",
           "workspace_bytes", "alloc_workspace", "profile_enable", "profile_collect", "profile_durations", "kernel_kinds",
           "TPError", "load"]


def _act_code(dt):
    if dt == torch.bfloat16:
        return TP_BF16
    if dt == torch.float32:
        return TP_F32
    raise TypeError("activations must be bfloat16 or float32, got %s" % dt)


def _w_code(dt):
    if dt == torch.bfloat16:
        return TP_BF16
    if dt == torch.float32:
        return TP_F32
    if dt in (torch.float8_e4m3fn, torch.uint8):
        return TP_FP8_E4M3FN
    if dt == torch.int8:
        return TP_INT8
    raise TypeError("weights must be bfloat16, float32, float8_e4m3fn (uint8 codes) or int8, got %s" % dt)


def _check_matrix(name, t, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("%s must be a 2-D tensor with unit stride along its rows" % name)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream_of(device, stream):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def workspace_bytes(M, h, I_full, t, act_dtype=torch.bfloat16, w_dtype=torch.bfloat16):
    """Bytes of device workspace ``shard_forward`` needs (0 for invalid arguments)."""
    return int(_lib.load().tp_mlp_workspace_bytes(int(M), int(h), int(I_full), int(t),
                                                  _act_code(act_dtype), _w_code(w_dtype)))


def alloc_workspace(nbytes, device):
    """A 256-byte aligned uint8 view of at least ``nbytes`` device bytes."""
    raw = torch.empty(int(nbytes) + 256, dtype=torch.uint8, device=device)
    off = (-raw.data_ptr()) % 256
    return raw[off:off + int(nbytes)]


class PreparedCall:
    """A library call with its arguments marshalled once (for tight loops).

    Holds references to the tensors it points at; calling it re-issues the
    same C call on the same stream.
    """

    def __init__(self, fn, args, keep):
        self._fn, self._args, self._keep = fn, args, keep

    def __call__(self):
        status = self._fn(*self._args)
        if status != 0:
            _lib.check(status)


def shard_forward(x, w_gate, w_up, w_down, *, t, k, s_gate=None, s_up=None, s_down=None,
                  partial=None, workspace=None, stream=None):
    """Rank k's fp32 partial P_k (M x h) of the TP-MLP; see ``include/tp_mlp.h``.

    x: (M, h) bf16 or fp32.  w_gate, w_up: (I_s, h); w_down: (h, I_s), in the
    (out, in) layout, bf16 / fp32 / float8_e4m3fn (or uint8 codes) / int8.  For
    one-byte weights s_gate, s_up (I_s) and s_down (h) are the fp32 per-row
    scales.
    ``partial`` (M, h) fp32 and ``workspace`` (uint8, >= workspace_bytes) may be
    passed to avoid allocation.  Work is enqueued on ``stream`` (default: the
    current stream) and the call returns without waiting.
    """
    call = prepare_shard_forward(x, w_gate, w_up, w_down, t=t, k=k, s_gate=s_gate, s_up=s_up,
                                 s_down=s_down, partial=partial, workspace=workspace, stream=stream)
    call()
    return call.partial


def prepare_shard_forward(x, w_gate, w_up, w_down, *, t, k, s_gate=None, s_up=None, s_down=None,
                          partial=None, workspace=None, stream=None):
    """Validate and marshal a shard_forward once; returns a PreparedCall
    (attribute ``partial`` is the output tensor)."""
    return _prepare_forward([x], False, w_gate, w_up, w_down, t, k, s_gate, s_up, s_down, partial, workspace,
                            stream)


def shard_forward_noalloc(x, w_gate, w_up, w_down, *, t, k, s_gate=None, s_up=None, s_down=None, partial,
                          stream=None):
    """``shard_forward`` through the allocation-free entry point
    (``include/tp_mlp.h``: tp_mlp_shard_forward_noalloc): the library's
    static per-device scratch replaces the workspace, and ``partial`` (M, h)
    fp32 must be given, so the call allocates nothing.  Calls that overlap in
    time on one device race on that scratch."""
    device = x.device
    _check_matrix("x", x, device)
    for name, m in (("w_gate", w_gate), ("w_up", w_up), ("w_down", w_down)):
        _check_matrix(name, m, device)
    _check_matrix("partial", partial, device)
    M, h = x.shape
    I_s = w_gate.shape[0]
    wc = _w_code(w_gate.dtype)
    if _w_code(w_up.dtype) != wc or _w_code(w_down.dtype) != wc:
        raise TypeError("w_gate, w_up and w_down must share a dtype")
    if tuple(w_up.shape) != (I_s, h) or tuple(w_gate.shape) != (I_s, h) or tuple(w_down.shape) != (h, I_s):
        raise ValueError("shard shapes must be w_gate/w_up (I_s, h) and w_down (h, I_s)")
    if w_gate.stride(0) != w_up.stride(0):
        raise ValueError("w_gate and w_up must share a leading dimension")
    for name, s, n in (("s_gate", s_gate, I_s), ("s_up", s_up, I_s), ("s_down", s_down, h)):
        _check_scales(s, device, n, name)
    if partial.dtype != torch.float32 or tuple(partial.shape) != (M, h):
        raise ValueError("partial must be float32 of shape (%d, %d)" % (M, h))
    _lib.check(_lib.load().tp_mlp_shard_forward_noalloc(
        M, h, I_s * int(t), int(t), int(k), _act_code(x.dtype), wc, _ptr(x), x.stride(0), _ptr(w_gate), _ptr(w_up),
        w_gate.stride(0), _ptr(w_down), w_down.stride(0), _ptr(s_gate), _ptr(s_up), _ptr(s_down), _ptr(partial),
        partial.stride(0), _stream_of(device, stream)))
    return partial


def shard_forward_sp(x_blocks, w_gate, w_up, w_down, *, t, k, s_gate=None, s_up=None, s_down=None,
                     partial=None, workspace=None, stream=None):
    """shard_forward with X given as the t ranks' row blocks (sequence-parallel
    input, ``include/tp_mlp.h``: tp_mlp_shard_forward_sp): ``x_blocks`` is a
    sequence of t (M/t, h) tensors with one leading dimension; the result
    equals shard_forward on their row concatenation, bit for bit."""
    call = prepare_shard_forward_sp(x_blocks, w_gate, w_up, w_down, t=t, k=k, s_gate=s_gate, s_up=s_up,
                                    s_down=s_down, partial=partial, workspace=workspace, stream=stream)
    call()
    return call.partial


def prepare_shard_forward_sp(x_blocks, w_gate, w_up, w_down, *, t, k, s_gate=None, s_up=None, s_down=None,
                             partial=None, workspace=None, stream=None):
    """Marshal a shard_forward_sp once; returns a PreparedCall."""
    if len(x_blocks) != int(t):
        raise ValueError("need t = %d row blocks, got %d" % (int(t), len(x_blocks)))
    return _prepare_forward(list(x_blocks), True, w_gate, w_up, w_down, t, k, s_gate, s_up, s_down, partial,
                            workspace, stream)


def _prepare_forward(xs, sp, w_gate, w_up, w_down, t, k, s_gate, s_up, s_down, partial, workspace, stream):
    x0 = xs[0]
    device = x0.device
    for j, xb in enumerate(xs):
        _check_matrix("x" if not sp else "x_blocks[%d]" % j, xb, device)
        if xb.shape != x0.shape or xb.dtype != x0.dtype or xb.stride(0) != x0.stride(0):
            raise ValueError("row blocks must share shape, dtype and leading dimension")
    for name, m in (("w_gate", w_gate), ("w_up", w_up), ("w_down", w_down)):
        _check_matrix(name, m, device)
    M, h = x0.shape[0] * len(xs), x0.shape[1]
    I_s = w_gate.shape[0]
    I_full = I_s * int(t)
    act, wc = _act_code(x0.dtype), _w_code(w_gate.dtype)
    if _w_code(w_up.dtype) != wc or _w_code(w_down.dtype) != wc:
        raise TypeError("w_gate, w_up and w_down must share a dtype")
    if tuple(w_up.shape) != (I_s, h) or tuple(w_gate.shape) != (I_s, h) or tuple(w_down.shape) != (h, I_s):
        raise ValueError("shard shapes must be w_gate/w_up (I_s, h) and w_down (h, I_s); got %s %s %s"
                         % (tuple(w_gate.shape), tuple(w_up.shape), tuple(w_down.shape)))
    for name, s, n in (("s_gate", s_gate, I_s), ("s_up", s_up, I_s), ("s_down", s_down, h)):
        _check_scales(s, device, n, name)
    if partial is None:
        partial = torch.empty((M, h), dtype=torch.float32, device=device)
    else:
        _check_matrix("partial", partial, device)
        if partial.dtype != torch.float32 or tuple(partial.shape) != (M, h):
            raise ValueError("partial must be float32 of shape (%d, %d)" % (M, h))
    if w_gate.stride(0) != w_up.stride(0):
        raise ValueError("w_gate and w_up must share a leading dimension")
    lib = _lib.load()
    need = int(lib.tp_mlp_workspace_bytes(M, h, I_full, int(t), act, wc))
    if workspace is None:
        workspace = alloc_workspace(max(need, 1), device)
    elif workspace.device != device:
        raise ValueError("workspace must be on %s" % device)
    ws_bytes = workspace.numel() * workspace.element_size()
    if sp:
        xarg = (ctypes.c_void_p * len(xs))(*[xb.data_ptr() for xb in xs])
        fn = lib.tp_mlp_shard_forward_sp
    else:
        xarg, fn = _ptr(x0), lib.tp_mlp_shard_forward
    args = (M, h, I_full, int(t), int(k), act, wc,
            xarg, x0.stride(0), _ptr(w_gate), _ptr(w_up), w_gate.stride(0),
            _ptr(w_down), w_down.stride(0), _ptr(s_gate), _ptr(s_up), _ptr(s_down),
            _ptr(partial), partial.stride(0), _ptr(workspace), ws_bytes, _stream_of(device, stream))
    call = PreparedCall(fn, args, (list(xs), w_gate, w_up, w_down, s_gate, s_up, s_down, partial, workspace))
    call.partial = partial
    return call


class PackedWeights:
    """A rank's three weight matrices packed for the decode kernels
    (``tp_mlp_pack_weights``): ``data`` (uint8 on the weights' device) plus
    the shapes and dtype code it was packed for."""

    def __init__(self, data, h, I_s, t, w_code):
        self.data, self.h, self.I_s, self.t, self.w_code = data, h, I_s, t, w_code


def packed_weights_bytes(h, I_full, t, w_dtype=torch.bfloat16):
    return int(_lib.load().tp_mlp_packed_weights_bytes(h, I_full, t, _w_code(w_dtype)))


def pack_weights(w_gate, w_up, w_down, *, t, out=None, stream=None):
    """Pack one rank's (out, in) weights for ``shard_forward_packed``; the
    copy runs on the GPU, enqueued on ``stream``."""
    device = w_gate.device
    for name, m in (("w_gate", w_gate), ("w_up", w_up), ("w_down", w_down)):
        _check_matrix(name, m, device)
    I_s, h = w_gate.shape
    wc = _w_code(w_gate.dtype)
    if _w_code(w_up.dtype) != wc or _w_code(w_down.dtype) != wc:
        raise TypeError("w_gate, w_up and w_down must share a dtype")
    if tuple(w_up.shape) != (I_s, h) or tuple(w_down.shape) != (h, I_s) or w_gate.stride(0) != w_up.stride(0):
        raise ValueError("shard shapes must be w_gate/w_up (I_s, h) with one leading dimension and w_down (h, I_s)")
    lib = _lib.load()
    need = int(lib.tp_mlp_packed_weights_bytes(h, I_s * int(t), int(t), wc))
    if need == 0:
        _lib.check(_lib.TP_ERR_UNSUPPORTED)
    if out is None:
        out = alloc_workspace(need, device)
    _lib.check(lib.tp_mlp_pack_weights(h, I_s * int(t), int(t), wc, _ptr(w_gate), _ptr(w_up), w_gate.stride(0),
                                       _ptr(w_down), w_down.stride(0), _ptr(out), out.numel() * out.element_size(),
                                       _stream_of(device, stream)))
    return PackedWeights(out, h, I_s, int(t), wc)


def packed_workspace_bytes(M, h, I_full, t, w_dtype=torch.bfloat16):
    """Workspace bytes of ``shard_forward_packed`` (0: shapes the packed forward does not take)."""
    return int(_lib.load().tp_mlp_packed_workspace_bytes(M, h, I_full, t, _w_code(w_dtype)))


def shard_forward_packed(x, packed, *, k, s_gate=None, s_up=None, s_down=None, partial=None, workspace=None,
                         stream=None):
    """``shard_forward`` with packed weights; x (M, h) bf16.  Decode sizes run
    the weight-streaming kernels (bit-identical to ``shard_forward``), larger
    M with bf16 weights the packed-weight MFMA GEMMs."""
    call = prepare_shard_forward_packed(x, packed, k=k, s_gate=s_gate, s_up=s_up, s_down=s_down, partial=partial,
                                        workspace=workspace, stream=stream)
    call()
    return call.partial


def prepare_shard_forward_packed(x, packed, *, k, s_gate=None, s_up=None, s_down=None, partial=None,
                                 workspace=None, stream=None):
    device = x.device
    _check_matrix("x", x, device)
    if packed.data.device != device:
        raise ValueError("packed weights must be on %s" % device)
    M, h = x.shape
    if h != packed.h:
        raise ValueError("x has %d columns, the weights were packed for h = %d" % (h, packed.h))
    for name, s, n in (("s_gate", s_gate, packed.I_s), ("s_up", s_up, packed.I_s), ("s_down", s_down, h)):
        _check_scales(s, device, n, name)
    if partial is None:
        partial = torch.empty((M, h), dtype=torch.float32, device=device)
    else:
        _check_matrix("partial", partial, device)
        if partial.dtype != torch.float32 or tuple(partial.shape) != (M, h):
            raise ValueError("partial must be float32 of shape (%d, %d)" % (M, h))
    lib = _lib.load()
    act = _act_code(x.dtype)
    I_full = packed.I_s * packed.t
    need = int(lib.tp_mlp_packed_workspace_bytes(M, h, I_full, packed.t, packed.w_code))
    if workspace is None:
        workspace = alloc_workspace(max(need, 1), device)
    elif workspace.device != device:
        raise ValueError("workspace must be on %s" % device)
    args = (M, h, I_full, packed.t, int(k), act, packed.w_code, _ptr(x), x.stride(0), _ptr(packed.data),
            packed.data.numel() * packed.data.element_size(), _ptr(s_gate), _ptr(s_up), _ptr(s_down), _ptr(partial), partial.stride(0), _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream_of(device, stream))
    call = PreparedCall(lib.tp_mlp_shard_forward_packed, args, (x, packed, s_gate, s_up, s_down, partial, workspace))
    call.partial = partial
    return call


def partial_reduce(partials, out=None, stream=None):
    """out = (((P_0 + P_1) + P_2) + ...) elementwise in fp32, fixed order.

    ``partials``: sequence of t same-shaped contiguous float32 device tensors.
    ``out`` may be ``partials[0]`` (in place); default: a new tensor.
    """
    call = prepare_partial_reduce(partials, out=out, stream=stream)
    call()
    return call.out


def prepare_partial_reduce(partials, out=None, stream=None):
    """Validate and marshal a partial_reduce once; returns a PreparedCall
    (attribute ``out`` is the output tensor)."""
    if len(partials) < 1:
        raise ValueError("need at least one partial")
    p0 = partials[0]
    device = p0.device
    for i, p in enumerate(partials):
        if p.dtype != torch.float32 or p.device != device or not p.is_contiguous() or p.shape != p0.shape:
            raise ValueError("partials[%d] must be a contiguous float32 tensor shaped like partials[0]" % i)
    if out is None:
        out = torch.empty_like(p0)
    elif out.dtype != torch.float32 or out.device != device or not out.is_contiguous() or out.shape != p0.shape:
        raise ValueError("out must be a contiguous float32 tensor shaped like the partials")
    arr = (ctypes.c_void_p * len(partials))(*[p.data_ptr() for p in partials])
    lib = _lib.load()
    call = PreparedCall(lib.tp_partial_reduce,
                        (p0.numel(), len(partials), arr, _ptr(out), _stream_of(device, stream)),
                        (list(partials), out))
    call.out = out
    return call


def partial_reduce_scatter(partials, k, out=None, stream=None):
    """Rank k's rows of the fixed-order sum (reduce-scatter form,
    ``include/tp_mlp.h``: tp_partial_reduce_scatter): ``partials`` are t
    contiguous float32 (rows, ...) tensors, rows % t == 0; returns rows
    [k*rows/t, (k+1)*rows/t) of their left-fold sum."""
    call = prepare_partial_reduce_scatter(partials, k, out=out, stream=stream)
    call()
    return call.out


def prepare_partial_reduce_scatter(partials, k, out=None, stream=None):
    """Marshal a partial_reduce_scatter once; returns a PreparedCall."""
    t = len(partials)
    if t < 1:
        raise ValueError("need at least one partial")
    p0 = partials[0]
    device = p0.device
    for i, p in enumerate(partials):
        if p.dtype != torch.float32 or p.device != device or not p.is_contiguous() or p.shape != p0.shape:
            raise ValueError("partials[%d] must be a contiguous float32 tensor shaped like partials[0]" % i)
    rows = p0.shape[0] if p0.dim() > 0 else 1
    row_len = p0.numel() // max(rows, 1)
    if rows % t:
        raise ValueError("rows (%d) must be a multiple of t (%d)" % (rows, t))
    shape = (rows // t,) + tuple(p0.shape[1:])
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=device)
    elif out.dtype != torch.float32 or out.device != device or not out.is_contiguous() or tuple(out.shape) != shape:
        raise ValueError("out must be a contiguous float32 tensor of shape %s" % (shape,))
    arr = (ctypes.c_void_p * t)(*[p.data_ptr() for p in partials])
    lib = _lib.load()
    call = PreparedCall(lib.tp_partial_reduce_scatter,
                        (rows, row_len, t, int(k), arr, _ptr(out), _stream_of(device, stream)),
                        (list(partials), out))
    call.out = out
    return call


def w8a8_workspace_bytes(M, h, I_full, t):
    """Bytes of device workspace ``shard_forward_w8a8`` needs (0 if invalid)."""
    return int(_lib.load().tp_mlp_w8a8_workspace_bytes(int(M), int(h), int(I_full), int(t)))


def shard_forward_w8a8(x, w_gate, w_up, w_down, *, t, k, s_gate, s_up, s_down, partial=None, workspace=None,
                       stream=None):
    """Rank k's fp32 partial with per-token fp8 activations and fp8 weights
    (``include/tp_mlp.h``: tp_mlp_shard_forward_w8a8).  x: (M, h) bf16;
    weights float8_e4m3fn (or uint8 codes) with fp32 row scales."""
    call = prepare_shard_forward_w8a8(x, w_gate, w_up, w_down, t=t, k=k, s_gate=s_gate, s_up=s_up,
                                      s_down=s_down, partial=partial, workspace=workspace, stream=stream)
    call()
    return call.partial


def prepare_shard_forward_w8a8(x, w_gate, w_up, w_down, *, t, k, s_gate, s_up, s_down, partial=None,
                               workspace=None, stream=None):
    """Marshal a shard_forward_w8a8 once; returns a PreparedCall (``partial``)."""
    device = x.device
    _check_matrix("x", x, device)
    for name, m in (("w_gate", w_gate), ("w_up", w_up), ("w_down", w_down)):
        _check_matrix(name, m, device)
        if _w_code(m.dtype) != TP_FP8_E4M3FN:
            raise TypeError("%s must hold e4m3fn codes" % name)
    if x.dtype != torch.bfloat16:
        raise TypeError("x must be bfloat16")
    M, h = x.shape
    I_s = w_gate.shape[0]
    I_full = I_s * int(t)
    for name, sc, n in (("s_gate", s_gate, I_s), ("s_up", s_up, I_s), ("s_down", s_down, h)):
        _check_scales(sc, device, n, name)
    if tuple(w_up.shape) != (I_s, h) or tuple(w_gate.shape) != (I_s, h) or tuple(w_down.shape) != (h, I_s):
        raise ValueError("shard shapes must be w_gate/w_up (I_s, h) and w_down (h, I_s)")
    if w_gate.stride(0) != w_up.stride(0):
        raise ValueError("w_gate and w_up must share a leading dimension")
    if partial is None:
        partial = torch.empty((M, h), dtype=torch.float32, device=device)
    need = w8a8_workspace_bytes(M, h, I_full, t)
    if workspace is None:
        workspace = alloc_workspace(max(need, 1), device)
    lib = _lib.load()
    args = (M, h, I_full, int(t), int(k), _ptr(x), x.stride(0), _ptr(w_gate), _ptr(w_up), w_gate.stride(0),
            _ptr(w_down), w_down.stride(0), _ptr(s_gate), _ptr(s_up), _ptr(s_down), _ptr(partial),
            partial.stride(0), _ptr(workspace), workspace.numel() * workspace.element_size(),
            _stream_of(device, stream))
    call = PreparedCall(lib.tp_mlp_shard_forward_w8a8, args,
                        (x, w_gate, w_up, w_down, s_gate, s_up, s_down, partial, workspace))
    call.partial = partial
    return call


def quantize_rows_e4m3(x, codes=None, scales=None, stream=None):
    """Per-row e4m3fn codes (uint8, same shape) and fp32 scales of a bf16
    matrix (``include/tp_mlp.h``: tp_quantize_rows_e4m3)."""
    device = x.device
    _check_matrix("x", x, device)
    if x.dtype != torch.bfloat16:
        raise TypeError("x must be bfloat16")
    rows, cols = x.shape
    if codes is None:
        codes = torch.empty((rows, cols), dtype=torch.uint8, device=device)
    if scales is None:
        scales = torch.empty((rows,), dtype=torch.float32, device=device)
    _lib.check(_lib.load().tp_quantize_rows_e4m3(rows, cols, _ptr(x), x.stride(0), _ptr(codes), codes.stride(0),
                                                 _ptr(scales), _stream_of(device, stream)))
    return codes, scales


def attn_qkv_width(n_heads, n_kv_heads, head_dim, t):
    """Width n_loc of one rank's QKV output, or -1 if the heads do not split
    over t (``include/tp_mlp.h``: tp_attn_qkv_width)."""
    return int(_lib.load().tp_attn_qkv_width(int(n_heads), int(n_kv_heads), int(head_dim), int(t)))


def _check_scales(s, device, n=None, name="scales"):
    """A scale vector is a contiguous float32 tensor on `device`; with `n`,
    it must hold exactly n elements (the C ABI takes no length, and the
    kernels read one scale per output row)."""
    if s is None:
        return
    if s.dtype != torch.float32 or s.device != device or not s.is_contiguous():
        raise ValueError("%s must be contiguous float32 tensors on %s" % (name, device))
    if n is not None and s.numel() != n:
        raise ValueError("%s must hold %d elements (one per output row), got %d" % (name, n, s.numel()))


def attn_qkv_workspace_bytes(M, h, n_heads, n_kv_heads, head_dim, t, act_dtype=torch.bfloat16,
                             w_dtype=torch.bfloat16):
    """Bytes of device workspace ``attn_qkv_forward`` needs (often 0)."""
    return int(_lib.load().tp_attn_qkv_workspace_bytes(int(M), int(h), int(n_heads), int(n_kv_heads),
                                                       int(head_dim), int(t), _act_code(act_dtype),
                                                       _w_code(w_dtype)))


def attn_qkv_forward(x, w_qkv, *, n_heads, n_kv_heads, head_dim, t, k, s_qkv=None, out=None, workspace=None,
                     stream=None):
    """Rank k's column-parallel QKV projection X W_qkv_k^T (M x n_loc, in x's
    dtype); ``w_qkv`` is the rank's (n_loc, h) rows [q heads | k heads | v
    heads] (``include/tp_mlp.h``: tp_attn_qkv_forward)."""
    call = prepare_attn_qkv_forward(x, w_qkv, n_heads=n_heads, n_kv_heads=n_kv_heads, head_dim=head_dim, t=t,
                                    k=k, s_qkv=s_qkv, out=out, workspace=workspace, stream=stream)
    call()
    return call.out


def prepare_attn_qkv_forward(x, w_qkv, *, n_heads, n_kv_heads, head_dim, t, k, s_qkv=None, out=None,
                             workspace=None, stream=None):
    """Marshal an attn_qkv_forward once; returns a PreparedCall (``out``)."""
    device = x.device
    _check_matrix("x", x, device)
    _check_matrix("w_qkv", w_qkv, device)
    M, h = x.shape
    n_loc = attn_qkv_width(n_heads, n_kv_heads, head_dim, t)
    if n_loc < 0:
        raise ValueError("heads (%d query, %d kv) do not split over t = %d" % (n_heads, n_kv_heads, t))
    _check_scales(s_qkv, device, n_loc, "s_qkv")
    if tuple(w_qkv.shape) != (n_loc, h):
        raise ValueError("w_qkv must be (%d, %d), got %s" % (n_loc, h, tuple(w_qkv.shape)))
    if out is None:
        out = torch.empty((M, n_loc), dtype=x.dtype, device=device)
    else:
        _check_matrix("out", out, device)
        if out.dtype != x.dtype or tuple(out.shape) != (M, n_loc):
            raise ValueError("out must be %s of shape (%d, %d)" % (x.dtype, M, n_loc))
    lib = _lib.load()
    need = attn_qkv_workspace_bytes(M, h, n_heads, n_kv_heads, head_dim, t, x.dtype, w_qkv.dtype)
    if workspace is None and need > 0:
        workspace = alloc_workspace(need, device)
    elif workspace is not None and workspace.device != device:
        raise ValueError("workspace must be on %s" % device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (M, h, int(n_heads), int(n_kv_heads), int(head_dim), int(t), int(k), _act_code(x.dtype),
            _w_code(w_qkv.dtype), _ptr(x), x.stride(0), _ptr(w_qkv), w_qkv.stride(0), _ptr(s_qkv), _ptr(out),
            out.stride(0), _ptr(workspace), ws_bytes, _stream_of(device, stream))
    call = PreparedCall(lib.tp_attn_qkv_forward, args, (x, w_qkv, s_qkv, out, workspace))
    call.out = out
    return call


def attn_out_forward(attn, w_o, *, n_heads, head_dim, t, k, s_o=None, partial=None, stream=None):
    """Rank k's row-parallel output projection: fp32 partial O_k W_o_k^T
    (M x h); ``attn`` is (M, n_heads/t*head_dim), ``w_o`` the rank's (h,
    n_heads/t*head_dim) column block (``include/tp_mlp.h``:
    tp_attn_out_forward)."""
    call = prepare_attn_out_forward(attn, w_o, n_heads=n_heads, head_dim=head_dim, t=t, k=k, s_o=s_o,
                                    partial=partial, stream=stream)
    call()
    return call.partial


def prepare_attn_out_forward(attn, w_o, *, n_heads, head_dim, t, k, s_o=None, partial=None, stream=None):
    """Marshal an attn_out_forward once; returns a PreparedCall (``partial``)."""
    device = attn.device
    _check_matrix("attn", attn, device)
    _check_matrix("w_o", w_o, device)
    M, K = attn.shape
    h = w_o.shape[0]
    _check_scales(s_o, device, h, "s_o")
    if int(n_heads) % int(t) or K != int(n_heads) // int(t) * int(head_dim) or w_o.shape[1] != K:
        raise ValueError("attn (%d, %d) and w_o %s do not match n_heads/t * head_dim = %s"
                         % (M, K, tuple(w_o.shape), int(n_heads) / int(t) * int(head_dim)))
    if partial is None:
        partial = torch.empty((M, h), dtype=torch.float32, device=device)
    else:
        _check_matrix("partial", partial, device)
        if partial.dtype != torch.float32 or tuple(partial.shape) != (M, h):
            raise ValueError("partial must be float32 of shape (%d, %d)" % (M, h))
    lib = _lib.load()
    args = (M, h, int(n_heads), int(head_dim), int(t), int(k), _act_code(attn.dtype), _w_code(w_o.dtype),
            _ptr(attn), attn.stride(0), _ptr(w_o), w_o.stride(0), _ptr(s_o), _ptr(partial), partial.stride(0),
            _stream_of(device, stream))
    call = PreparedCall(lib.tp_attn_out_forward, args, (attn, w_o, s_o, partial))
    call.partial = partial
    return call


def kernel_kinds():
    lib = _lib.load()
    return [lib.tp_kernel_kind_name(i).decode() for i in range(lib.tp_kernel_kind_count())]


def profile_enable(on=True, kinds=None):
    """Time the library's launches of the given kernel kinds (names from
    kernel_kinds(); None = all) while on; off with on=False."""
    if not on:
        mask = 0
    elif kinds is None:
        mask = -1
    else:
        names = kernel_kinds()
        mask = 0
        for k in kinds:
            mask |= 1 << names.index(k)
    _lib.check(_lib.load().tp_profile_enable(mask))


def profile_reserve(records):
    """Create timing events for `records` launches ahead of a measured loop."""
    _lib.check(_lib.load().tp_profile_reserve(int(records)))


def profile_durations(kind):
    """Durations in milliseconds of the recorded launches of one kernel kind
    (a name from kernel_kinds()), in launch order; the record is kept for
    profile_collect()."""
    lib = _lib.load()
    k = kernel_kinds().index(kind)
    n = ctypes.c_int64(0)
    _lib.check(lib.tp_profile_durations(k, None, 0, ctypes.byref(n)))
    buf = (ctypes.c_float * max(n.value, 1))()
    _lib.check(lib.tp_profile_durations(k, buf, n.value, ctypes.byref(n)))
    return [float(buf[i]) for i in range(n.value)]


def profile_collect():
    """{kernel kind: (total milliseconds, launches)} since the last collect."""
    lib = _lib.load()
    n = lib.tp_kernel_kind_count()
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int64 * n)()
    _lib.check(lib.tp_profile_collect(ms, cnt, n))
    names = kernel_kinds()
    return {names[i]: (ms[i], cnt[i]) for i in range(n) if cnt[i]}
