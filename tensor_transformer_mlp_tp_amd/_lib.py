"""ctypes binding of libtp_mlp.so (argument marshalling only).

Every step of the computation runs in the library's HIP kernels; this module
converts torch tensors to pointers, sizes and the current stream, calls the C
ABI and turns non-OK statuses into exceptions.  It never computes a result
itself and never falls back to another implementation: if the library is
missing, loading fails with an error that says how to build it.
"""

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
# The in-tree library, built from csrc/ by build.py.
LIB_PATH = os.path.join(PKG, "libtp_mlp.so")

TP_F32, TP_BF16, TP_FP8_E4M3FN, TP_INT8 = 0, 1, 2, 3
TP_OK, TP_ERR_INVALID_ARG, TP_ERR_UNSUPPORTED, TP_ERR_WORKSPACE, TP_ERR_HIP = 0, 1, 2, 3, 4

EXPORTED_SYMBOLS = (
    "tp_mlp_workspace_bytes",
    "tp_mlp_shard_forward",
    "tp_mlp_shard_forward_noalloc",
    "tp_mlp_packed_weights_bytes",
    "tp_mlp_pack_weights",
    "tp_mlp_shard_forward_packed",
    "tp_mlp_packed_workspace_bytes",
    "tp_partial_reduce",
    "tp_mlp_shard_forward_sp",
    "tp_partial_reduce_scatter",
    "tp_mlp_w8a8_workspace_bytes",
    "tp_mlp_shard_forward_w8a8",
    "tp_quantize_rows_e4m3",
    "tp_attn_qkv_width",
    "tp_attn_qkv_forward",
    "tp_attn_qkv_workspace_bytes",
    "tp_attn_out_forward",
    "tp_status_string",
    "tp_last_error",
    "tp_kernel_kind_count",
    "tp_kernel_kind_name",
    "tp_profile_enable",
    "tp_profile_collect",
    "tp_profile_durations",
    "tp_profile_reserve",
)


class TPError(RuntimeError):
    def __init__(self, status, message):
        super().__init__("%s (%s)" % (message, _STATUS_NAMES.get(status, status)))
        self.status = status


_STATUS_NAMES = {0: "TP_OK", 1: "TP_ERR_INVALID_ARG", 2: "TP_ERR_UNSUPPORTED",
                 3: "TP_ERR_WORKSPACE", 4: "TP_ERR_HIP"}

_lib = None


def load():
    """Load libtp_mlp.so from the package directory (once)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError("libtp_mlp.so is not built; run `python -m tensor_transformer_mlp_tp_amd.build` "
                          "(expected at %s)" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    c_i64, c_i32, vp, fp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.POINTER(ctypes.c_float)
    lib.tp_mlp_workspace_bytes.argtypes = [c_i64, c_i64, c_i64, c_i32, c_i32, c_i32]
    lib.tp_mlp_workspace_bytes.restype = ctypes.c_size_t
    lib.tp_mlp_shard_forward.argtypes = [
        c_i64, c_i64, c_i64, c_i32, c_i32, c_i32, c_i32,
        vp, c_i64, vp, vp, c_i64, vp, c_i64, vp, vp, vp, vp, c_i64, vp, ctypes.c_size_t, vp]
    lib.tp_mlp_shard_forward.restype = c_i32
    lib.tp_mlp_shard_forward_noalloc.argtypes = [
        c_i64, c_i64, c_i64, c_i32, c_i32, c_i32, c_i32,
        vp, c_i64, vp, vp, c_i64, vp, c_i64, vp, vp, vp, vp, c_i64, vp]
    lib.tp_mlp_shard_forward_noalloc.restype = c_i32
    lib.tp_partial_reduce.argtypes = [c_i64, c_i32, ctypes.POINTER(vp), vp, vp]
    lib.tp_partial_reduce.restype = c_i32
    lib.tp_mlp_shard_forward_sp.argtypes = [
        c_i64, c_i64, c_i64, c_i32, c_i32, c_i32, c_i32,
        ctypes.POINTER(vp), c_i64, vp, vp, c_i64, vp, c_i64, vp, vp, vp, vp, c_i64, vp, ctypes.c_size_t, vp]
    lib.tp_mlp_shard_forward_sp.restype = c_i32
    lib.tp_partial_reduce_scatter.argtypes = [c_i64, c_i64, c_i32, c_i32, ctypes.POINTER(vp), vp, vp]
    lib.tp_partial_reduce_scatter.restype = c_i32
    lib.tp_mlp_packed_weights_bytes.argtypes = [c_i64, c_i64, c_i32, c_i32]
    lib.tp_mlp_packed_weights_bytes.restype = ctypes.c_size_t
    lib.tp_mlp_pack_weights.argtypes = [c_i64, c_i64, c_i32, c_i32, vp, vp, c_i64, vp, c_i64, vp, ctypes.c_size_t, vp]
    lib.tp_mlp_pack_weights.restype = c_i32
    lib.tp_mlp_shard_forward_packed.argtypes = [
        c_i64, c_i64, c_i64, c_i32, c_i32, c_i32, c_i32, vp, c_i64, vp, ctypes.c_size_t, vp, vp, vp, vp, c_i64, vp,
        ctypes.c_size_t, vp]
    lib.tp_mlp_shard_forward_packed.restype = c_i32
    lib.tp_mlp_packed_workspace_bytes.argtypes = [c_i64, c_i64, c_i64, c_i32, c_i32]
    lib.tp_mlp_packed_workspace_bytes.restype = ctypes.c_size_t
    lib.tp_mlp_w8a8_workspace_bytes.argtypes = [c_i64, c_i64, c_i64, c_i32]
    lib.tp_mlp_w8a8_workspace_bytes.restype = ctypes.c_size_t
    lib.tp_mlp_shard_forward_w8a8.argtypes = [
        c_i64, c_i64, c_i64, c_i32, c_i32,
        vp, c_i64, vp, vp, c_i64, vp, c_i64, vp, vp, vp, vp, c_i64, vp, ctypes.c_size_t, vp]
    lib.tp_mlp_shard_forward_w8a8.restype = c_i32
    lib.tp_quantize_rows_e4m3.argtypes = [c_i64, c_i64, vp, c_i64, vp, c_i64, vp, vp]
    lib.tp_quantize_rows_e4m3.restype = c_i32
    lib.tp_attn_qkv_width.argtypes = [c_i64, c_i64, c_i64, c_i32]
    lib.tp_attn_qkv_width.restype = c_i64
    lib.tp_attn_qkv_forward.argtypes = [
        c_i64, c_i64, c_i64, c_i64, c_i64, c_i32, c_i32, c_i32, c_i32,
        vp, c_i64, vp, c_i64, vp, vp, c_i64, vp, ctypes.c_size_t, vp]
    lib.tp_attn_qkv_workspace_bytes.argtypes = [c_i64, c_i64, c_i64, c_i64, c_i64, c_i32, c_i32, c_i32]
    lib.tp_attn_qkv_workspace_bytes.restype = ctypes.c_size_t
    lib.tp_attn_qkv_forward.restype = c_i32
    lib.tp_attn_out_forward.argtypes = [
        c_i64, c_i64, c_i64, c_i64, c_i32, c_i32, c_i32, c_i32,
        vp, c_i64, vp, c_i64, vp, vp, c_i64, vp]
    lib.tp_attn_out_forward.restype = c_i32
    lib.tp_status_string.argtypes = [c_i32]
    lib.tp_status_string.restype = ctypes.c_char_p
    lib.tp_last_error.argtypes = []
    lib.tp_last_error.restype = ctypes.c_char_p
    lib.tp_kernel_kind_count.argtypes = []
    lib.tp_kernel_kind_count.restype = c_i32
    lib.tp_kernel_kind_name.argtypes = [c_i32]
    lib.tp_kernel_kind_name.restype = ctypes.c_char_p
    lib.tp_profile_enable.argtypes = [c_i32]
    lib.tp_profile_enable.restype = c_i32
    lib.tp_profile_collect.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(c_i64), c_i32]
    lib.tp_profile_collect.restype = c_i32
    lib.tp_profile_reserve.argtypes = [c_i64]
    lib.tp_profile_reserve.restype = c_i32
    lib.tp_profile_durations.argtypes = [c_i32, ctypes.POINTER(ctypes.c_float), c_i64, ctypes.POINTER(c_i64)]
    lib.tp_profile_durations.restype = c_i32
    _lib = lib
    return lib


def check(status):
    if status != TP_OK:
        raise TPError(status, load().tp_last_error().decode())
