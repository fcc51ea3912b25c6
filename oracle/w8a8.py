"""Plain definition of the fp8 x fp8 (W8A8) rank forward.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The pages give fp8 only as a one-byte-per-parameter mode (the shard planner
of the scalablesystem.dev page).  The W8A8 variant quantises the activations
too, per token, and its steps are taken in this order (the plainest reading,
listed with the other readings of the pages):

1. X (bf16) -> per-row scale s_m = float32(amax_m / 448) (1 for an all-zero
   row) and codes q = e4m3fn(float32(x / s_m)): nearest code, ties to even,
   saturating at 448.  These are decisions on floating-point values, so they
   are taken in the same precision as the kernels (float32 quotient of exact
   bf16 inputs), and the codes are compared bit for bit.
2. G, U = deq(Xq) deq(W_gate)^T, deq(Xq) deq(W_up)^T in float64, where
   deq(code) * scale is exact in float64 (row scales s_m, s_gate, s_up).
3. A = SiLU(G) * U, rounded to bf16 as the kernels store it: float32 first,
   then nearest-even bf16 (the kernels hold G and U in float32).
4. A -> per-row codes and scales as in step 1.
5. P_k = deq(Aq) deq(W_down)^T in float64.

No blocking or reordering beyond those steps.
"""

import numpy as np

from .formats import bf16_bits_to_f64, bf16_round_bits, e4m3fn_encode, e4m3fn_to_f64
from .mlp import silu

E4M3_MAX = np.float32(448.0)


def quantise_rows_e4m3(x32):
    """Per-row dynamic e4m3fn quantisation of float32 rows (step 1):
    returns (codes uint8, scales float32)."""
    x32 = np.asarray(x32, dtype=np.float32)
    amax = np.max(np.abs(x32), axis=1)
    s = np.where(amax == 0, np.float32(1.0), (amax / E4M3_MAX).astype(np.float32)).astype(np.float32)
    q = e4m3fn_encode((x32 / s[:, None]).astype(np.float32))
    return q, s


def dequantise_rows(codes, scales):
    """codes * per-row scale, float64 (exact)."""
    return e4m3fn_to_f64(codes) * np.asarray(scales, dtype=np.float64)[:, None]


def rank_partial_w8a8_from_storage(x_bits, w_gate, w_up, w_down, s_gate, s_up, s_down, return_codes=False):
    """P_k of the W8A8 forward from the stored bytes: x_bits (M x h bf16 bit
    patterns), weight codes (e4m3fn, uint8) with float32 row scales."""
    x32 = bf16_bits_to_f64(x_bits).astype(np.float32)       # exact
    xq, sx = quantise_rows_e4m3(x32)
    xd = dequantise_rows(xq, sx)
    wg = dequantise_rows(w_gate, s_gate)
    wu = dequantise_rows(w_up, s_up)
    wd = dequantise_rows(w_down, s_down)
    g = xd @ wg.T
    u = xd @ wu.T
    a = silu(g) * u
    a_bits = bf16_round_bits(a.astype(np.float32))
    a32 = bf16_bits_to_f64(a_bits).astype(np.float32)
    aq, sa = quantise_rows_e4m3(a32)
    p = dequantise_rows(aq, sa) @ wd.T
    if return_codes:
        return p, dict(xq=xq, sx=sx, a_bits=a_bits, aq=aq, sa=sa)
    return p
