"""Plain float64 definition of one rank's attention-block projections.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Notation (weights in the ``nn.Linear`` ``(out, in)`` layout):

* X: M x h tokens; head size d; W_q: n_heads*d x h; W_k, W_v: n_kv_heads*d x h;
  W_o: h x n_heads*d.  Head i of Q = X W_q^T is its columns [i*d, (i+1)*d),
  produced by rows [i*d, (i+1)*d) of W_q; likewise for K and V.
* TPAttentionBlock in "The Tensor-Parallel Shard Group" section of the
  scalablesystem.dev page: the QKV projection is column-parallel, so a rank
  computes the projections of its own heads with no communication; attention
  runs locally over those heads; the output projection is row-parallel, its
  per-rank outputs summed by the all-reduce.  Section 12.2.1 of the
  arunshar.com chapter: rank k handles n_heads/t heads, split like the MLP's
  first matrix (contiguous blocks, the same reading as the MLP's slices).
* Grouped-query attention: the KV-head count must divide by the TP degree
  (the question on uneven division on the scalablesystem.dev page); when the
  degree is a multiple of the KV-head count each rank keeps one KV head,
  replicated over t / n_kv_heads ranks (section "The KV cache splits too,
  until it doesn't" of the vidyal.ai page).  Rank k's query heads are
  [k*q_loc, (k+1)*q_loc), q_loc = n_heads/t; its KV heads [k*kv_loc,
  (k+1)*kv_loc), kv_loc = n_kv_heads/t, or the single head k // (t/n_kv_heads)
  when replicated.
* A rank's QKV weight stacks its rows as [query heads | key heads | value
  heads], heads in global order; its output columns follow the same order.
* The output projection of rank k takes the attention output of its query
  heads, O_k (M x q_loc*d), and W_o's matching column block
  W_o[:, k*q_loc*d : (k+1)*q_loc*d]; P_k = O_k W_o_k^T and sum_k P_k = O W_o^T.

No blocking or reordering beyond the definition: one library matmul each.
"""

import numpy as np

from .formats import bf16_bits_to_f64, e4m3fn_to_f64, int8_to_f64


def local_heads(n_heads, n_kv_heads, t, k):
    """(query heads, KV heads) of rank k out of t, as lists of global indices."""
    if t < 1 or not (0 <= k < t):
        raise ValueError("need t >= 1 and 0 <= k < t")
    if n_heads % t or n_heads % n_kv_heads:
        raise ValueError("query heads must divide by t and by the KV-head count")
    q_loc = n_heads // t
    q = list(range(k * q_loc, (k + 1) * q_loc))
    if n_kv_heads % t == 0:
        kv_loc = n_kv_heads // t
        kv = list(range(k * kv_loc, (k + 1) * kv_loc))
    elif t % n_kv_heads == 0:
        kv = [k // (t // n_kv_heads)]
    else:
        raise ValueError("KV heads neither divide by t nor divide t")
    return q, kv


def head_rows(heads, head_dim):
    """Row indices (of a per-head stacked matrix) of the given heads."""
    return np.concatenate([np.arange(i * head_dim, (i + 1) * head_dim) for i in heads]).astype(np.int64)


def qkv_rank_weight(w_q, w_k, w_v, n_heads, n_kv_heads, head_dim, t, k):
    """Rank k's stacked QKV weight (n_loc x h) taken from the full matrices."""
    q, kv = local_heads(n_heads, n_kv_heads, t, k)
    return np.concatenate([np.asarray(w_q)[head_rows(q, head_dim)],
                           np.asarray(w_k)[head_rows(kv, head_dim)],
                           np.asarray(w_v)[head_rows(kv, head_dim)]], axis=0)


def o_proj_rank_weight(w_o, n_heads, head_dim, t, k):
    """Rank k's column block of the full output projection (h x q_loc*d)."""
    q, _ = local_heads(n_heads, n_heads, t, k)
    return np.asarray(w_o)[:, head_rows(q, head_dim)]


def linear(a, w):
    """a W^T in float64 (the projection of one rank, either side)."""
    return np.asarray(a, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T


def _decode(arr, dtype):
    if dtype == "bf16":
        return bf16_bits_to_f64(arr)
    if dtype == "f32":
        a = np.asarray(arr)
        if a.dtype != np.float32:
            raise TypeError("f32 storage must be float32")
        return a.astype(np.float64)
    if dtype == "e4m3fn":
        return e4m3fn_to_f64(arr)
    if dtype == "int8":
        return int8_to_f64(arr)
    raise ValueError("unknown storage dtype %r" % (dtype,))


def linear_from_storage(a, a_dtype, w, w_dtype, s=None):
    """a W^T in float64 from the raw storage the library receives; for one-byte
    weights (e4m3fn, int8) row n of W is dequantised as code * s[n] (exact in
    float64)."""
    af = _decode(a, a_dtype)
    wf = _decode(w, w_dtype)
    if w_dtype in ("e4m3fn", "int8"):
        if s is None:
            raise ValueError("one-byte weights need per-row scales")
        wf = wf * np.asarray(s, dtype=np.float64)[:, None]
    return linear(af, wf)
