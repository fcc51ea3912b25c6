"""Plain float64 definition of the tensor-parallel MLP shard and partial sum.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Notation (weights in the ``nn.Linear`` ``(out, in)`` layout used by the
ColumnParallelLinear / RowParallelLinear classes in "The Tensor-Parallel Shard
Group" section of the scalablesystem.dev page):

* X: M x h tokens;  W_gate, W_up: I x h;  W_down: h x I.
* t ranks; rank k owns the contiguous intermediate slice S_k = [k*I/t, (k+1)*I/t)
  (the column blocks A_1 | ... | A_t of section 12.2.1 of the arunshar.com
  chapter, taken as contiguous blocks).
* Gate/up are column-parallel (rank k holds rows S_k of W_gate and W_up), down
  is row-parallel (rank k holds columns S_k of W_down), per the same section
  of the scalablesystem.dev page and "Step 1" of the vidyal.ai page.
* The activation is SwiGLU: SiLU applied to the gate projection, multiplied
  elementwise by the up projection (the pages write GeLU for the two-matrix
  Megatron MLP and say Llama adds a second input matrix split the same way;
  SiLU(gate) * up is the reading used here).
* Rank k's partial is P_k = (SiLU(X W_gate[S_k]^T) * (X W_up[S_k]^T)) W_down[:, S_k]^T
  and the all-reduce adds the partials: Y = sum_k P_k (section 12.2.1, Z = sum Z_k).

No blocking, fusion or reordering beyond the definition: two library matmuls,
an elementwise SiLU and product, one more matmul.
"""

import numpy as np

from .formats import bf16_bits_to_f64, e4m3fn_to_f64, int8_to_f64


def silu(z):
    """SiLU(z) = z * sigmoid(z) = z / (1 + exp(-z)), float64.

    For very negative z, exp(-z) overflows to +inf and the quotient is -0,
    which is the limit of the function; the overflow warning is silenced.
    """
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def mlp_full(x, w_gate, w_up, w_down):
    """Unsharded MLP output Y = (SiLU(X Wg^T) * (X Wu^T)) Wd^T in float64."""
    x = np.asarray(x, dtype=np.float64)
    g = x @ np.asarray(w_gate, dtype=np.float64).T
    u = x @ np.asarray(w_up, dtype=np.float64).T
    a = silu(g) * u
    return a @ np.asarray(w_down, dtype=np.float64).T


def mlp_partial(x, w_gate_k, w_up_k, w_down_k):
    """Rank k's partial P_k from the shard matrices the rank holds.

    w_gate_k, w_up_k: I_s x h (rows S_k of the full matrices);
    w_down_k: h x I_s (columns S_k of the full W_down).  The formula is the
    same as the unsharded one applied to the shard, which is exactly what the
    column split (activation applied locally) and the row split (partial sum)
    give.
    """
    return mlp_full(x, w_gate_k, w_up_k, w_down_k)


def shard_slice(I, t, k):
    """Contiguous intermediate slice S_k of rank k out of t (I must divide)."""
    if t < 1 or not (0 <= k < t):
        raise ValueError("need t >= 1 and 0 <= k < t")
    if I % t != 0:
        raise ValueError("intermediate size must be divisible by the TP degree")
    i_s = I // t
    return slice(k * i_s, (k + 1) * i_s)


def shard_of_full(w_gate, w_up, w_down, t, k):
    """Views of rank k's shards of full (out, in) matrices."""
    s = shard_slice(np.shape(w_gate)[0], t, k)
    return w_gate[s, :], w_up[s, :], w_down[:, s]


def fold_fp32(partials):
    """The fixed-order float32 sum of t partial buffers.

    Y = (((P_0 + P_1) + P_2) + ...) + P_{t-1}, each addition an IEEE binary32
    round-to-nearest-even add (numpy float32 arithmetic, no fused operations).
    The pages point out that the all-reduce's summation order changes the bits
    (the "Quality, Evaluation, and Guardrails" section of the scalablesystem.dev
    page); this left fold over k = 0 .. t-1 is the order pinned here.
    """
    if len(partials) < 1:
        raise ValueError("need at least one partial")
    y = np.array(partials[0], dtype=np.float32, copy=True)
    for p in partials[1:]:
        p = np.asarray(p)
        if p.dtype != np.float32:
            raise TypeError("partials must be float32")
        y = y + p
    return y


def gather_rows(blocks):
    """All-gather of the t ranks' sequence slices: X is their row
    concatenation, block j holding rows [j*s/t, (j+1)*s/t) (sequence
    parallelism, section 12.3.1 of the arunshar.com chapter, step 3)."""
    return np.concatenate([np.asarray(b) for b in blocks], axis=0)


def reduce_scatter_fp32(partials, k):
    """Rank k's part of the reduce-scatter that replaces the all-reduce under
    sequence parallelism (section 12.3.1 of the arunshar.com chapter, step 1):
    the fully reduced rows [k*rows/t, (k+1)*rows/t), t = len(partials), of the
    same fixed-order float32 sum as fold_fp32."""
    t = len(partials)
    rows = np.asarray(partials[0]).shape[0]
    if rows % t:
        raise ValueError("rows must be a multiple of t")
    r = rows // t
    return fold_fp32([np.asarray(p)[k * r:(k + 1) * r] for p in partials])


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


SCALED_FORMATS = ("e4m3fn", "int8")


def rank_partial_from_storage(x, x_dtype, w_gate, w_up, w_down, w_dtype,
                              s_gate=None, s_up=None, s_down=None):
    """P_k in float64 from the raw storage the library receives.

    For one-byte weights (e4m3fn, int8) the reference weights are the
    dequantised values q * s with s the fp32 scale of the output channel: s_gate[j] / s_up[j]
    multiply row j of the gate / up shard, s_down[n] multiplies row n of the
    down shard.  The product of an e4m3 value and an fp32 scale is exact in
    float64.
    """
    xf = _decode(x, x_dtype)
    wg = _decode(w_gate, w_dtype)
    wu = _decode(w_up, w_dtype)
    wd = _decode(w_down, w_dtype)
    if w_dtype in SCALED_FORMATS:
        if s_gate is None or s_up is None or s_down is None:
            raise ValueError("one-byte weights need per-channel scales")
        wg = wg * np.asarray(s_gate, dtype=np.float64)[:, None]
        wu = wu * np.asarray(s_up, dtype=np.float64)[:, None]
        wd = wd * np.asarray(s_down, dtype=np.float64)[:, None]
    return mlp_partial(xf, wg, wu, wd)


def rms_normalised_max_error(out, ref):
    """max |out - ref| / sqrt(mean(ref^2)), in float64."""
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if out.shape != ref.shape:
        raise ValueError("shape mismatch %r vs %r" % (out.shape, ref.shape))
    rms = np.sqrt(np.mean(ref * ref))
    if rms == 0.0:
        return float(np.max(np.abs(out - ref))) if out.size else 0.0
    return float(np.max(np.abs(out - ref)) / rms)
