"""Seeded synthetic inputs and the workload table for the TP-MLP shard.

This module is shared by the tests, the benchmark and the CPU oracle's callers.
It holds no part of the MLP's arithmetic (no projection, activation or
reduction): only shapes, seeds, random draws, the rounding of those draws to
the storage formats the library consumes (bf16, OCP e4m3fn with per-channel
fp32 scales) and byte / FLOP accounting.

Recipe (one rule for every tensor):

* ``z`` = ``numpy.random.Generator(PCG64(seed)).standard_normal(n, float32)``;
* ``w`` = ``float32(std) * z`` (binary32 multiply, round-to-nearest-even);
* bf16 storage: ``w`` rounded to bfloat16, round-to-nearest-even;
* f32 storage: ``w`` itself;
* e4m3fn storage (per output channel j of the shard, i.e. per row of the
  ``(out, in)`` matrix): ``s_j = float32(amax_j / 448)`` (``s_j = 1`` if the
  row is all zero) and ``q = e4m3fn_rne(clamp(float32(w / s_j), -448, 448))``.

Seeds: ``seed = 1000 * config_id + tensor_id + 1_000_000 * weight_set`` with
tensor ids X = 1, W_gate = 2 + 10 k, W_up = 3 + 10 k, W_down = 4 + 10 k for
shard k, and partial buffer j = 100 + j; for the attention projections
W_qkv = 5 + 10 k, W_o = 6 + 10 k, the output projection's input O = 7, and
the full W_q, W_k, W_v, W_o of the split-against-unsplit case 200 .. 203.  ``weight_set`` 0 is the set the
parity tests use; the benchmark rotates through further sets so that weight
reads come from HBM rather than from the 256 MB last-level cache.

The shapes are those of Llama 3.1 70B (h = 8192, FFN 28672) and 405B
(h = 16384) tensor-parallel ranks.  The pages print the 70B shape ("Constraints"
section of the scalablesystem.dev page; worked example of section 12.2.1 of the
arunshar.com chapter) and the 405B hidden size (case studies of the same
chapter).  No trained weights are involved: values are Gaussian stand-ins.
"""

import concurrent.futures

import numpy as np

# ---------------------------------------------------------------------------
# workload table
# ---------------------------------------------------------------------------

CONFIGS = {
    1: dict(name="tiny_t4", desc="tiny MLP, t=4 shards, all shards summed",
            M=(16,), h=256, I=1024, t=4, act="f32", w="f32",
            std_x=1.0, std_gu=1.0 / 16.0, std_down=1.0 / 32.0,
            reduce_n=None),
    2: dict(name="llama70b_tp8_decode", desc="70B-shaped TP=8 rank decode",
            M=(1, 8, 64), h=8192, I=28672, t=8, act="bf16", w="bf16",
            std_x=1.0, std_gu=0.02, std_down=0.02, reduce_n=None),
    3: dict(name="llama70b_tp8_prefill", desc="70B-shaped TP=8 rank prefill",
            M=(4096,), h=8192, I=28672, t=8, act="bf16", w="bf16",
            std_x=1.0, std_gu=0.02, std_down=0.02, reduce_n=4096 * 8192),
    4: dict(name="llama70b_tp4_fp8", desc="70B-shaped TP=4 rank, fp8 e4m3 weights",
            M=(32, 2048), h=8192, I=28672, t=4, act="bf16", w="e4m3fn",
            std_x=1.0, std_gu=0.02, std_down=0.02, reduce_n=None),
    9: dict(name="llama70b_tp2_int8", desc="70B-shaped TP=2 rank, int8 weights (W8A16)",
            M=(1, 8, 2048), h=8192, I=28672, t=2, act="bf16", w="int8",
            std_x=1.0, std_gu=0.02, std_down=0.02, reduce_n=None),
    5: dict(name="llama405b_tp8_prefill", desc="405B-shaped TP=8 rank prefill",
            M=(8192,), h=16384, I=53248, t=8, act="bf16", w="bf16",
            std_x=1.0, std_gu=0.01, std_down=0.01, reduce_n=8192 * 16384),
}

TENSOR_X = 1
TENSOR_PARTIAL_BASE = 100

# Attention-block projections of one rank (Llama 3.1 70B: 64 query heads,
# 8 KV heads of size 128; "Constraints" section of the scalablesystem.dev page
# and "The KV cache splits too, until it doesn't" on the vidyal.ai page).
# O stands for the attention output of the rank's heads (the input of the
# output projection), drawn like X.
ATTN_CONFIGS = {
    6: dict(name="llama70b_tp8_attn", desc="70B-shaped TP=8 rank, attention projections",
            M=(1, 8, 64, 4096), h=8192, n_heads=64, n_kv_heads=8, head_dim=128, t=8,
            act="bf16", w="bf16", std_x=1.0, std_w=0.02),
    7: dict(name="llama70b_tp4_attn_fp8", desc="70B-shaped TP=4 rank, attention projections, fp8 weights",
            M=(32, 2048), h=8192, n_heads=64, n_kv_heads=8, head_dim=128, t=4,
            act="bf16", w="e4m3fn", std_x=1.0, std_w=0.02),
    8: dict(name="tiny_attn_t4", desc="tiny attention projections, t=4 (KV heads replicated)",
            M=(16,), h=256, n_heads=8, n_kv_heads=2, head_dim=32, t=4,
            act="f32", w="f32", std_x=1.0, std_w=1.0 / 16.0),
}

TENSOR_O = 7
TENSOR_WQ_FULL, TENSOR_WK_FULL, TENSOR_WV_FULL, TENSOR_WO_FULL = 200, 201, 202, 203


def tensor_id_qkv(k):
    return 5 + 10 * k


def tensor_id_o(k):
    return 6 + 10 * k


def tensor_id_gate(k):
    return 2 + 10 * k


def tensor_id_up(k):
    return 3 + 10 * k


def tensor_id_down(k):
    return 4 + 10 * k


def seed_of(config_id, tensor_id, weight_set=0):
    return 1000 * int(config_id) + int(tensor_id) + 1_000_000 * int(weight_set)


# ---------------------------------------------------------------------------
# draws and storage rounding
# ---------------------------------------------------------------------------

def draw_f32(seed, shape, std):
    """float32(std) * z with z ~ N(0, 1) float32 from PCG64(seed)."""
    n = int(np.prod(shape)) if len(shape) else 1
    z = np.random.Generator(np.random.PCG64(seed)).standard_normal(n, dtype=np.float32)
    w = np.float32(std) * z
    return w.reshape(shape)


def f32_to_bf16_bits(w):
    """Round binary32 values to bfloat16 (nearest, ties to even); uint16 bits.

    NaN inputs are not expected from Gaussian draws and are rejected.
    """
    w = np.ascontiguousarray(w, dtype=np.float32)
    if np.isnan(w).any():
        raise ValueError("NaN in bf16 rounding input")
    u = w.view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits):
    """Widen bf16 bits to float32 (exact); used to build reduce inputs etc."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


E4M3FN_MAX = np.float32(448.0)


def f32_to_e4m3fn(v):
    """Round float32 values (|v| <= 448) to OCP e4m3fn codes, nearest-even.

    Works on the magnitude: in the subnormal range (|v| < 2^-6) the step is
    2^-9 and the code is the rounded multiple (a result of 8 steps is the
    smallest normal, code 0x08, so the formula stays continuous); above it the
    value is split as 2^e * r / 8 with r rounded to an integer in [8, 16]
    (16 carries into the next binade).  Ties go to the even integer, which is
    the even mantissa.  The sign bit is copied (so -0 maps to 0x80).
    """
    v = np.asarray(v, dtype=np.float32)
    if np.isnan(v).any():
        raise ValueError("NaN in e4m3fn rounding input")
    a = np.abs(v).astype(np.float64)
    if (a > 448.0).any():
        raise ValueError("e4m3fn input out of range; clamp first")
    code = np.zeros(a.shape, dtype=np.int64)
    sub = a < 2.0 ** -6
    code[sub] = np.rint(a[sub] * 2.0 ** 9).astype(np.int64)
    nrm = ~sub
    if nrm.any():
        _, ex = np.frexp(a[nrm])          # a = f * 2^ex, f in [0.5, 1)
        e = ex.astype(np.int64) - 1       # 2^e <= a < 2^(e+1)
        r = np.rint(a[nrm] / np.ldexp(1.0, e - 3)).astype(np.int64)
        carry = r == 16
        e = np.where(carry, e + 1, e)
        r = np.where(carry, 8, r)
        code[nrm] = ((e + 7) << 3) | (r - 8)
    sign = np.signbit(v).astype(np.int64) << 7
    return (code | sign).astype(np.uint8)


def quantise_rows_e4m3fn(w):
    """Per-row (output channel) e4m3fn quantisation of an (out, in) float32 matrix.

    Returns (codes uint8 of w's shape, scales float32 of length rows).
    """
    w = np.asarray(w, dtype=np.float32)
    amax = np.max(np.abs(w), axis=1)
    s = (amax / E4M3FN_MAX).astype(np.float32)
    s = np.where(amax == 0, np.float32(1.0), s).astype(np.float32)
    scaled = (w / s[:, None]).astype(np.float32)
    scaled = np.clip(scaled, -E4M3FN_MAX, E4M3FN_MAX)
    return f32_to_e4m3fn(scaled), s


INT8_MAX = np.float32(127.0)


def quantise_rows_int8(w):
    """Per-row symmetric int8 quantisation of an (out, in) float32 matrix:
    s = float32(amax / 127) (1 for an all-zero row), q = round-half-even of
    float32(w / s) clamped to [-127, 127].  Returns (codes as uint8 bytes,
    scales float32)."""
    w = np.asarray(w, dtype=np.float32)
    amax = np.max(np.abs(w), axis=1)
    s = (amax / INT8_MAX).astype(np.float32)
    s = np.where(amax == 0, np.float32(1.0), s).astype(np.float32)
    scaled = (w / s[:, None]).astype(np.float32)
    q = np.clip(np.rint(scaled), -127, 127).astype(np.int8)
    return q.view(np.uint8), s


def to_storage(w32, dtype):
    """float32 draws -> storage dict for the given dtype."""
    if dtype == "f32":
        return dict(data=np.ascontiguousarray(w32, dtype=np.float32), scale=None)
    if dtype == "bf16":
        return dict(data=f32_to_bf16_bits(w32), scale=None)
    if dtype == "e4m3fn":
        q, s = quantise_rows_e4m3fn(w32)
        return dict(data=q, scale=s)
    if dtype == "int8":
        q, s = quantise_rows_int8(w32)
        return dict(data=q, scale=s)
    raise ValueError("unknown dtype %r" % (dtype,))


def _parallel(fn, items):
    """Map fn over items on a few threads (numpy releases the GIL in the draws)."""
    if len(items) <= 1:
        return [fn(i) for i in items]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(len(items), 8)) as ex:
        return list(ex.map(fn, items))


# ---------------------------------------------------------------------------
# tensors of a configuration
# ---------------------------------------------------------------------------

def make_x(config_id, M, h, dtype, std=1.0, weight_set=0):
    """Token activations X (M x h) in storage form (bf16 bits or float32)."""
    w = draw_f32(seed_of(config_id, TENSOR_X, weight_set), (M, h), std)
    return to_storage(w, dtype)["data"]


def make_shard_weights(config_id, h, I_s, k, dtype, std_gu, std_down, weight_set=0):
    """Rank k's shards drawn directly: W_gate_k, W_up_k (I_s x h), W_down_k (h x I_s).

    Returns a dict with storage arrays ``w_gate``, ``w_up``, ``w_down`` and,
    for e4m3fn, the scales ``s_gate`` (I_s), ``s_up`` (I_s), ``s_down`` (h).
    """
    jobs = [(tensor_id_gate(k), (I_s, h), std_gu), (tensor_id_up(k), (I_s, h), std_gu),
            (tensor_id_down(k), (h, I_s), std_down)]
    g, u, d = _parallel(lambda j: to_storage(draw_f32(seed_of(config_id, j[0], weight_set), j[1], j[2]), dtype),
                        jobs)
    return dict(w_gate=g["data"], w_up=u["data"], w_down=d["data"],
                s_gate=g["scale"], s_up=u["scale"], s_down=d["scale"])


def make_full_weights(config_id, h, I, dtype, std_gu, std_down, weight_set=0):
    """Full unsharded matrices (for the tiny split-against-unsplit case)."""
    return make_shard_weights(config_id, h, I, 0, dtype, std_gu, std_down, weight_set)


def make_partials(config_id, t, n, weight_set=0):
    """t float32 partial buffers of n elements, each N(0, 1)."""
    return _parallel(lambda j: draw_f32(seed_of(config_id, TENSOR_PARTIAL_BASE + j, weight_set), (n,), 1.0),
                     list(range(t)))


def attn_widths(n_heads, n_kv_heads, head_dim, t):
    """(n_loc, K_o): a rank's QKV output width and output-projection input
    width.  KV heads split over t, or one per rank when t is a multiple of
    their count."""
    q_loc = n_heads // t
    kv_loc = n_kv_heads // t if n_kv_heads % t == 0 else 1
    return (q_loc + 2 * kv_loc) * head_dim, q_loc * head_dim


def make_attn_weights(config_id, h, n_loc, k_o, k, dtype, std, weight_set=0):
    """Rank k's projection weights drawn directly: W_qkv_k (n_loc x h) and
    W_o_k (h x k_o), storage arrays plus (e4m3fn) per-row scales."""
    jobs = [(tensor_id_qkv(k), (n_loc, h)), (tensor_id_o(k), (h, k_o))]
    q, o = _parallel(lambda j: to_storage(draw_f32(seed_of(config_id, j[0], weight_set), j[1], std), dtype), jobs)
    return dict(w_qkv=q["data"], s_qkv=q["scale"], w_o=o["data"], s_o=o["scale"])


def make_attn_out_input(config_id, M, k_o, dtype, std=1.0, weight_set=0):
    """The output projection's input O_k (M x k_o) in storage form."""
    return to_storage(draw_f32(seed_of(config_id, TENSOR_O, weight_set), (M, k_o), std), dtype)["data"]


def make_attn_full_weights(config_id, h, n_heads, n_kv_heads, head_dim, dtype, std, weight_set=0):
    """Full W_q, W_k, W_v (per-head stacked rows, x h) and W_o (h x n_heads*d)
    for the split-against-unsplit case."""
    jobs = [(TENSOR_WQ_FULL, (n_heads * head_dim, h)), (TENSOR_WK_FULL, (n_kv_heads * head_dim, h)),
            (TENSOR_WV_FULL, (n_kv_heads * head_dim, h)), (TENSOR_WO_FULL, (h, n_heads * head_dim))]
    q, kk, v, o = _parallel(
        lambda j: to_storage(draw_f32(seed_of(config_id, j[0], weight_set), j[1], std), dtype), jobs)
    return dict(w_q=q["data"], w_k=kk["data"], w_v=v["data"], w_o=o["data"])


# ---------------------------------------------------------------------------
# accounting (algorithmic bytes and FLOPs; no arithmetic of the method)
# ---------------------------------------------------------------------------

BYTES = {"f32": 4, "bf16": 2, "e4m3fn": 1, "int8": 1}
SCALED = ("e4m3fn", "int8")    # one byte per weight + an fp32 scale per output row


def forward_flops(M, h, I_s):
    """Three GEMMs of 2*M*h*I_s each (gate, up, down)."""
    return 6 * int(M) * int(h) * int(I_s)


def forward_bytes(M, h, I_s, act="bf16", w="bf16"):
    """Algorithmic HBM bytes of one rank forward: weights + X + fp32 partial (+ scales).

    The intermediate activation A is not counted: a fully fused forward would
    not move it.
    """
    b = 3 * h * I_s * BYTES[w] + M * h * BYTES[act] + M * h * 4
    if w in SCALED:
        b += (2 * I_s + h) * 4
    return int(b)


def gateup_bytes(M, h, I_s, act="bf16", w="bf16"):
    """Algorithmic bytes of the gate/up phase: two weight shards, X, A written."""
    b = 2 * h * I_s * BYTES[w] + M * h * BYTES[act] + M * I_s * BYTES[act]
    if w in SCALED:
        b += 2 * I_s * 4
    return int(b)


def down_bytes(M, h, I_s, act="bf16", w="bf16"):
    """Algorithmic bytes of the down phase: down shard, A read, P written."""
    b = h * I_s * BYTES[w] + M * I_s * BYTES[act] + M * h * 4
    if w in SCALED:
        b += h * 4
    return int(b)


def reduce_bytes(n, t):
    """t fp32 reads plus one fp32 write per element."""
    return int((t + 1) * 4 * n)


def linear_flops(M, N, K):
    return 2 * int(M) * int(N) * int(K)


def linear_bytes(M, N, K, act="bf16", w="bf16", out="bf16"):
    """Algorithmic bytes of one projection: weight, input and output once
    (+ per-row scales for one-byte weights)."""
    b = N * K * BYTES[w] + M * K * BYTES[act] + M * N * BYTES[out]
    if w in SCALED:
        b += N * 4
    return int(b)
