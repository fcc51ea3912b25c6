"""GPU parity of tp_mlp_shard_forward against the float64 oracle.

Metric: max |P_gpu - P_ref| / rms(P_ref) with the tolerances of the contract
(2e-2 bf16 and fp32, 6e-2 fp8 weights against the dequantised reference).
Small shapes span several tiles with ragged tails in M and N and are checked
element by element, and so are the configurations at their full sizes
(decode and prefill: every tile and every stream-K tail tile of the launch
the benchmark times).
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
import tensor_transformer_mlp_tp_amd as tp
from helpers import TOL_BF16, TOL_FP8, TOL_INT8, make_case, upload_case, oracle_partial, to_device

pytestmark = pytest.mark.gpu


def run_forward(d, t, k):
    p = tp.shard_forward(d["x"], d["w_gate"], d["w_up"], d["w_down"], t=t, k=k,
                         s_gate=d["s_gate"], s_up=d["s_up"], s_down=d["s_down"])
    torch.cuda.synchronize()
    return p


def check(p_gpu, ref, tol, label):
    err = oracle.rms_normalised_max_error(p_gpu, ref)
    print("%s: err=%.3e (tol %.0e)" % (label, err, tol), flush=True)
    assert np.all(np.isfinite(p_gpu)), label
    assert err <= tol, (label, err)
    return err


# ------------------------------------------------------------ tiny config: split vs unsplit

def test_tiny_t4_all_shards_sum_to_unsplit():
    c = workloads.CONFIGS[1]
    M, h, I, t = c["M"][0], c["h"], c["I"], c["t"]
    x = workloads.make_x(1, M, h, "f32")
    full = workloads.make_full_weights(1, h, I, "f32", c["std_gu"], c["std_down"])
    xd = to_device(x, "f32")
    parts = []
    for k in range(t):
        wg, wu, wd = oracle.shard_of_full(full["w_gate"], full["w_up"], full["w_down"], t, k)
        wd = np.ascontiguousarray(wd)
        p = tp.shard_forward(xd, to_device(wg, "f32"), to_device(wu, "f32"), to_device(wd, "f32"), t=t, k=k)
        torch.cuda.synchronize()
        ref_k = oracle.rank_partial_from_storage(x, "f32", wg, wu, wd, "f32")
        check(p.cpu().numpy(), ref_k, TOL_BF16, "tiny shard %d" % k)
        parts.append(p)
    y = tp.partial_reduce(parts)
    torch.cuda.synchronize()
    y_ref = oracle.mlp_full(x, full["w_gate"], full["w_up"], full["w_down"])
    err = check(y.cpu().numpy(), y_ref, TOL_BF16, "tiny sum of shards vs unsplit")
    assert err < 1e-4   # fp32 arithmetic: expected ~1e-6
    # the reduce is the left fold of exactly these partials
    fold = oracle.fold_fp32([p.cpu().numpy() for p in parts])
    assert np.array_equal(y.cpu().numpy().view(np.uint32), fold.view(np.uint32))


# ------------------------------------------------------------ small shapes, many tiles, ragged

DECODE_M = [1, 2, 5, 8, 15, 16, 17, 31, 33, 48, 63, 64]
PREFILL_M = [65, 200, 256, 257, 300, 513]


@pytest.mark.parametrize("M", DECODE_M + PREFILL_M)
@pytest.mark.parametrize("w", ["bf16", "e4m3fn", "int8"])
def test_small_shapes(M, w):
    # h = 320 (256-wide down tiles: 1 full + a ragged one), I_s = 192 (128-channel
    # gate/up tiles: 1 full + a ragged one)
    h, I_s, t, k = 320, 192, 4, 1
    print("small shape M=%d w=%s" % (M, w), flush=True)
    x, ws = make_case(40, M, h, I_s, "bf16", w, 0.05, 0.05, k=k, weight_set=M)
    d = upload_case(x, ws, "bf16", w)
    p = run_forward(d, t, k).cpu().numpy()
    tol = {"bf16": TOL_BF16, "e4m3fn": TOL_FP8, "int8": TOL_INT8}[w]
    check(p, oracle_partial(x, ws, "bf16", w), tol, "M=%d %s" % (M, w))


@pytest.mark.parametrize("M", [1, 64, 300])
def test_fp32_path_general_shapes(M):
    # fp32 path accepts any h and I_s
    h, I_s, t = 100, 36, 3
    x = workloads.make_x(41, M, h, "f32")
    ws = workloads.make_shard_weights(41, h, I_s, 2, "f32", 0.1, 0.1)
    d = upload_case(x, ws, "f32", "f32")
    p = run_forward(d, t, 2).cpu().numpy()
    err = check(p, oracle_partial(x, ws, "f32", "f32"), TOL_BF16, "fp32 M=%d" % M)
    assert err < 1e-4


def test_k_independence_and_determinism():
    M, h, I_s, t = 37, 256, 128, 4
    x, ws = make_case(42, M, h, I_s, "bf16", "bf16", 0.05, 0.05)
    d = upload_case(x, ws, "bf16", "bf16")
    outs = [run_forward(d, t, k).cpu().numpy() for k in (0, 3, 0)]
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
    assert np.array_equal(outs[0].view(np.uint32), outs[2].view(np.uint32))
    for M2 in (300,):
        x, ws = make_case(42, M2, h, I_s, "bf16", "bf16", 0.05, 0.05)
        d = upload_case(x, ws, "bf16", "bf16")
        a, b = run_forward(d, t, 0).cpu().numpy(), run_forward(d, t, 2).cpu().numpy()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_strided_views_of_full_matrices():
    # a caller holding full matrices passes row / column offsets with leading dimensions
    M, h, I, t, k = 20, 128, 512, 4, 2
    I_s = I // t
    x = workloads.make_x(43, M, h, "bf16")
    full = workloads.make_full_weights(43, h, I, "bf16", 0.05, 0.05)
    xd = to_device(x, "bf16")
    G, U, D = (to_device(full[n], "bf16") for n in ("w_gate", "w_up", "w_down"))
    s = slice(k * I_s, (k + 1) * I_s)
    p = tp.shard_forward(xd, G[s], U[s], D[:, s], t=t, k=k)
    torch.cuda.synchronize()
    wg, wu, wd = oracle.shard_of_full(full["w_gate"], full["w_up"], full["w_down"], t, k)
    ref = oracle.rank_partial_from_storage(x, "bf16", wg, wu, np.ascontiguousarray(wd), "bf16")
    check(p.cpu().numpy(), ref, TOL_BF16, "strided shard views")
    for M2 in (300,):
        x2 = workloads.make_x(44, M2, h, "bf16")
        p = tp.shard_forward(to_device(x2, "bf16"), G[s], U[s], D[:, s], t=t, k=k)
        torch.cuda.synchronize()
        ref = oracle.rank_partial_from_storage(x2, "bf16", wg, wu, np.ascontiguousarray(wd), "bf16")
        check(p.cpu().numpy(), ref, TOL_BF16, "strided shard views prefill")


def test_extreme_activations():
    # large pre-activations exercise the SiLU limits (-0 below about -88, identity above)
    M, h, I_s, t = 16, 128, 64, 2
    x = workloads.f32_to_bf16_bits(np.full((M, h), 1.0, np.float32))
    w32 = np.zeros((I_s, h), np.float32)
    w32[: I_s // 2, :] = 1.0      # gate = +128 for the first half of the channels
    w32[I_s // 2:, :] = -1.0      # gate = -128 for the second half
    wg = workloads.f32_to_bf16_bits(w32)
    wu = workloads.f32_to_bf16_bits(np.full((I_s, h), 0.5, np.float32))
    wd = workloads.f32_to_bf16_bits(np.full((h, I_s), 0.25, np.float32))
    ws = dict(w_gate=wg, w_up=wu, w_down=wd, s_gate=None, s_up=None, s_down=None)
    for M2 in (M, 100):
        xx = workloads.f32_to_bf16_bits(np.full((M2, h), 1.0, np.float32))
        d = upload_case(xx, ws, "bf16", "bf16")
        p = run_forward(d, t, 0).cpu().numpy()
        ref = oracle_partial(xx, ws, "bf16", "bf16")
        check(p, ref, TOL_BF16, "extreme M=%d" % M2)


# ------------------------------------------------------------ the configurations at full size

def _full_decode(cfg, M):
    c = workloads.CONFIGS[cfg]
    I_s = c["I"] // c["t"]
    print("config %d decode M=%d" % (cfg, M), flush=True)
    x, ws = make_case(cfg, M, c["h"], I_s, c["act"], c["w"], c["std_gu"], c["std_down"])
    d = upload_case(x, ws, c["act"], c["w"])
    p = run_forward(d, c["t"], 0).cpu().numpy()
    tol = TOL_FP8 if c["w"] == "e4m3fn" else TOL_BF16
    check(p, oracle_partial(x, ws, c["act"], c["w"]), tol, "config %d M=%d (all elements)" % (cfg, M))


@pytest.mark.parametrize("M", [1, 8, 64])
def test_config2_decode_full(M):
    _full_decode(2, M)


def test_config4_fp8_decode_full():
    _full_decode(4, 32)


def _full_prefill(cfg, M):
    """Every element of the configuration's prefill partial against the fp64
    oracle (several seconds of host BLAS at these sizes), then a second call
    for determinism."""
    c = workloads.CONFIGS[cfg]
    I_s = c["I"] // c["t"]
    print("config %d prefill M=%d" % (cfg, M), flush=True)
    x, ws = make_case(cfg, M, c["h"], I_s, c["act"], c["w"], c["std_gu"], c["std_down"])
    d = upload_case(x, ws, c["act"], c["w"])
    p = run_forward(d, c["t"], 0)
    got = p.cpu().numpy()
    assert np.all(np.isfinite(got))
    p2 = run_forward(d, c["t"], 0)
    assert torch.equal(p.view(torch.int32), p2.view(torch.int32))
    del p2, d
    tol = TOL_FP8 if c["w"] == "e4m3fn" else TOL_BF16
    print("config %d prefill M=%d: oracle on all rows" % (cfg, M), flush=True)
    check(got, oracle_partial(x, ws, c["act"], c["w"]), tol, "config %d M=%d (all elements)" % (cfg, M))


def test_config3_prefill_full():
    _full_prefill(3, 4096)


def test_config4_fp8_prefill_full():
    _full_prefill(4, 2048)


def test_config5_prefill_full():
    _full_prefill(5, 8192)


@pytest.mark.parametrize("cfg,M", [
    (3, 300),    # 70B shard: both GEMMs on 128-token tiles, gate/up tiles in 3 stream-K pieces, down in 2
    (3, 100),    # ... 64-token tiles (2 x 28 gate/up tiles in 4 pieces)
    (4, 48),     # fp8 weights above 32 tokens: 64-token prefill tiles instead of the decode kernels
])
def test_full_shape_short_tiles(cfg, M):
    _full_prefill(cfg, M)


# ------------------------------------------------------------ 256 x 256 tiles (enough tiles to fill the chip)

@pytest.mark.parametrize("M,h,I_s", [
    (2048, 512, 3072),    # gate/up: 8 x 24 = 192 tiles of 256 x 256; down on shorter tiles
    (2000, 512, 3136),    # gate/up: ragged last M-tile (208 tokens) and last channel tile (64 of 128)
    (2048, 6144, 256),    # down: 8 x 24 = 192 tiles; K = 256
    (1900, 6464, 320),    # down: ragged M-tile (108 tokens) and feature tile (64 of 256), K = 320
])
def test_full_tiles_ragged(M, h, I_s):
    print("256x256 tiles M=%d h=%d I_s=%d" % (M, h, I_s), flush=True)
    x, ws = make_case(49, M, h, I_s, "bf16", "bf16", 0.05, 0.05, weight_set=M)
    d = upload_case(x, ws, "bf16", "bf16")
    p = run_forward(d, 2, 0)
    p2 = run_forward(d, 2, 1)
    assert torch.equal(p.view(torch.int32), p2.view(torch.int32))
    check(p.cpu().numpy(), oracle_partial(x, ws, "bf16", "bf16"), TOL_BF16, "256x256 M=%d h=%d I_s=%d" % (M, h, I_s))


# ------------------------------------------------------------ stream-K tail of the prefill GEMMs

@pytest.mark.parametrize("M,h,I_s", [
    (300, 2112, 2112),   # both GEMMs: every tile cut along K in 2 uneven pieces (33 k-tiles); ragged tiles
    (65, 8192, 448),     # gate/up: 4 tiles (the last ragged) cut in 5 pieces; down whole
    (600, 1024, 4096),   # down: 12 tiles in 4 pieces; gate/up whole
    (600, 2048, 2048),   # gate/up: 128-token tiles (5 x 16) in 2 pieces; down: 64-token tiles in 2 pieces
])
@pytest.mark.parametrize("w", ["bf16", "e4m3fn", "int8"])
def test_stream_k_tail(M, h, I_s, w):
    """Tiles cut along K: the last piece to arrive adds the pieces' fp32 slots
    in k order.  The arrival counters live in the workspace, whose contents
    on entry must not matter, and the result must not depend on which piece
    arrives last (bit-identical over calls)."""
    t = 2
    print("stream-K M=%d h=%d I_s=%d w=%s" % (M, h, I_s, w), flush=True)
    x, ws = make_case(45, M, h, I_s, "bf16", w, 0.05, 0.05, weight_set=M)
    d = upload_case(x, ws, "bf16", w)
    nbytes = tp.workspace_bytes(M, h, I_s * t, t, torch.bfloat16, d["w_gate"].dtype)
    assert nbytes > M * I_s * 2 + 256      # the stream-K scratch is part of it
    scratch = tp.alloc_workspace(nbytes, "cuda")
    outs = []
    for fill in (0x7F, 0x00, 0xFF):
        scratch.fill_(fill)
        outs.append(tp.shard_forward(d["x"], d["w_gate"], d["w_up"], d["w_down"], t=t, k=0, s_gate=d["s_gate"],
                                     s_up=d["s_up"], s_down=d["s_down"], workspace=scratch))
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int32), outs[0].view(torch.int32))
    tol = {"bf16": TOL_BF16, "e4m3fn": TOL_FP8, "int8": TOL_INT8}[w]
    check(outs[0].cpu().numpy(), oracle_partial(x, ws, "bf16", w), tol, "stream-K M=%d %s" % (M, w))


def test_stream_k_runs_across_tiles():
    """256-token tiles past the last whole round cut along K: gate/up has 10 x
    32 = 320 tiles (64 past the round, each in 4 pieces of 32 of its 128
    k-tiles) and down 10 x 32 = 320 (64 in 4 pieces of 16 of 64); the last
    token tile is ragged.  The arrival counters and piece slots live in the
    workspace, whose contents on entry must not matter, and the result must
    not depend on which piece arrives last (bit-identical over calls)."""
    M, h, I_s, t = 2500, 8192, 4096, 2
    print("stream-K runs M=%d h=%d I_s=%d" % (M, h, I_s), flush=True)
    x, ws = make_case(50, M, h, I_s, "bf16", "bf16", 0.02, 0.02)
    d = upload_case(x, ws, "bf16", "bf16")
    nbytes = tp.workspace_bytes(M, h, I_s * t, t)
    assert nbytes >= M * I_s * 2 + 256 * 256 * 256 * 4        # counters and 256 piece slots
    scratch = tp.alloc_workspace(nbytes, "cuda")
    outs = []
    for fill in (0x7F, 0x00, 0xFF):
        scratch.fill_(fill)
        outs.append(tp.shard_forward(d["x"], d["w_gate"], d["w_up"], d["w_down"], t=t, k=0, workspace=scratch))
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int32), outs[0].view(torch.int32))
    check(outs[0].cpu().numpy(), oracle_partial(x, ws, "bf16", "bf16"), TOL_BF16, "stream-K runs (all elements)")


def test_stream_k_tail_after_whole_rounds():
    """More tiles than CUs: gate/up has 17 x 16 = 272 tiles, 256 computed whole
    and the 16 of the last (ragged) M-tile cut in 2 pieces; every element."""
    M, h, I_s, t = 4300, 2048, 2048, 2
    print("stream-K after whole rounds M=%d" % M, flush=True)
    x, ws = make_case(46, M, h, I_s, "bf16", "bf16", 0.05, 0.05)
    d = upload_case(x, ws, "bf16", "bf16")
    p = run_forward(d, t, 0)
    check(p.cpu().numpy(), oracle_partial(x, ws, "bf16", "bf16"), TOL_BF16, "M=%d (all elements)" % M)
    p2 = run_forward(d, t, 0)
    assert torch.equal(p.view(torch.int32), p2.view(torch.int32))


# ------------------------------------------------------------ streaming decode path, several slots per wave

@pytest.mark.parametrize("M", [1, 7, 8, 12, 13, 16, 33, 64])
@pytest.mark.parametrize("w", ["bf16", "e4m3fn"])
def test_stream_decode_shapes(M, w):
    # h and I_s multiples of the slot width (128 bf16 / 256 fp8 k-values) take
    # the streaming kernels; uneven slot counts per wave, ragged token blocks.
    # bf16 up to 16 tokens: one row block per wave below 8 tokens (gate/up) /
    # 13 tokens (down), two from there; the packed layout gives the same bits.
    h, I_s = (512, 640) if w == "bf16" else (1024, 1280)
    print("stream decode M=%d w=%s" % (M, w), flush=True)
    x, ws = make_case(45, M, h, I_s, "bf16", w, 0.05, 0.05, weight_set=M)
    d = upload_case(x, ws, "bf16", w)
    ref = oracle_partial(x, ws, "bf16", w)
    outs = []
    for rep in range(3):   # repeated calls give identical bits
        outs.append(run_forward(d, 4, 1).cpu().numpy())
    check(outs[0], ref, TOL_FP8 if w == "e4m3fn" else TOL_BF16, "stream M=%d %s" % (M, w))
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
    assert np.array_equal(outs[0].view(np.uint32), outs[2].view(np.uint32))
    if w == "bf16" or M <= 32:
        pk = tp.pack_weights(d["w_gate"], d["w_up"], d["w_down"], t=4)
        pp = tp.shard_forward_packed(d["x"], pk, k=1, s_gate=d["s_gate"], s_up=d["s_up"], s_down=d["s_down"])
        torch.cuda.synchronize()
        assert np.array_equal(pp.cpu().numpy().view(np.uint32), outs[0].view(np.uint32))


# ------------------------------------------------------------ decode split-K streams

# bf16 weights at 49-64 tokens and one-byte weights at 17-32 take the split-K
# streams: tiles of 112 (gate/up) or 128 (down) weight rows, K cut into
# ranges whose fp32 sums the last range to arrive adds in order.  (gate/up
# tiles x ranges, down tiles x ranges; steps of 32 k bf16 / 64 k one-byte.)
SK_CASES = [
    (64, 8192, 448, "bf16"),      # 8 x 32 ranges of 8 steps; 64 x 4 ranges of 3-4 steps
    (57, 1088, 3584, "bf16"),     # 64 x 4 of 8-9; ragged 9 x 28 of 4 (1088 rows = 8.5 tiles)
    (64, 256, 14336, "bf16"),     # 256 whole tiles (no split); 2 x 128 ranges of 3-4 steps
    (32, 2048, 1024, "e4m3fn"),   # ragged 19 x 13 of 2-3 (2048 rows = 18.3 tiles); 16 x 16 of 1
    (17, 2048, 1024, "int8"),
]


@pytest.mark.parametrize("M,h,I_s,w", SK_CASES)
def test_decode_split_k(M, h, I_s, w):
    """Every element against the oracle; the arrival counters and range slots
    live in the workspace, whose contents on entry must not matter, and the
    result must not depend on which range arrives last (bit-identical over
    calls with a dirtied workspace)."""
    t = 2
    print("decode split-K M=%d h=%d I_s=%d w=%s" % (M, h, I_s, w), flush=True)
    x, ws = make_case(62, M, h, I_s, "bf16", w, 0.05, 0.05, weight_set=M)
    d = upload_case(x, ws, "bf16", w)
    nbytes = tp.workspace_bytes(M, h, I_s * t, t, w_dtype=d["w_gate"].dtype)
    assert nbytes > M * I_s * 2     # counters and range slots past A
    scratch = tp.alloc_workspace(nbytes, "cuda")
    outs = []
    for fill in (0x7F, 0x00, 0xFF):
        scratch.fill_(fill)
        outs.append(tp.shard_forward(d["x"], d["w_gate"], d["w_up"], d["w_down"], t=t, k=0, s_gate=d["s_gate"],
                                     s_up=d["s_up"], s_down=d["s_down"], workspace=scratch))
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int32), outs[0].view(torch.int32))
    tol = {"bf16": TOL_BF16, "e4m3fn": TOL_FP8, "int8": TOL_INT8}[w]
    check(outs[0].cpu().numpy(), oracle_partial(x, ws, "bf16", w), tol, "split-K M=%d %s (all elements)" % (M, w))


def test_prefill_stream_k_in_a_graph():
    """A prefill forward whose GEMMs have stream-K tails, captured in a HIP
    graph: the arrival counters are cleared by a kernel inside the graph, so
    every replay (with eager work and a dirtied workspace in between) must
    equal the eager result bit for bit."""
    M, h, I_s, t = 300, 2112, 2112, 2
    x, ws = make_case(48, M, h, I_s, "bf16", "bf16", 0.05, 0.05)
    d = upload_case(x, ws, "bf16", "bf16")
    ref = run_forward(d, t, 0).clone()
    scratch = tp.alloc_workspace(tp.workspace_bytes(M, h, I_s * t, t), "cuda")
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        call = tp.prepare_shard_forward(d["x"], d["w_gate"], d["w_up"], d["w_down"], t=t, k=0, workspace=scratch)
        call()   # warm-up outside capture
        s.synchronize()
        with torch.cuda.graph(g, stream=s):
            call()
    for i in range(4):
        scratch.fill_(0x7F if i % 2 else 0xFF)          # counters and slots hold garbage
        call.partial.zero_()
        other = run_forward(d, t, 1)                     # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(call.partial.view(torch.int32), ref.view(torch.int32)), i
        assert torch.equal(other.view(torch.int32), ref.view(torch.int32)), i   # k does not change P's value


def test_decode_many_calls_and_graph():
    # many calls on two streams in turn, then a captured graph replayed
    M, h, I_s = 8, 512, 512
    x, ws = make_case(46, M, h, I_s, "bf16", "bf16", 0.05, 0.05)
    d = upload_case(x, ws, "bf16", "bf16")
    ref = run_forward(d, 2, 0).clone()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [torch.empty_like(ref) for _ in range(2)]
    for i in range(150):
        s = streams[i % 2]
        with torch.cuda.stream(s):
            tp.shard_forward(d["x"], d["w_gate"], d["w_up"], d["w_down"], t=2, k=0, partial=outs[i % 2])
        s.synchronize()
        assert torch.equal(outs[i % 2].view(torch.int32), ref.view(torch.int32)), i
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        # a prepared call is bound to the stream current when it is prepared
        call = tp.prepare_shard_forward(d["x"], d["w_gate"], d["w_up"], d["w_down"], t=2, k=0)
        call()   # warm-up outside capture
        s.synchronize()
        call.partial.zero_()
        with torch.cuda.graph(g, stream=s):
            call()
    for i in range(5):
        call.partial.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(call.partial.view(torch.int32), ref.view(torch.int32)), i
