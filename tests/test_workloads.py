"""Input recipe and accounting checks (host only)."""

import numpy as np

from conftest import read_golden
import workloads


def test_draws_are_seeded_and_distinct():
    a = workloads.draw_f32(workloads.seed_of(2, 1), (4, 8), 1.0)
    b = workloads.draw_f32(workloads.seed_of(2, 1), (4, 8), 1.0)
    c = workloads.draw_f32(workloads.seed_of(2, 2), (4, 8), 1.0)
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    assert workloads.seed_of(3, 4, 1) != workloads.seed_of(3, 4, 0)


def test_shard_weight_shapes_and_dtypes():
    w = workloads.make_shard_weights(4, 64, 32, 1, "e4m3fn", 0.02, 0.02)
    assert w["w_gate"].shape == (32, 64) and w["w_gate"].dtype == np.uint8
    assert w["w_down"].shape == (64, 32)
    assert w["s_gate"].shape == (32,) and w["s_down"].shape == (64,)
    w = workloads.make_shard_weights(2, 64, 32, 0, "bf16", 0.02, 0.02)
    assert w["w_up"].dtype == np.uint16 and w["s_up"] is None


def test_draw_statistics():
    w = workloads.draw_f32(1, (200000,), 0.02)
    assert abs(w.mean()) < 2e-4 and abs(w.std() - 0.02) < 2e-4


def test_flops_pinned_to_page_figure():
    fig = {r[0]: float(r[1]) for r in read_golden("page_figures.txt")}
    # one GEMM of the worked example: tokens = b * s = 32 * 2048, h = 8192, I_s = 28672 / 8
    one_gemm = workloads.forward_flops(32 * 2048, 8192, 28672 // 8) // 3
    assert one_gemm == fig["gemm_flops_b32_s2048_h8192_ffn28672_t8"]


def test_partial_message_size_pinned_to_page_figure():
    fig = {r[0]: float(r[1]) for r in read_golden("page_figures.txt")}
    h = workloads.CONFIGS[2]["h"]
    # one token's partial in the pages' bf16 wire format; this library keeps fp32 (twice that)
    assert h * workloads.BYTES["bf16"] == fig["allreduce_bytes_per_token_bf16"]
    assert fig["allreduces_per_token"] * fig["allreduce_bytes_per_token_bf16"] == fig["reduced_bytes_per_token"]
    assert abs(fig["weights_bytes_70b_gb"] / 8 - fig["weights_bytes_per_gpu_tp8_gb"]) < 0.05


def test_decode_bytes():
    # 3 shards of 8192 x 3584 bf16 + X (M x 8192 bf16) + P (M x 8192 fp32)
    assert workloads.forward_bytes(1, 8192, 3584) == 176209920
    assert workloads.forward_bytes(64, 8192, 3584) == 179306496
    assert workloads.gateup_bytes(1, 8192, 3584) + workloads.down_bytes(1, 8192, 3584) == \
        workloads.forward_bytes(1, 8192, 3584) + 2 * 3584 * 2
    assert workloads.reduce_bytes(4096 * 8192, 8) == 1207959552
