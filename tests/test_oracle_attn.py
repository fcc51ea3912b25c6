"""Pins for the oracle's attention-block projections (``oracle/attn.py``).

Independent of the oracle's own code path: a hand-worked example, head
counts and KV-cache bytes printed on the pages, closed forms with one-hot
weights, pure-Python brute force, and the split-equals-unsplit invariant
(sum of the output-projection partials; reassembly of the QKV columns).
"""

import itertools

import numpy as np
import pytest

from conftest import read_golden
import oracle
import workloads


def _worked():
    rows = {r[0]: [float(v) for v in r[1:]] for r in read_golden("tiny_attn_worked.txt")}
    x = np.array(rows["X"]).reshape(1, 3)
    wq = np.array(rows["W_q"]).reshape(4, 3)
    wk = np.array(rows["W_k"]).reshape(2, 3)
    wv = np.array(rows["W_v"]).reshape(2, 3)
    o = np.array(rows["O"]).reshape(1, 4)
    wo = np.array(rows["W_o"]).reshape(3, 4)
    return x, wq, wk, wv, o, wo, rows


@pytest.mark.parametrize("t", [2, 4])
def test_hand_worked_qkv(t):
    x, wq, wk, wv, _, _, rows = _worked()
    for k in range(t):
        w = oracle.qkv_rank_weight(wq, wk, wv, 4, 2, 1, t, k)
        got = oracle.linear(x, w)[0]
        assert got.tolist() == rows["QKV_t%d_%d" % (t, k)]


@pytest.mark.parametrize("t", [2, 4])
def test_hand_worked_o_proj(t):
    _, _, _, _, o, wo, rows = _worked()
    q_loc = 4 // t
    total = np.zeros(3)
    for k in range(t):
        p = oracle.linear(o[:, k * q_loc:(k + 1) * q_loc], oracle.o_proj_rank_weight(wo, 4, 1, t, k))[0]
        assert p.tolist() == rows["P_t%d_%d" % (t, k)]
        total += p
    assert total.tolist() == rows["Y"]
    assert oracle.linear(o, wo)[0].tolist() == rows["Y"]


# ------------------------------------------------------- page head counts

def _fig():
    return {r[0]: [float(v) for v in r[1:]] for r in read_golden("attn_heads.txt")}


def test_page_head_counts_70b():
    fig = _fig()
    q, kv = oracle.local_heads(64, 8, 8, 0)
    assert len(q) == fig["q_heads_per_gpu_tp8"][0]
    assert len(kv) == fig["kv_heads_per_gpu_tp8"][0]
    # KV bytes per token per GPU: K and V, 80 layers, its KV heads, head size 128, 2 bytes
    per_head = 2 * 80 * 128 * 2
    assert per_head * 8 == fig["kv_bytes_per_token_unsharded"][0]
    for t, key in ((8, "kv_bytes_per_token_tp8_gpu"), (16, "kv_bytes_per_token_tp16_gpu")):
        for k in range(t):
            assert per_head * len(oracle.local_heads(64, 8, t, k)[1]) == fig[key][0]
    group = sum(per_head * len(oracle.local_heads(64, 8, 16, k)[1]) for k in range(16))
    assert group == fig["kv_bytes_per_token_tp16_group"][0]
    # each KV head sits on the stated number of GPUs at TP = 16
    owners = {}
    for k in range(16):
        for j in oracle.local_heads(64, 8, 16, k)[1]:
            owners.setdefault(j, []).append(k)
    assert sorted(owners) == list(range(8))
    assert all(len(v) == fig["kv_replicas_tp16"][0] for v in owners.values())


def test_page_allowed_tp_sizes():
    allowed = []
    for t in range(1, 65):
        try:
            oracle.local_heads(64, 8, t, 0)
            allowed.append(t)
        except ValueError:
            pass
    assert allowed == [int(v) for v in _fig()["allowed_tp_64_heads"]]
    with pytest.raises(ValueError):
        oracle.local_heads(40, 8, 16, 0)   # 40 / 16 is not an integer


# ------------------------------------------------- closed forms, invariants

def _rand(seed, shape):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape)


@pytest.mark.parametrize("nh,nkv,d,t", [(8, 2, 3, 2), (8, 2, 3, 4), (8, 8, 2, 4), (12, 4, 2, 2), (6, 1, 2, 3)])
def test_one_hot_weights_select_inputs(nh, nkv, d, t):
    """W row r = e_{f(r)}: output column c of a rank is X[:, f(its global row)]."""
    h = 29
    x = _rand(1, (3, h))
    fq = lambda r: (5 * r + 1) % h
    fk = lambda r: (7 * r + 2) % h
    fv = lambda r: (11 * r + 3) % h
    wq = np.zeros((nh * d, h)); wq[np.arange(nh * d), [fq(r) for r in range(nh * d)]] = 1
    wk = np.zeros((nkv * d, h)); wk[np.arange(nkv * d), [fk(r) for r in range(nkv * d)]] = 1
    wv = np.zeros((nkv * d, h)); wv[np.arange(nkv * d), [fv(r) for r in range(nkv * d)]] = 1
    q_loc = nh // t
    for k in range(t):
        out = oracle.linear(x, oracle.qkv_rank_weight(wq, wk, wv, nh, nkv, d, t, k))
        kv_heads = list(range(k * nkv // t, (k + 1) * nkv // t)) if nkv % t == 0 else [k * nkv // t]
        cols = [fq(r) for r in range(k * q_loc * d, (k + 1) * q_loc * d)]
        cols += [fk(j * d + i) for j in kv_heads for i in range(d)]
        cols += [fv(j * d + i) for j in kv_heads for i in range(d)]
        assert np.array_equal(out, x[:, cols])


def test_brute_force_linear():
    a = _rand(2, (3, 5))
    w = _rand(3, (4, 5))
    got = oracle.linear(a, w)
    for m, n in itertools.product(range(3), range(4)):
        s = 0.0
        for i in range(5):
            s += a[m, i] * w[n, i]
        assert got[m, n] == pytest.approx(s, rel=1e-14, abs=1e-14)


@pytest.mark.parametrize("nh,nkv,t", [(8, 2, 2), (8, 2, 4), (8, 2, 8), (16, 4, 4), (4, 4, 1)])
def test_rank_outputs_reassemble_unsharded(nh, nkv, t):
    d, h, M = 4, 24, 5
    x = _rand(4, (M, h))
    wq, wk, wv = _rand(5, (nh * d, h)), _rand(6, (nkv * d, h)), _rand(7, (nkv * d, h))
    q_full, k_full, v_full = x @ wq.T, x @ wk.T, x @ wv.T
    q_loc = nh // t
    qs, ks, vs = [], [], []
    for k in range(t):
        out = oracle.linear(x, oracle.qkv_rank_weight(wq, wk, wv, nh, nkv, d, t, k))
        kv_w = (out.shape[1] - q_loc * d) // 2
        qs.append(out[:, :q_loc * d])
        ks.append(out[:, q_loc * d:q_loc * d + kv_w])
        vs.append(out[:, q_loc * d + kv_w:])
    np.testing.assert_allclose(np.concatenate(qs, 1), q_full, rtol=1e-12, atol=1e-12)
    if nkv % t == 0:
        np.testing.assert_allclose(np.concatenate(ks, 1), k_full, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(np.concatenate(vs, 1), v_full, rtol=1e-12, atol=1e-12)
    else:
        rep = t // nkv
        for k in range(t):
            j = k // rep
            np.testing.assert_allclose(ks[k], k_full[:, j * d:(j + 1) * d], rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(vs[k], v_full[:, j * d:(j + 1) * d], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("nh,t", [(8, 2), (8, 8), (12, 3), (4, 1)])
def test_o_proj_partials_sum_to_unsharded(nh, t):
    d, h, M = 3, 10, 4
    o = _rand(8, (M, nh * d))
    wo = _rand(9, (h, nh * d))
    q_loc = nh // t
    parts = [oracle.linear(o[:, k * q_loc * d:(k + 1) * q_loc * d], oracle.o_proj_rank_weight(wo, nh, d, t, k))
             for k in range(t)]
    np.testing.assert_allclose(sum(parts), o @ wo.T, rtol=1e-12, atol=1e-12)


def test_rank_depends_only_on_its_heads():
    nh, nkv, d, t, h = 8, 4, 2, 4, 12
    x = _rand(10, (2, h))
    wq, wk, wv = _rand(11, (nh * d, h)), _rand(12, (nkv * d, h)), _rand(13, (nkv * d, h))
    k = 1
    base = oracle.linear(x, oracle.qkv_rank_weight(wq, wk, wv, nh, nkv, d, t, k))
    wq2 = wq.copy(); wq2[0:d] += 1.0          # query head 0 belongs to rank 0
    wk2 = wk.copy(); wk2[0:d] += 1.0          # KV head 0 belongs to rank 0
    assert np.array_equal(base, oracle.linear(x, oracle.qkv_rank_weight(wq2, wk2, wv, nh, nkv, d, t, k)))
    wq3 = wq.copy(); wq3[2 * d] += 1.0        # query head 2 belongs to rank 1
    assert not np.array_equal(base, oracle.linear(x, oracle.qkv_rank_weight(wq3, wk, wv, nh, nkv, d, t, k)))
    wv3 = wv.copy(); wv3[d] += 1.0            # KV head 1 belongs to rank 1
    assert not np.array_equal(base, oracle.linear(x, oracle.qkv_rank_weight(wq, wk, wv3, nh, nkv, d, t, k)))


def test_linear_from_storage_decodes_formats():
    a = workloads.draw_f32(1, (3, 64), 1.0)
    w = workloads.draw_f32(2, (5, 64), 0.02)
    ab = workloads.f32_to_bf16_bits(a)
    wb = workloads.f32_to_bf16_bits(w)
    # bf16 bits widened by a shift are the values the oracle must use
    a_ref = workloads.bf16_bits_to_f32(ab).astype(np.float64)
    w_ref = workloads.bf16_bits_to_f32(wb).astype(np.float64)
    np.testing.assert_allclose(oracle.linear_from_storage(ab, "bf16", wb, "bf16"), a_ref @ w_ref.T,
                               rtol=1e-13, atol=1e-13)
    q, s = workloads.quantise_rows_e4m3fn(w)
    deq = oracle.e4m3fn_to_f64(q) * s.astype(np.float64)[:, None]
    np.testing.assert_allclose(oracle.linear_from_storage(ab, "bf16", q, "e4m3fn", s), a_ref @ deq.T,
                               rtol=1e-13, atol=1e-13)
    with pytest.raises(ValueError):
        oracle.linear_from_storage(ab, "bf16", q, "e4m3fn")
