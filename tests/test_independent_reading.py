"""The C oracle against a second, independent reading of the same rules
(tests/independent_reading.py, numpy): every code, scale, block sum and fp32
output must agree bit for bit.  The two share only the seeded inputs."""
import json
import os

import numpy as np
import pytest

import oracle
import workloads as wl
from tests import independent_reading as ind

HERE = os.path.dirname(__file__)


def _bits(a):
    a = np.ascontiguousarray(a)
    return a.view(np.uint32) if a.dtype == np.float32 else a


def _same(a, b):
    a, b = np.asarray(a), np.asarray(b)
    assert a.shape == b.shape and a.dtype == b.dtype, (a.shape, a.dtype, b.shape, b.dtype)
    if a.dtype == np.float32:
        nan = np.isnan(a)
        assert np.array_equal(nan, np.isnan(b))
        assert np.array_equal(_bits(np.where(nan, 0, a)), _bits(np.where(nan, 0, b)))
    else:
        assert np.array_equal(a, b)


def _special_weight_rows(K):
    """Rows whose blocks hit the rule's corner cases: an all-zero block, a
    +-amax tie (sign decided by the lowest index), a block whose scale is
    subnormal in fp16, one whose fp32 scale underflows the fp16 range, huge
    values, a block of equal magnitudes, and one with a single non-zero."""
    rows = np.zeros((6, K), dtype=np.float32)
    r = np.random.default_rng(7)
    rows[:] = r.standard_normal((6, K), dtype=np.float32) * np.float32(0.02)
    rows[0, :32] = 0.0
    rows[1, 32:64] = np.linspace(-0.5, 0.5, 32, dtype=np.float32)
    rows[1, 40], rows[1, 50] = np.float32(-0.7), np.float32(0.7)
    rows[2, :32] *= np.float32(1e-4)                   # fp16 subnormal scale
    rows[3, :32] *= np.float32(1e-8)                   # scale below fp16's range
    rows[4, :32] *= np.float32(1e6)                    # scale near fp16's top
    rows[5, :32] = np.float32(0.25)
    rows[5, 32:64] = 0.0
    rows[5, 45] = np.float32(-3.0)
    return rows


def _e_blocks():
    with open(os.path.join(HERE, "golden", "hand_examples.json")) as f:
        g = json.load(f)
    return g


@pytest.mark.parametrize("M,K,seed", [(64, 512, 0), (33, 96, 1), (7, 4096, 2)])
def test_q4_quantize_agrees(M, K, seed):
    w = wl.weight(seed, 0, 0, M, K)
    w = np.concatenate([w, _special_weight_rows(K)])
    qs, d = oracle.q4_quantize(w)
    qs2, d2 = ind.q4_quantize(w)
    _same(qs, qs2)
    _same(d, d2)
    _same(oracle.q4_unpack_codes(qs, K), ind.q4_codes(qs2))


def test_hand_blocks_agree():
    """The hand-derived blocks: each sits where a plausible other reading of
    a rule (divide instead of reciprocal-multiply, codes from the fp16 scale,
    the last index of a +-amax tie, halves to even) gives other codes."""
    g = _e_blocks()
    e1 = [-8 + (j % 16) for j in range(32)]          # E1, stated as a formula
    w = [e1] + [g[k]["w"] for k in ("E2a", "E2b")] + [g[k]["q4_w"] for k in ("E7", "E8")]
    w = np.asarray(w, dtype=np.float32)
    for a, b in zip(oracle.q4_quantize(w), ind.q4_quantize(w)):
        _same(a, b)
    v = np.asarray([g["E4"]["v"], g["E7"]["q8_v"]], dtype=np.float32)
    for a, b in zip(oracle.q8_quantize(v), ind.q8_quantize(v)):
        _same(a, b)
    w8 = np.asarray([g["E8"]["q8_0_w"]], dtype=np.float32)
    for a, b in zip(oracle.q8w_quantize(w8), ind.q8w_quantize(w8)):
        _same(a, b)


@pytest.mark.parametrize("B,K,seed", [(5, 512, 0), (3, 96, 1), (2, 14336, 2), (1, 2048, 3)])
def test_rmsnorm_q8_agrees(B, K, seed):
    x = wl.activation(seed, 0, 0, B, K)
    g = wl.norm_weight(seed, 0, 0, K)
    x[0, :32] = 0.0                                   # a zero block after the norm
    got = oracle.q8_quantize_rmsnorm(x, g, wl.RMS_EPS)
    ref = ind.q8_quantize_rmsnorm(x, g, wl.RMS_EPS)
    for a, b in zip(got, ref):
        _same(a, b)
    v = x * np.float32(3.0)
    for a, b in zip(oracle.q8_quantize_rmsnorm(v, None, 0.0, no_norm=True), ind.q8_quantize(v)):
        _same(a, b)


def test_rmsnorm_q8_agrees_on_degenerate_rows():
    K = 256
    x = np.zeros((4, K), dtype=np.float32)
    x[1] = np.float32(2.5)                            # constant row
    x[2, 7] = np.float32(4096.0)                      # one spike
    x[3] = np.float32(1e-20)                          # eps dominates
    x = np.concatenate([x, np.zeros((1, K), dtype=np.float32)])
    x[4, :4] = np.float32([4096.0, 1.0, 1.0, 1.0])    # in-block order of the squares shows
    g = np.ones(K, dtype=np.float32)
    for a, b in zip(oracle.q8_quantize_rmsnorm(x, g, 1e-5), ind.q8_quantize_rmsnorm(x, g, 1e-5)):
        _same(a, b)


@pytest.mark.parametrize("per_row", [False, True])
def test_rmsnorm_add_q8_agrees(per_row):
    B, K = 4, 1024
    x = wl.activation(5, 0, 0, B, K)
    g = wl.norm_weight(5, 0, 0, K)
    a = wl.activation(5, 0, 1, B if per_row else 1, K)
    a = a if per_row else a[0]
    for u, v in zip(oracle.q8_quantize_rmsnorm_add(x, g, a, 1e-5), ind.q8_quantize_rmsnorm_add(x, g, a, 1e-5)):
        _same(u, v)


@pytest.mark.parametrize("M,K,B,seed", [(48, 512, 3, 0), (17, 2048, 1, 1), (5, 96, 8, 2)])
def test_block_dots_and_product_agree(M, K, B, seed):
    w = wl.weight(seed, 1, 0, M, K)
    qs, d = oracle.q4_quantize(w)
    xq, xd, _ = oracle.q8_quantize_rmsnorm(wl.activation(seed, 1, 0, B, K), wl.norm_weight(seed, 1, 0, K), 1e-5)
    _same(oracle.block_dots(qs, K, xq), ind.block_dots(qs, xq))
    y, _ = oracle.mul_mat(qs, d, xq, xd)
    _same(y, ind.mul_mat(qs, d, xq, xd))


def test_q8_0_weights_agree():
    M, K, B = 40, 1024, 3
    w = np.concatenate([wl.weight(4, 0, 0, M, K), _special_weight_rows(K)])
    qw, d = oracle.q8w_quantize(w)
    qw2, d2 = ind.q8w_quantize(w)
    _same(qw, qw2)
    _same(d, d2)
    xq, xd, _ = oracle.q8_quantize_rmsnorm(wl.activation(4, 0, 0, B, K), wl.norm_weight(4, 0, 0, K), 1e-5)
    y, _ = oracle.mul_mat_q8w(qw, d, xq, xd)
    _same(y, ind.mul_mat_q8w(qw, d, xq, xd))


@pytest.mark.parametrize("n_x_slots", [1, 4])
def test_mul_mat_id_agrees(n_x_slots):
    E, M, K, T, top_k = 6, 24, 256, 5, 4
    qs, d = zip(*(oracle.q4_quantize(wl.weight(6, e, 0, M, K)) for e in range(E)))
    qs, d = np.stack(qs), np.stack(d)
    xq, xd, _ = oracle.q8_quantize_rmsnorm(wl.activation(6, 0, 0, T * n_x_slots, K), wl.norm_weight(6, 0, 0, K),
                                           1e-5)
    xq = xq.reshape(T, n_x_slots, K)
    xd = xd.reshape(T, n_x_slots, K // 32)
    ids = wl.expert_ids(6, T, E, top_k)
    ids[1, 2] = E          # out of range: NaN row
    ids[3, 0] = -1
    _same(oracle.mul_mat_id(qs, d, xq, xd, ids), ind.mul_mat_id(qs, d, xq, xd, ids))


@pytest.mark.parametrize("weighted", [False, True])
def test_expert_sum_agrees(weighted):
    T, top_k, M = 4, 8, 96
    y = wl.activation(8, 0, 0, T * top_k, M).reshape(T, top_k, M)
    y[2, 5, 7] = np.nan
    w = wl.expert_weights(8, T, top_k) if weighted else None
    _same(oracle.moe_expert_sum(y, w), ind.moe_expert_sum(y, w))


def test_swiglu_q8_agrees():
    B, F = 3, 1408
    gate = wl.activation(9, 0, 0, B, F) * np.float32(6.0)
    up = wl.activation(9, 0, 1, B, F)
    gate[0, :8] = np.array([0.0, -0.0, 100.0, -100.0, 88.5, -17.5, 40.0, -40.0], dtype=np.float32)
    for a, b in zip(oracle.q8_quantize_swiglu(gate, up), ind.q8_quantize_swiglu(gate, up)):
        _same(a, b)
    t = np.concatenate([np.linspace(-20, 90, 4001, dtype=np.float32),
                        np.array([np.nan, np.inf, -np.inf, 88.0, -17.0], dtype=np.float32)])
    _same(oracle.exp_q(t), ind.exp_q(t))
