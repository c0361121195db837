"""Pins of the oracle's block dots, scale-and-accumulate and expert routing.

Pinned against: the hand example E5 (I = -2032, y bits), brute-force integer
products computed with numpy int64 matmul on decoded codes, the fp64
dequantised matmul (numpy float64 matmul of (q-8)*d_w and q8*d_x, whose
products are exact), the fp32 forward error bound of a length-nb sum, the
K-block permutation invariance of the exact integer sums, the offset
identity sum (q-8) x = sum q x - 8 sum x, and, for the expert-routed product,
a loop of plain products, the E = 1 / top_k = 1 reduction and NaN rows for
bad ids.  The expert-plane sum is pinned by an example whose value depends on
the summation order, exact integer sums, the correctly rounded single
product, and the fp32 error bound of the chain against an fp64 sum.
"""
import numpy as np
import pytest

import oracle
import workloads

U = 2.0 ** -24


def _decode_codes(qs, K):
    """Decode the qs plane independently of the oracle: byte j of a block
    holds code j (low nibble) and code j + 16 (high nibble)."""
    M = qs.shape[0]
    b = qs.reshape(M, K // 32, 16).astype(np.int64)
    return np.concatenate([b & 15, b >> 4], axis=2).reshape(M, K)


def _make(seed, M, K, B, sigma=0.02):
    w = workloads.weight(seed, 0, 0, M, K, sigma)
    x = workloads.activation(seed, 0, 0, B, K)
    g = workloads.norm_weight(seed, 0, 0, K)
    qs, d = oracle.q4_quantize(w)
    xq, xd, xs = oracle.q8_quantize_rmsnorm(x, g, 1e-5)
    return qs, d, xq, xd, xs


def test_hand_example_e5(hand_examples):
    e5 = hand_examples["E5"]
    w = np.array([[-8 + (j % 16) for j in range(32)]], dtype=np.float32)
    qs, d = oracle.q4_quantize(w)
    xq, xd, _ = oracle.q8_quantize_rmsnorm(np.ones((1, 32), np.float32), np.ones(32, np.float32), 1e-5)
    assert int(oracle.block_dots(qs, 32, xq)[0, 0, 0]) == e5["I"]
    y, y64 = oracle.mul_mat(qs, d, xq, xd)
    assert int(y.view(np.uint32)[0, 0]) == int(e5["y_bits"], 16)


@pytest.mark.parametrize("M,K,B", [(1, 32, 1), (7, 64, 3), (33, 1408, 2), (64, 256, 4), (5, 4096, 1)])
def test_block_dots_brute_force(M, K, B):
    g = np.random.default_rng(M * 1000 + K + B)
    qs = g.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
    xq = g.integers(-127, 128, size=(B, K), dtype=np.int8)
    I = oracle.block_dots(qs, K, xq)
    q = _decode_codes(qs, K) - 8
    nb = K // 32
    ref = np.einsum("mbj,nbj->nmb", q.reshape(M, nb, 32), xq.astype(np.int64).reshape(B, nb, 32))
    assert np.array_equal(I.astype(np.int64), ref)
    # extreme codes: |I| reaches 32 * 8 * 127 = 32512
    qs_min = np.zeros((1, 16), np.uint8)
    xq_max = np.full((1, 32), 127, np.int8)
    assert int(oracle.block_dots(qs_min, 32, xq_max)[0, 0, 0]) == -32512


@pytest.mark.parametrize("M,K,B", [(16, 512, 1), (40, 1408, 3), (24, 2048, 2)])
def test_offset_identity(M, K, B):
    qs, d, xq, xd, xs = _make(1, M, K, B)
    I = oracle.block_dots(qs, K, xq).astype(np.int64)
    q = _decode_codes(qs, K)
    nb = K // 32
    raw = np.einsum("mbj,nbj->nmb", q.reshape(M, nb, 32), xq.astype(np.int64).reshape(B, nb, 32))
    assert np.array_equal(I, raw - 8 * xs.astype(np.int64)[:, None, :])


@pytest.mark.parametrize("M,K,B", [(1, 32, 1), (17, 512, 1), (64, 1408, 4), (32, 4096, 8), (3, 8192, 2)])
def test_mul_mat_vs_fp64_dequant(M, K, B):
    qs, d, xq, xd, _ = _make(2, M, K, B)
    y, y64 = oracle.mul_mat(qs, d, xq, xd)
    Wd = oracle.dequantize_q4(qs, d, K)
    Xd = oracle.dequantize_q8(xq, xd)
    ref = Xd @ Wd.T                                     # [B][M], fp64
    terms_abs = np.abs(Xd) @ np.abs(Wd).T
    assert np.all(np.abs(y64 - ref) <= 4 * K * 2.0 ** -53 * terms_abs + 1e-300)
    nb = K // 32
    assert np.all(np.abs(y.astype(np.float64) - y64) <= (nb + 3) * U * terms_abs)


def test_mul_mat_tiny_workload_tolerance():
    """The tiny single product (W 256x512, x[512], seed 0): fp32 result vs the
    fp64 sum within the normwise gates used for the GPU (max-rel 1e-4, NMSE
    1e-7); the oracle is far inside them."""
    t = workloads.TINY
    w = workloads.weight(0, 0, 0, t.M, t.K)
    x = workloads.activation(0, 0, 0, 1, t.K)
    g = workloads.norm_weight(0, 0, 0, t.K)
    qs, d = oracle.q4_quantize(w)
    xq, xd, _ = oracle.q8_quantize_rmsnorm(x, g, workloads.RMS_EPS)
    y, y64 = oracle.mul_mat(qs, d, xq, xd)
    err = y.astype(np.float64) - y64
    assert np.abs(err).max() / np.abs(y64).max() < 1e-6
    assert (err ** 2).sum() / (y64 ** 2).sum() < 1e-12


@pytest.mark.parametrize("K", [256, 1408])
def test_k_block_permutation_invariance(K):
    M, B = 12, 3
    qs, d, xq, xd, _ = _make(3, M, K, B)
    nb = K // 32
    perm = np.random.default_rng(K).permutation(nb)
    qs_p = qs.reshape(M, nb, 16)[:, perm].reshape(M, K // 2)
    d_p = d[:, perm]
    xq_p = xq.reshape(B, nb, 32)[:, perm].reshape(B, K)
    xd_p = xd[:, perm]
    I = oracle.block_dots(qs, K, xq)
    I_p = oracle.block_dots(qs_p, K, xq_p)
    assert np.array_equal(I[:, :, perm], I_p)
    _, y64 = oracle.mul_mat(qs, d, xq, xd)
    _, y64p = oracle.mul_mat(qs_p, d_p, xq_p, xd_p)
    assert np.all(np.abs(y64 - y64p) <= 2.0 ** -40 * np.abs(y64).max())


@pytest.mark.parametrize("nthreads", [2, 3, 8])
def test_multithreaded_is_bit_identical(nthreads):
    qs, d, xq, xd, _ = _make(4, 101, 1024, 3)
    y1, a = oracle.mul_mat(qs, d, xq, xd, nthreads=1)
    yn, b = oracle.mul_mat(qs, d, xq, xd, nthreads=nthreads)
    assert np.array_equal(y1.view(np.uint32), yn.view(np.uint32))
    assert np.array_equal(a.view(np.uint64), b.view(np.uint64))


# ----------------------------------------------------------------------------- MUL_MAT_ID

def _moe_inputs(seed, E, M, K, T, top_k, n_x_slots):
    w = np.stack([workloads.weight(seed, 0, e, M, K) for e in range(E)])
    qs, d = oracle.q4_quantize(w.reshape(E * M, K))
    qs = qs.reshape(E, M, K // 2)
    d = d.reshape(E, M, K // 32)
    x = workloads.activation(seed, 0, 0, T * n_x_slots, K)
    g = workloads.norm_weight(seed, 0, 0, K)
    xq, xd, _ = oracle.q8_quantize_rmsnorm(x, g, 1e-5)
    xq = xq.reshape(T, n_x_slots, K)
    xd = xd.reshape(T, n_x_slots, K // 32)
    ids = workloads.expert_ids(seed, T, E, top_k)
    return qs, d, xq, xd, ids


@pytest.mark.parametrize("n_slots_mode", ["broadcast", "per_slot"])
def test_mul_mat_id_equals_loop(n_slots_mode):
    E, M, K, T, top_k = 6, 40, 1408, 5, 3
    n_x_slots = 1 if n_slots_mode == "broadcast" else top_k
    qs, d, xq, xd, ids = _moe_inputs(5, E, M, K, T, top_k, n_x_slots)
    y = oracle.mul_mat_id(qs, d, xq, xd, ids, nthreads=2)
    for t in range(T):
        for s in range(top_k):
            e = ids[t, s]
            r = 0 if n_x_slots == 1 else s
            ref, _ = oracle.mul_mat(qs[e], d[e], xq[t, r][None], xd[t, r][None])
            assert np.array_equal(y[t, s].view(np.uint32), ref[0].view(np.uint32))


def test_mul_mat_id_single_expert_reduces_to_mul_mat():
    E, M, K, T, top_k = 1, 24, 512, 4, 1
    qs, d, xq, xd, ids = _moe_inputs(6, E, M, K, T, top_k, 1)
    y = oracle.mul_mat_id(qs, d, xq, xd, ids)
    ref, _ = oracle.mul_mat(qs[0], d[0], xq[:, 0], xd[:, 0])
    assert np.array_equal(y[:, 0], ref)


def test_mul_mat_id_bad_ids_give_nan_rows():
    E, M, K, T, top_k = 4, 8, 64, 3, 2
    qs, d, xq, xd, ids = _moe_inputs(7, E, M, K, T, top_k, 1)
    ids = ids.copy()
    ids[0, 1] = E
    ids[2, 0] = -1
    y = oracle.mul_mat_id(qs, d, xq, xd, ids)
    assert np.all(np.isnan(y[0, 1])) and np.all(np.isnan(y[2, 0]))
    assert np.all(np.isfinite(y[0, 0])) and np.all(np.isfinite(y[1])) and np.all(np.isfinite(y[2, 1]))


def test_expert_ids_distinct_and_in_range():
    ids = workloads.expert_ids(0, 16, 64, 8)
    assert ids.shape == (16, 8) and ids.dtype == np.int32
    assert ids.min() >= 0 and ids.max() < 64
    assert all(len(set(r.tolist())) == 8 for r in ids)


def test_expert_sum_follows_the_add_chain_order():
    # 1 + 2^-24 + 2^-24: the in-order chain rounds twice back to 1, while adding
    # the two small planes first gives 1 + 2^-23 (exact)
    y = np.array([[[1.0], [U], [U]]], dtype=np.float32)
    assert oracle.moe_expert_sum(y)[0, 0] == np.float32(1.0)
    assert oracle.moe_expert_sum(np.ascontiguousarray(y[:, ::-1]))[0, 0] == np.float32(1.0 + 2 * U)


def test_expert_sum_exact_on_integers():
    g = np.random.default_rng(11)
    T, top_k, M = 5, 8, 33
    yi = g.integers(-1000, 1001, size=(T, top_k, M))
    wi = g.integers(-8, 9, size=(T, top_k))
    out = oracle.moe_expert_sum(yi.astype(np.float32), wi.astype(np.float32))
    assert np.array_equal(out.astype(np.int64), np.einsum("tsm,ts->tm", yi, wi))
    out1 = oracle.moe_expert_sum(yi.astype(np.float32))
    assert np.array_equal(out1.astype(np.int64), yi.sum(axis=1))


def test_expert_sum_single_slot_is_the_rounded_product():
    g = np.random.default_rng(12)
    y = g.standard_normal((4, 1, 50)).astype(np.float32)
    w = g.standard_normal((4, 1)).astype(np.float32)
    exact = y.astype(np.float64) * w.astype(np.float64)[:, :, None]   # exact in fp64
    assert np.array_equal(oracle.moe_expert_sum(y, w), exact[:, 0].astype(np.float32))


def test_expert_sum_error_bound_and_nan_planes():
    T, top_k, M = 16, 8, 300
    g = np.random.default_rng(13)
    y = g.standard_normal((T, top_k, M)).astype(np.float32)
    w = workloads.expert_weights(3, T, top_k)
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-6) and (w > 0).all()
    out = oracle.moe_expert_sum(y, w).astype(np.float64)
    terms = y.astype(np.float64) * w.astype(np.float64)[:, :, None]
    ref = terms.sum(axis=1)
    n = 2 * top_k
    bound = n * U / (1 - n * U) * np.abs(terms).sum(axis=1)
    assert np.all(np.abs(out - ref) <= bound)
    y[3, 5, :] = np.nan
    out = oracle.moe_expert_sum(y, w)
    assert np.all(np.isnan(out[3])) and np.all(np.isfinite(np.delete(out, 3, axis=0)))
