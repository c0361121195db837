"""Pins of the oracle's Q8_0 weight type (int8 codes, fp16 block scale).

Pinned against: hand examples (a block whose scale is exactly 1, so the codes
are the values; halves rounded away from zero; the all-zero block), the
closed-form round-trip bound, brute-force int64 block products on the codes,
the fp64 dequantised product (exact products in fp64), the fp32 forward error
bound of the block sum, and invariance of the exact block sums under a common
permutation of the K blocks.
"""
import numpy as np
import pytest

import oracle
import workloads

U = 2.0 ** -24


def test_q8w_unit_scale_block_codes_are_the_values():
    w = np.zeros((1, 32), np.float32)
    w[0, :31] = np.arange(31) - 15
    w[0, 31] = 127.0                          # amax = 127 -> d = 1 exactly
    qw, d = oracle.q8w_quantize(w)
    assert d[0, 0] == 0x3C00
    assert qw[0].tolist() == (np.arange(31) - 15).tolist() + [127]


def test_q8w_halves_round_away_from_zero_and_zero_block():
    w = np.zeros((2, 32), np.float32)
    w[0, :6] = [0.5, 1.5, -0.5, -2.5, 2.5, -127.0]   # d = 1 (amax 127 carried by a negative value)
    qw, d = oracle.q8w_quantize(w)
    assert d[0, 0] == 0x3C00 and qw[0, :6].tolist() == [1, 2, -1, -3, 3, -127]
    assert d[1, 0] == 0 and not qw[1].any()


@pytest.mark.parametrize("seed", [0, 1])
def test_q8w_round_trip_bound(seed):
    w = workloads.weight(seed, 0, 3, 64, 2048)
    qw, d = oracle.q8w_quantize(w)
    wb = w.reshape(64, -1, 32).astype(np.float64)
    d32 = np.abs(wb).max(axis=2) / 127.0                       # the fp32 scale up to one rounding
    err = np.abs(wb - oracle.dequantize_q8w(qw, d).reshape(64, -1, 32)).max(axis=2)
    # rounding (1/2 code) + fp16 scale rounding over at most 127 codes + the fp32 steps
    assert np.all(err <= d32 * (0.5 + 127 * 2.0 ** -11 + 2.0 ** -16) + 1e-30)
    assert np.abs(qw.astype(np.int64)).max() <= 127


def test_q8w_block_dots_brute_force_and_permutation():
    M, K, B = 9, 256, 3
    qw, _ = oracle.q8w_quantize(workloads.weight(2, 0, 0, M, K))
    x = workloads.activation(2, 0, 0, B, K)
    xq, xd, _ = oracle.q8_quantize_rmsnorm(x, workloads.norm_weight(2, 0, 0, K), workloads.RMS_EPS)
    I = oracle.block_dots_q8w(qw, xq)
    ref = np.einsum("mbj,nbj->nmb", qw.reshape(M, -1, 32).astype(np.int64), xq.reshape(B, -1, 32).astype(np.int64))
    assert np.array_equal(I, ref)
    perm = np.random.default_rng(3).permutation(K // 32)
    Ip = oracle.block_dots_q8w(np.ascontiguousarray(qw.reshape(M, -1, 32)[:, perm].reshape(M, K)),
                               np.ascontiguousarray(xq.reshape(B, -1, 32)[:, perm].reshape(B, K)))
    assert np.array_equal(Ip, I[:, :, perm])


@pytest.mark.parametrize("M,K,B", [(33, 1408, 2), (16, 4096, 5)])
def test_q8w_product_fp64_and_bound(M, K, B):
    qw, d = oracle.q8w_quantize(workloads.weight(4, 0, 1, M, K))
    x = workloads.activation(4, 0, 0, B, K)
    xq, xd, _ = oracle.q8_quantize_rmsnorm(x, workloads.norm_weight(4, 0, 0, K), workloads.RMS_EPS)
    y, y64 = oracle.mul_mat_q8w(qw, d, xq, xd, nthreads=2)
    ref = oracle.dequantize_q8(xq, xd) @ oracle.dequantize_q8w(qw, d).T
    assert np.allclose(y64, ref, rtol=1e-12, atol=1e-12)
    I = oracle.block_dots_q8w(qw, xq).astype(np.float64)
    terms = np.abs(I * oracle.f16_bits_to_f32(d).astype(np.float64)[None] * xd.astype(np.float64)[:, None])
    nb = K // 32
    g = (nb + 2) * U / (1 - (nb + 2) * U)
    assert np.all(np.abs(y.astype(np.float64) - y64) <= g * terms.sum(axis=2) + 1e-30)
