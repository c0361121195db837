"""Seeded random shapes through every route against the oracle.

The fixed-shape suites pin each blocking class, tail and edge case; this one
draws shapes the suites do not list (ragged M, K from one block to 320 blocks,
B from 1 to 64), for Q4 and Q8_0 weights, single products on the automatic
and both forced routes, grouped launches mixing formats and widths, and
expert-routed products.  Block sums are compared bit for bit, outputs within
the normwise gates of tests/gpu_util.py.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import assert_close, to_dev

pytestmark = pytest.mark.gpu

q = pytest.importorskip("block_quantized_matmul_q8_amd")

NTHREADS = 16


@pytest.fixture(autouse=True)
def _auto_path():
    q.q4q8_set_path(q.PATH_AUTO)
    yield
    q.q4q8_set_path(q.PATH_AUTO)


def _shape(rng, b_max=64):
    M = int(rng.integers(1, 1400))
    K = 32 * int(rng.integers(1, 321))
    B = int(rng.integers(1, 9)) if rng.random() < 0.6 else int(rng.integers(9, b_max + 1))
    return M, K, B


def _product(seed, i, M, K, B, q8_0):
    w = workloads.weight(seed, 2, i, M, K)
    x = workloads.activation(seed, 2, i, B, K)
    g = workloads.norm_weight(seed, 2, i, K)
    xq, xd, _ = oracle.q8_quantize_rmsnorm(x, g, workloads.RMS_EPS)
    if q8_0:
        qw, d = oracle.q8w_quantize(w)
        I_o = oracle.block_dots_q8w(qw, xq)
        y_o, _ = oracle.mul_mat_q8w(qw, d, xq, xd, nthreads=NTHREADS)
    else:
        qw, d = oracle.q4_quantize(w)
        I_o = oracle.block_dots(qw, K, xq)
        y_o, _ = oracle.mul_mat(qw, d, xq, xd, nthreads=NTHREADS)
    return qw, d, xq, xd, I_o, y_o


@pytest.mark.parametrize("q8_0", [False, True], ids=["q4", "q8_0"])
def test_random_single_products(q8_0):
    rng = np.random.default_rng(7100 + q8_0)
    for i in range(10):
        M, K, B = _shape(rng)
        qw, d, xq, xd, I_o, y_o = _product(7100, i, M, K, B, q8_0)
        args = (to_dev(qw), to_dev(d.view(np.int16)), to_dev(xq), to_dev(xd))
        blocksums = q.mul_mat_q8_0_q8_blocksums if q8_0 else q.mul_mat_q4q8_blocksums
        plain = q.mul_mat_q8_0_q8 if q8_0 else q.mul_mat_q4q8
        paths = [q.PATH_AUTO, q.PATH_GEMM] + ([q.PATH_GEMV] if B <= 8 else [])
        for path in paths:
            q.q4q8_set_path(path)
            tag = f"case {i} M={M} K={K} B={B} path={path}"
            y, I = blocksums(*args)
            torch.cuda.synchronize()
            assert np.array_equal(I.cpu().numpy(), I_o), tag
            assert_close(y.cpu().numpy(), y_o, tag)
            y2 = plain(*args)
            torch.cuda.synchronize()
            assert_close(y2.cpu().numpy(), y_o, tag + " (production instance)")
        q.q4q8_set_path(q.PATH_AUTO)


@pytest.mark.parametrize("case", range(4))
def test_random_groups(case):
    """A group of random products at one random width, each product's format
    drawn at random: outputs match the oracle and equal the single calls bit
    for bit, each single call on the group's route (a group of 5..8 columns
    that mixes formats or shapes runs the lane-per-block kernel, where a
    single call could take the multi-column one)."""
    rng = np.random.default_rng(7200 + case)
    B = int(rng.integers(1, 9)) if case < 3 else int(rng.integers(9, 48))
    dev = torch.device("cuda:0")
    problems, refs, fmt = [], [], []
    for i in range(int(rng.integers(2, 8))):
        M, K, _ = _shape(rng)
        q8_0 = bool(rng.random() < 0.4)
        qw, d, xq, xd, _, y_o = _product(7200 + case, i, M, K, B, q8_0)
        p = {"qw" if q8_0 else "qs": to_dev(qw), "d": to_dev(d.view(np.int16)), "xq": to_dev(xq),
             "xd": to_dev(xd), "y": torch.full((B, M), float("nan"), dtype=torch.float32, device=dev)}
        problems.append(p)
        refs.append(y_o)
        fmt.append(q8_0)
    grp = q.Group(problems, B=B)
    grp()
    torch.cuda.synchronize()
    for p, y_o, q8_0 in zip(problems, refs, fmt):
        w = p["qw"] if q8_0 else p["qs"]
        tag = f"case {case} B={B} M={w.shape[0]} q8_0={q8_0}"
        assert_close(p["y"].cpu().numpy(), y_o, tag)
        lanes = B <= 8 and not grp.plan.mfma_columns
        q.q4q8_set_path(q.PATH_GEMV_LANES if lanes else q.PATH_AUTO)
        single = (q.mul_mat_q8_0_q8 if q8_0 else q.mul_mat_q4q8)(w, p["d"], p["xq"], p["xd"])
        torch.cuda.synchronize()
        q.q4q8_set_path(q.PATH_AUTO)
        assert np.array_equal(single.cpu().numpy().view(np.uint32), p["y"].cpu().numpy().view(np.uint32)), tag


@pytest.mark.parametrize("case", range(5))
def test_random_expert_routing(case):
    """Random expert count, shape, token count, top-k and activation-slot form."""
    rng = np.random.default_rng(7300 + case)
    E = int(rng.integers(1, 41))
    M = int(rng.integers(1, 700))
    K = 32 * int(rng.integers(1, 129))
    T = int(rng.integers(1, 25))
    top_k = int(rng.integers(1, min(E, 8) + 1))
    S = top_k if rng.random() < 0.5 else 1
    w = np.stack([workloads.weight(7300 + case, 3, e, M, K) for e in range(E)])
    qs, d = oracle.q4_quantize(w.reshape(E * M, K))
    qs, d = qs.reshape(E, M, K // 2), d.reshape(E, M, K // 32)
    x = workloads.activation(7300 + case, 3, S, T * S, K)
    g = workloads.norm_weight(7300 + case, 3, S, K)
    xq, xd, _ = oracle.q8_quantize_rmsnorm(x, g, workloads.RMS_EPS)
    xq, xd = xq.reshape(T, S, K), xd.reshape(T, S, K // 32)
    ids = workloads.expert_ids(7300 + case, T, E, top_k)
    y = q.mul_mat_id_q4q8(to_dev(qs), to_dev(d.view(np.int16)), to_dev(xq), to_dev(xd), to_dev(ids))
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    y_o = oracle.mul_mat_id(qs, d, xq, xd, ids, nthreads=NTHREADS)
    for t in range(T):
        for s in range(top_k):
            assert_close(y[t, s], y_o[t, s], f"case {case} E={E} M={M} K={K} T={T} top_k={top_k} S={S} t={t} s={s}")
