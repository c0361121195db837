"""GPU parity of the multi-column MFMA streaming kernel (B = 5..8 columns,
rows of at least four whole 128-byte segments: K a multiple of 256 and at
least 1024 for Q4, of 128 and at least 512 for Q8_0)
against the oracle: block sums bit for bit (its debug instance), outputs
within max-rel 1e-4 / NMSE 1e-7, every output written.

Shapes stress the kernel's corners: four chunks per row (one per wave of
the workgroup), chunk counts that do not divide by four, row counts around the
64-row window and 16-row group, one column group only partly used (B odd),
more windows than resident workgroups (each then streams several windows
and its load fronts cross from one window, or product, to the next), Q8_0
weights, and grouped launches that take the kernel (plan.mfma_columns == 1)
or fall back to the lane-per-block one (K not of whole segments, mixed weight
formats, four or fewer columns)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import assert_close, to_dev

pytestmark = pytest.mark.gpu

q = pytest.importorskip("block_quantized_matmul_q8_amd")


def _inputs(seed, M, K, B, q8_0=False):
    w = workloads.weight(seed, 1, M % 5, M, K)
    x = workloads.activation(seed, 1, 0, B, K)
    g = workloads.norm_weight(seed, 1, 0, K)
    xq, xd, _ = oracle.q8_quantize_rmsnorm(x, g, workloads.RMS_EPS)
    if q8_0:
        qw, d = oracle.q8w_quantize(w)
        return qw, d, xq, xd
    qs, d = oracle.q4_quantize(w)
    return qs, d, xq, xd


SHAPES = [(1, 1024, 5), (15, 1280, 8), (16, 1536, 5), (63, 2048, 6), (64, 1792, 7), (65, 4096, 6),
          (200, 14336, 8), (129, 8192, 5), (17, 1024, 8), (31, 2304, 7), (33, 3328, 5)]


@pytest.mark.parametrize("q8_0", [False, True])
@pytest.mark.parametrize("M,K,B", SHAPES)
def test_multicolumn_blocksums_and_outputs(M, K, B, q8_0):
    print(f"[multicol] M={M} K={K} B={B} q8_0={q8_0}", flush=True)
    w, d, xq, xd = _inputs(31, M, K, B, q8_0)
    args = (to_dev(w), to_dev(d.view(np.int16)), to_dev(xq), to_dev(xd))
    y = torch.full((B, M), float("nan"), device="cuda:0")
    I = torch.full((B, M, K // 32), -(2 ** 31), dtype=torch.int32, device="cuda:0")
    q.q4q8_dispatch_counts(reset=True)
    if q8_0:
        q.mul_mat_q8_0_q8_blocksums(*args, y=y, I=I)
        I_o = oracle.block_dots_q8w(w, xq)
        y_o, _ = oracle.mul_mat_q8w(w, d, xq, xd, nthreads=16)
    else:
        q.mul_mat_q4q8_blocksums(*args, y=y, I=I)
        I_o = oracle.block_dots(w, K, xq)
        y_o, _ = oracle.mul_mat(w, d, xq, xd, nthreads=16)
    torch.cuda.synchronize()
    assert q.q4q8_dispatch_counts(reset=True)["gemv"] == 1
    assert "gemv_mfma_kernel" in q.q4q8_last_kernel()
    assert np.array_equal(I.cpu().numpy(), I_o)
    yh = y.cpu().numpy()
    assert np.isfinite(yh).all()
    assert_close(yh, y_o, f"M={M} K={K} B={B}")
    # the production instance (no block sums) agrees with the debug one
    y2 = torch.full((B, M), float("nan"), device="cuda:0")
    if q8_0:
        q.mul_mat_q8_0_q8(*args, y=y2)
    else:
        q.mul_mat_q4q8(*args, y=y2)
    torch.cuda.synchronize()
    assert np.array_equal(y2.cpu().numpy(), yh)


@pytest.mark.parametrize("M,K,B", [(33, 640, 5), (40, 512, 6)])
def test_multicolumn_q8_0_half_segments(M, K, B):
    """Q8_0 rows of 640 / 512 elements: five / four whole 128-byte segments
    (Q4 rows of these K are too short for the kernel)."""
    test_multicolumn_blocksums_and_outputs(M, K, B, True)


def test_multicolumn_many_windows_per_workgroup():
    """More 64-row windows than the launch has workgroups: every workgroup
    streams several windows back to back."""
    M, K, B = 140000, 1024, 5
    print(f"[multicol many] M={M} K={K} B={B}", flush=True)
    w, d, xq, xd = _inputs(33, M, K, B)
    y = torch.full((B, M), float("nan"), device="cuda:0")
    q.mul_mat_q4q8(to_dev(w), to_dev(d.view(np.int16)), to_dev(xq), to_dev(xd), y=y)
    torch.cuda.synchronize()
    assert "gemv_mfma_kernel" in q.q4q8_last_kernel()
    y_o, _ = oracle.mul_mat(w, d, xq, xd, nthreads=16)
    yh = y.cpu().numpy()
    assert np.isfinite(yh).all()
    assert_close(yh, y_o, "many windows")


@pytest.mark.parametrize("K", [96, 128, 192, 512, 768, 1088])
def test_partial_segments_take_the_lane_kernel(K):
    """Q4 rows that are not four or more whole 128-byte segments: the
    lane-per-block kernel serves them."""
    w, d, xq, xd = _inputs(32, 40, K, 5)
    y = q.mul_mat_q4q8(to_dev(w), to_dev(d.view(np.int16)), to_dev(xq), to_dev(xd))
    torch.cuda.synchronize()
    assert "gemv_mfma_kernel" not in q.q4q8_last_kernel()
    y_o, _ = oracle.mul_mat(w, d, xq, xd)
    assert_close(y.cpu().numpy(), y_o, f"K={K}")


@pytest.mark.parametrize("B,Ks,q8_0,expect_mfma", [
    (5, (2048, 1024, 4096), (), 1),
    (6, (2048, 96), (), 0),
    (7, (14336, 1280), (), 1),
    (5, (2048, 1024), (1,), 0),
    (6, (2048, 512), (), 0),
    (7, (1024, 640), (0, 1), 1),
    (8, (1024, 1536, 2048), (), 1),
    (4, (2048, 4096), (), 0),
    (3, (2048, 4096), (), 0),
])
def test_grouped_multicolumn(B, Ks, q8_0, expect_mfma):
    print(f"[multicol group] B={B} Ks={Ks} q8_0={q8_0}", flush=True)
    probs, refs = [], []
    big = B == 8  # many windows per workgroup, the load fronts crossing products
    for i, K in enumerate(Ks):
        M = 40000 + 1000 * i if big else 96 + 40 * i
        w, d, xq, xd = _inputs(40 + i, M, K, B, q8_0=(i in q8_0))
        y = torch.full((B, M), float("nan"), device="cuda:0")
        key = "qw" if i in q8_0 else "qs"
        probs.append({key: to_dev(w), "d": to_dev(d.view(np.int16)), "y": y, "xq": to_dev(xq), "xd": to_dev(xd)})
        if i in q8_0:
            refs.append(oracle.mul_mat_q8w(w, d, xq, xd, nthreads=16)[0])
        else:
            refs.append(oracle.mul_mat(w, d, xq, xd, nthreads=16)[0])
    grp = q.Group(probs, B=B)
    assert grp.plan.mfma_columns == expect_mfma
    grp()
    torch.cuda.synchronize()
    for p, r in zip(probs, refs):
        yh = p["y"].cpu().numpy()
        assert np.isfinite(yh).all()
        assert_close(yh, r, f"B={B}")


def test_lanes_path_forces_the_lane_kernel():
    """Q4Q8_PATH_GEMV_LANES: the same product through the lane-per-block
    kernel, and group plans built under it without the multi-column one; both
    kernels against the oracle."""
    M, K, B = 300, 2048, 6
    w, d, xq, xd = _inputs(34, M, K, B)
    args = (to_dev(w), to_dev(d.view(np.int16)), to_dev(xq), to_dev(xd))
    y_o, _ = oracle.mul_mat(w, d, xq, xd, nthreads=16)
    try:
        for path, mfma in ((q.PATH_AUTO, True), (q.PATH_GEMV_LANES, False)):
            q.q4q8_set_path(path)
            y = q.mul_mat_q4q8(*args)
            torch.cuda.synchronize()
            assert ("gemv_mfma_kernel" in q.q4q8_last_kernel()) == mfma
            assert_close(y.cpu().numpy(), y_o, f"path {path}")
            out = torch.full((B, M), float("nan"), device="cuda:0")
            grp = q.Group([{"qs": args[0], "d": args[1], "y": out, "xq": args[2], "xd": args[3]}], B=B)
            assert grp.plan.mfma_columns == int(mfma)
            grp()
            torch.cuda.synchronize()
            assert np.array_equal(out.cpu().numpy().view(np.uint32), y.cpu().numpy().view(np.uint32))
    finally:
        q.q4q8_set_path(q.PATH_AUTO)
