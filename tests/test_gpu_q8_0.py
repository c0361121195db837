"""GPU parity of the Q8_0 weight type (q8_0_quantize, mul_mat_q8_0_q8) against
the oracle.

Quantised codes and fp16 scales are compared bit for bit, per-block int32 sums
bit for bit (debug instance of the same kernel template), outputs within the
normwise gates max-rel <= 1e-4 and NMSE <= 1e-7 (fp32 accumulation order
differs from the sequential oracle).  Both routes (streaming B <= 8, int8-MFMA
tiles above) are covered on ragged shapes, the K-split register classes, the
Llama-3-8B decode matrices at full shape and a prefill matrix on sampled
outputs.
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


def _inputs(seed, M, K, B, layer=0, matrix=0, slot=0):
    w = workloads.weight(seed, layer, matrix, M, K)
    x = workloads.activation(seed, layer, slot, B, K)
    g = workloads.norm_weight(seed, layer, slot, K)
    qw, d = oracle.q8w_quantize(w)
    xq, xd, _ = oracle.q8_quantize_rmsnorm(x, g, workloads.RMS_EPS)
    return qw, d, xq, xd


def _run(qw, d, xq, xd, blocksums=True):
    args = (to_dev(qw), to_dev(d.view(np.int16)), to_dev(xq), to_dev(xd))
    if blocksums:
        y, I = q.mul_mat_q8_0_q8_blocksums(*args)
        torch.cuda.synchronize()
        return y.cpu().numpy(), I.cpu().numpy()
    y = q.mul_mat_q8_0_q8(*args)
    torch.cuda.synchronize()
    return y.cpu().numpy(), None


@pytest.fixture(autouse=True)
def _auto_path():
    q.q4q8_set_path(q.PATH_AUTO)
    yield
    q.q4q8_set_path(q.PATH_AUTO)


@pytest.mark.parametrize("M,K", [(1, 32), (7, 96), (300, 4096), (1000, 2048), (3, 14336)])
def test_quantize_bit_exact(M, K):
    w = workloads.weight(31, 0, M % 5, M, K)
    w[0, :32] = 0.0                      # an all-zero block: d = 0, codes 0
    if K >= 64:
        w[-1, 32:64] = 0.0
        w[-1, 40] = -3.5                 # a lone extreme: codes -127 and 0
    qw, d = q.q8_0_quantize(to_dev(w))
    torch.cuda.synchronize()
    qw_o, d_o = oracle.q8w_quantize(w)
    assert np.array_equal(qw.cpu().numpy(), qw_o)
    assert np.array_equal(d.cpu().numpy().view(np.uint16), d_o)


SHAPES = [
    (1, 32, 1), (7, 64, 1), (256, 512, 1), (129, 1408, 2), (1000, 2048, 3), (33, 4096, 4),
    (64, 14336, 1), (300, 8192, 2),                                  # streaming route, K in one wave
    (130, 1408, 5), (256, 512, 8), (33, 4096, 6), (77, 2048, 7),     # streaming route, 5 to 8 columns
    (64, 14336, 2), (40, 16384, 4), (70, 8224, 3), (50, 14336, 8),   # streaming route, K split over waves
    (3, 32768, 1), (5, 65536, 1), (40, 32768, 2),
    (130, 1408, 9), (1000, 2048, 33), (257, 4096, 130), (64, 14336, 16),
    (128, 64, 128), (1, 32, 200), (77, 8224, 20),                    # tiled route (K = 8224: a 1-block last stage)
]


@pytest.mark.parametrize("M,K,B", SHAPES)
def test_blocksums_and_outputs(M, K, B):
    qw, d, xq, xd = _inputs(41, M, K, B, matrix=M % 7)
    y, I = _run(qw, d, xq, xd)
    assert np.array_equal(I, oracle.block_dots_q8w(qw, xq))
    y_o, _ = oracle.mul_mat_q8w(qw, d, xq, xd, nthreads=NTHREADS)
    assert_close(y, y_o, f"M={M} K={K} B={B}")
    y2, _ = _run(qw, d, xq, xd, blocksums=False)
    assert_close(y2, y_o, "production instance")


@pytest.mark.parametrize("B", [1, 2, 3, 4, 5, 8, 9])
def test_forced_routes_agree(B):
    M, K = 200, 1408
    qw, d, xq, xd = _inputs(42, M, K, B)
    y_o, _ = oracle.mul_mat_q8w(qw, d, xq, xd, nthreads=NTHREADS)
    I_o = oracle.block_dots_q8w(qw, xq)
    q.q4q8_set_path(q.PATH_GEMM)
    yg, Ig = _run(qw, d, xq, xd)
    assert np.array_equal(Ig, I_o)
    assert_close(yg, y_o, "forced gemm")
    q.q4q8_set_path(q.PATH_GEMV)
    if B <= 8:
        yv, Iv = _run(qw, d, xq, xd)
        assert np.array_equal(Iv, I_o)
        assert_close(yv, y_o, "forced gemv")
    else:
        with pytest.raises(q.Q4Q8Error) as ei:
            _run(qw, d, xq, xd)
        assert ei.value.status == q.Q4Q8_E_UNSUPPORTED


def test_extreme_codes():
    """Every weight and activation code at +-127: the largest block sums
    (|I| = 32 * 127 * 127) stay exact through the magic-seed rescale."""
    M, K, B = 70, 2048, 3
    qw = np.where(np.arange(M * K).reshape(M, K) % 3 == 0, -127, 127).astype(np.int8)
    d = oracle.f32_to_f16_bits(np.full((M, K // 32), 0.01, dtype=np.float32))
    xq = np.full((B, K), 127, dtype=np.int8)
    xq[1] = -127
    xd = np.full((B, K // 32), 0.02, dtype=np.float32)
    for path in (q.PATH_GEMV, q.PATH_GEMM):
        q.q4q8_set_path(path)
        y, I = _run(qw, d, xq, xd)
        assert np.array_equal(I, oracle.block_dots_q8w(qw, xq))
        y_o, _ = oracle.mul_mat_q8w(qw, d, xq, xd)
        assert_close(y, y_o, f"path {path}")


def test_empty_problems():
    dev = torch.device("cuda:0")
    qw = torch.zeros((0, 32), dtype=torch.int8, device=dev)
    d = torch.zeros((0, 1), dtype=torch.int16, device=dev)
    xq = torch.zeros((3, 32), dtype=torch.int8, device=dev)
    xd = torch.zeros((3, 1), dtype=torch.float32, device=dev)
    assert q.mul_mat_q8_0_q8(qw, d, xq, xd).shape == (3, 0)
    qw = torch.zeros((5, 32), dtype=torch.int8, device=dev)
    d = torch.zeros((5, 1), dtype=torch.int16, device=dev)
    assert q.mul_mat_q8_0_q8(qw, d, xq[:0], xd[:0]).shape == (0, 5)


def test_full_decode_layer_8b():
    """Every Llama-3-8B layer-0 matrix at full shape as Q8_0, B = 1 and 8,
    GPU-quantised weights and GPU prologue."""
    layer = workloads.LLAMA_3_8B
    dev = torch.device("cuda:0")
    for B in (1, 8):
        acts = {}
        for slot, K in workloads.slot_k(layer).items():
            x = workloads.activation(0, 0, slot, B, K)
            g = workloads.norm_weight(0, 0, slot, K)
            xq, xd, _ = q.q8_quantize_rmsnorm(to_dev(x), to_dev(g), workloads.RMS_EPS)
            xq_o, xd_o, _ = oracle.q8_quantize_rmsnorm(x, g, workloads.RMS_EPS)
            acts[slot] = (xq, xd, xq_o, xd_o)
        for mi, mat in enumerate(layer):
            w = workloads.weight(0, 0, mi, mat.M, mat.K)
            qw, d = q.q8_0_quantize(to_dev(w))
            qw_o, d_o = oracle.q8w_quantize(w)
            assert np.array_equal(qw.cpu().numpy(), qw_o), mat.name
            assert np.array_equal(d.cpu().numpy().view(np.uint16), d_o), mat.name
            xq, xd, xq_o, xd_o = acts[mat.slot]
            y = q.mul_mat_q8_0_q8(qw, d, xq, xd)
            torch.cuda.synchronize(dev)
            y_o, _ = oracle.mul_mat_q8w(qw_o, d_o, xq_o, xd_o, nthreads=NTHREADS, want_y64=False)
            assert_close(y.cpu().numpy(), y_o, f"{mat.name} B={B}")


def test_prefill_sampled():
    """Prefill of the Llama-3-8B gate matrix (14336 x 4096) as Q8_0 at T = 2048
    on the tiled route: 48 sampled rows x 48 sampled tokens recomputed by the
    oracle."""
    dev = torch.device("cuda:0")
    T, M, K = 2048, 14336, 4096
    rng = np.random.default_rng(7)
    x = workloads.activation(2, 0, 2, T, K)
    g = workloads.norm_weight(2, 0, 2, K)
    xq, xd, _ = q.q8_quantize_rmsnorm(to_dev(x), to_dev(g), workloads.RMS_EPS)
    w = workloads.weight(2, 0, 4, M, K)
    qw, d = q.q8_0_quantize(to_dev(w))
    y = q.mul_mat_q8_0_q8(qw, d, xq, xd)
    torch.cuda.synchronize(dev)
    rows = np.sort(rng.choice(M, 48, replace=False))
    toks = np.sort(rng.choice(T, 48, replace=False))
    rows[-1], toks[-1] = M - 1, T - 1
    qw_o, d_o = oracle.q8w_quantize(w[rows])
    xq_o, xd_o, _ = oracle.q8_quantize_rmsnorm(x[toks], g, workloads.RMS_EPS)
    assert np.array_equal(xq.cpu().numpy()[toks], xq_o)
    y_o, _ = oracle.mul_mat_q8w(qw_o, d_o, xq_o, xd_o, nthreads=NTHREADS, want_y64=False)
    assert_close(y.cpu().numpy()[np.ix_(toks, rows)], y_o, "prefill gate T=2048")


@pytest.mark.parametrize("B", [1, 3, 6, 8, 20])
def test_group_mixes_weight_formats(B):
    """One grouped launch over Q4 and Q8_0 products (streaming for B <= 8,
    tiled above), some on Q8 planes and some on fp32 rows through the
    prologue pass; every output against the oracle and, bit for bit, against
    the single-product entry point on the same codes where both take the
    same kernel (a group mixing weight formats streams through the
    lane-per-block kernel at every B <= 8, a single product of B = 5..8 may
    take the multi-column one, whose fp32 sums run in another order)."""
    shapes = [(300, 2048), (77, 4096), (1000, 1408), (33, 14336), (129, 512), (64, 8192)]
    probs, refs = [], []
    dev = torch.device("cuda:0")
    for i, (M, K) in enumerate(shapes):
        w = workloads.weight(51, 0, i, M, K)
        x = workloads.activation(51, 0, i, B, K)
        g = workloads.norm_weight(51, 0, i, K)
        xq_o, xd_o, _ = oracle.q8_quantize_rmsnorm(x, g, workloads.RMS_EPS)
        y = torch.zeros((B, M), dtype=torch.float32, device=dev)
        p = {"d": None, "y": y}
        if i % 2 == 0:
            qw, d = oracle.q8w_quantize(w)
            p["qw"] = to_dev(qw)
            y_o, _ = oracle.mul_mat_q8w(qw, d, xq_o, xd_o, nthreads=NTHREADS, want_y64=False)
        else:
            qs, d = oracle.q4_quantize(w)
            p["qs"] = to_dev(qs)
            y_o, _ = oracle.mul_mat(qs, d, xq_o, xd_o, nthreads=NTHREADS, want_y64=False)
        p["d"] = to_dev(d.view(np.int16))
        if i % 3 == 0:
            p.update(x=to_dev(x), g=to_dev(g), eps=workloads.RMS_EPS)
        else:
            p.update(xq=to_dev(xq_o), xd=to_dev(xd_o))
        probs.append(p)
        refs.append((y_o, xq_o, xd_o))
    grp = q.Group(probs, B=B)
    assert grp.plan.mfma_columns == 0
    grp()
    torch.cuda.synchronize()
    group_kernel = q.q4q8_last_kernel()
    n_bitwise = 0
    for i, (p, (y_o, xq_o, xd_o)) in enumerate(zip(probs, refs)):
        M, K = shapes[i]
        assert_close(p["y"].cpu().numpy(), y_o, f"product {i} M={M} K={K} B={B}")
        xq_d, xd_d = to_dev(xq_o), to_dev(xd_o)
        if "qw" in p:
            y1 = q.mul_mat_q8_0_q8(p["qw"], p["d"], xq_d, xd_d)
        else:
            y1 = q.mul_mat_q4q8(p["qs"], p["d"], xq_d, xd_d)
        torch.cuda.synchronize()
        if ("gemv_mfma_kernel" in q.q4q8_last_kernel()) == ("gemv_mfma_kernel" in group_kernel):
            n_bitwise += 1
            assert np.array_equal(y1.cpu().numpy().view(np.uint32), p["y"].cpu().numpy().view(np.uint32)), i
    if not 5 <= B <= 8:
        assert n_bitwise == len(shapes)


@pytest.mark.parametrize("B", [2, 8])
def test_mixed_group_in_a_graph(B):
    """A group mixing Q4 and Q8_0 products, some on fp32 rows (prologue pass),
    captured in a HIP graph; every replay, with eager launches of the same
    group in between, equals the eager result bit for bit, which matches the
    oracle."""
    dev = torch.device("cuda:0")
    shapes = [(1024, 4096), (512, 14336), (2048, 2048), (300, 4096)]
    probs, refs = [], []
    for i, (M, K) in enumerate(shapes):
        w = workloads.weight(61, 0, i, M, K)
        x = workloads.activation(61, 0, i % 2, B, K)
        g = workloads.norm_weight(61, 0, i % 2, K)
        xq_o, xd_o, _ = oracle.q8_quantize_rmsnorm(x, g, workloads.RMS_EPS)
        p = {"y": torch.zeros((B, M), dtype=torch.float32, device=dev)}
        if i % 2 == 0:
            qw, d = oracle.q8w_quantize(w)
            p["qw"] = to_dev(qw)
            refs.append(oracle.mul_mat_q8w(qw, d, xq_o, xd_o, nthreads=NTHREADS, want_y64=False)[0])
        else:
            qs, d = oracle.q4_quantize(w)
            p["qs"] = to_dev(qs)
            refs.append(oracle.mul_mat(qs, d, xq_o, xd_o, nthreads=NTHREADS, want_y64=False)[0])
        p["d"] = to_dev(d.view(np.int16))
        p.update(x=to_dev(x), g=to_dev(g), eps=workloads.RMS_EPS)
        probs.append(p)
    grp = q.Group(probs, B=B)
    assert grp.plan.weight_formats == 3
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        grp()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    eager = [p["y"].cpu().numpy().copy() for p in probs]
    for i, (y, ref) in enumerate(zip(eager, refs)):
        assert_close(y, ref, f"eager product {i}")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        grp()
    for rep in range(3):
        for p in probs:
            p["y"].zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (p, y) in enumerate(zip(probs, eager)):
            assert np.array_equal(p["y"].cpu().numpy().view(np.uint32), y.view(np.uint32)), (rep, i)
        grp()                      # eager work between replays
        torch.cuda.synchronize()
