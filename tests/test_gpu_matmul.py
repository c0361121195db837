"""GPU parity of mul_mat_q4q8 against the oracle.

Per-block int32 sums are compared bit for bit (debug instance of the same
kernel template), outputs within the normwise gates max-rel <= 1e-4 and
NMSE <= 1e-7 (fp32 accumulation order differs from the sequential oracle, so
several fp32 results are correct).  Full-size shapes of the Llama-3.2-1B and
Llama-3-8B decode layers are checked in full; prefill (T = 512, 2048) is
checked on sampled rows and tokens that the oracle computes one by one.
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
    qs, d = oracle.q4_quantize(w)
    xq, xd, _ = oracle.q8_quantize_rmsnorm(x, g, workloads.RMS_EPS)
    return qs, d, xq, xd


def _run(qs, d, xq, xd, blocksums=True):
    args = (to_dev(qs), to_dev(d.view(np.int16)), to_dev(xq), to_dev(xd))
    if blocksums:
        y, I = q.mul_mat_q4q8_blocksums(*args)
        torch.cuda.synchronize()
        return y.cpu().numpy(), I.cpu().numpy()
    y = q.mul_mat_q4q8(*args)
    torch.cuda.synchronize()
    return y.cpu().numpy(), None


@pytest.fixture(autouse=True)
def _auto_path():
    q.q4q8_set_path(q.PATH_AUTO)
    yield
    q.q4q8_set_path(q.PATH_AUTO)


SHAPES = [
    (1, 32, 1), (7, 64, 1), (256, 512, 1), (129, 1408, 2), (1000, 2048, 3), (33, 4096, 4),
    (64, 14336, 1), (300, 8192, 2),                                  # GEMV route, K in one wave
    (130, 1408, 5), (256, 512, 8), (33, 4096, 6), (77, 2048, 7),     # GEMV route, 5 to 8 columns
    (64, 14336, 2), (40, 16384, 4), (70, 8224, 3), (50, 14336, 8),   # GEMV route, K split over waves
    (3, 32768, 1), (5, 65536, 1), (40, 32768, 2),
    (130, 1408, 9), (1000, 2048, 33), (257, 4096, 130), (64, 14336, 16),
    (128, 64, 128), (1, 32, 200), (77, 8224, 20),                    # GEMM route (K = 8224: a 1-block last stage)
]


@pytest.mark.parametrize("M,K,B", SHAPES)
def test_blocksums_and_outputs(M, K, B):
    qs, d, xq, xd = _inputs(21, M, K, B, matrix=M % 7)
    y, I = _run(qs, d, xq, xd)
    assert np.array_equal(I, oracle.block_dots(qs, K, xq))
    y_o, _ = oracle.mul_mat(qs, d, xq, xd, nthreads=NTHREADS)
    assert_close(y, y_o, f"M={M} K={K} B={B}")
    y2, _ = _run(qs, d, xq, xd, blocksums=False)   # production instance agrees with the debug one
    assert_close(y2, y_o, "production instance")


@pytest.mark.parametrize("B", [1, 2, 3, 4, 5, 8, 9])
def test_forced_routes_agree(B):
    """Cross-check of the two routes (the GGML page keeps force-route switches
    only for such cross-checks): identical block sums, outputs both in tolerance."""
    M, K = 200, 1408
    qs, d, xq, xd = _inputs(22, M, K, B)
    y_o, _ = oracle.mul_mat(qs, d, xq, xd, nthreads=NTHREADS)
    I_o = oracle.block_dots(qs, K, xq)
    q.q4q8_set_path(q.PATH_GEMM)
    yg, Ig = _run(qs, d, xq, xd)
    assert np.array_equal(Ig, I_o)
    assert_close(yg, y_o, "forced gemm")
    if B <= 8:
        q.q4q8_set_path(q.PATH_GEMV)
        yv, Iv = _run(qs, d, xq, xd)
        assert np.array_equal(Iv, I_o)
        assert_close(yv, y_o, "forced gemv")
    else:
        q.q4q8_set_path(q.PATH_GEMV)
        with pytest.raises(q.Q4Q8Error) as ei:
            _run(qs, d, xq, xd)
        assert ei.value.status == q.Q4Q8_E_UNSUPPORTED


def test_route_counters():
    qs, d, xq, xd = _inputs(23, 64, 512, 16)
    q.q4q8_dispatch_counts(reset=True)
    _run(qs, d, xq[:1], xd[:1], blocksums=False)
    _run(qs, d, xq, xd, blocksums=False)
    c = q.q4q8_dispatch_counts(reset=True)
    assert c["gemv"] == 1 and c["gemm"] == 1


def test_degenerate_single_output():
    """m = 1, n = 1 with a long K: a single scalar dot (the OpenVINO page
    reports a GPU tolerance failure on exactly this degenerate shape)."""
    for K in (32, 2048, 14336):
        qs, d, xq, xd = _inputs(24, 1, K, 1)
        y, I = _run(qs, d, xq, xd)
        assert np.array_equal(I, oracle.block_dots(qs, K, xq))
        y_o, y64 = oracle.mul_mat(qs, d, xq, xd)
        assert_close(y, y_o, f"K={K}")


def test_empty_problems():
    dev = torch.device("cuda:0")
    qs = torch.zeros((0, 16), dtype=torch.uint8, device=dev)
    d = torch.zeros((0, 1), dtype=torch.int16, device=dev)
    xq = torch.zeros((3, 32), dtype=torch.int8, device=dev)
    xd = torch.zeros((3, 1), dtype=torch.float32, device=dev)
    assert q.mul_mat_q4q8(qs, d, xq, xd).shape == (3, 0)
    qs = torch.zeros((5, 16), dtype=torch.uint8, device=dev)
    d = torch.zeros((5, 1), dtype=torch.int16, device=dev)
    y = q.mul_mat_q4q8(qs, d, xq[:0], xd[:0])
    assert y.shape == (0, 5)


@pytest.mark.parametrize("model", ["llama-3.2-1b", "llama-3-8b"])
def test_full_decode_layer(model):
    """Every matrix of layer 0 at full shape, B = 1 (and B = 2, 4, 8 for the
    8B layer), through the fused prologue and the auto route."""
    layer = workloads.LLAMA_3_2_1B if model == "llama-3.2-1b" else workloads.LLAMA_3_8B
    batches = (1,) if model == "llama-3.2-1b" else (1, 2, 4, 8)
    dev = torch.device("cuda:0")
    for B in batches:
        acts = {}
        for slot, K in workloads.slot_k(layer).items():
            x = workloads.activation(0, 0, slot, B, K)
            g = workloads.norm_weight(0, 0, slot, K)
            xq, xd, _ = q.q8_quantize_rmsnorm(to_dev(x), to_dev(g), workloads.RMS_EPS)
            xq_o, xd_o, _ = oracle.q8_quantize_rmsnorm(x, g, workloads.RMS_EPS)
            assert np.array_equal(xq.cpu().numpy(), xq_o)
            acts[slot] = (xq, xd, xq_o, xd_o)
        for mi, mat in enumerate(layer):
            w = workloads.weight(0, 0, mi, mat.M, mat.K)
            qs, d = q.q4_quantize(to_dev(w))
            qs_o, d_o = oracle.q4_quantize(w)
            assert np.array_equal(qs.cpu().numpy(), qs_o), mat.name
            xq, xd, xq_o, xd_o = acts[mat.slot]
            y = q.mul_mat_q4q8(qs, d, xq, xd)
            torch.cuda.synchronize(dev)
            y_o, _ = oracle.mul_mat(qs_o, d_o, xq_o, xd_o, nthreads=NTHREADS, want_y64=False)
            assert_close(y.cpu().numpy(), y_o, f"{model} {mat.name} B={B}")


@pytest.mark.parametrize("T", [512, 2048])
def test_full_prefill_layer_sampled(T):
    """Prefill at full shape (T tokens, all seven Llama-3-8B matrices): the GPU
    computes every output (all of y must be written: it starts as NaN); its
    activation codes and scales equal the oracle prologue's bit for bit on
    sampled tokens, and the oracle recomputes 48 sampled rows x 48 sampled
    tokens of each matrix one by one from its own codes and scales."""
    dev = torch.device("cuda:0")
    layer = workloads.LLAMA_3_8B
    rng = np.random.default_rng(T)
    acts = {}
    for slot, K in workloads.slot_k(layer).items():
        x = workloads.activation(1, 0, slot, T, K)
        g = workloads.norm_weight(1, 0, slot, K)
        xq, xd, _ = q.q8_quantize_rmsnorm(to_dev(x), to_dev(g), workloads.RMS_EPS)
        acts[slot] = (xq, xd, x, g)
    for mi, mat in enumerate(layer):
        w = workloads.weight(1, 0, mi, mat.M, mat.K)
        qs, d = q.q4_quantize(to_dev(w))
        xq, xd, x, g = acts[mat.slot]
        y = torch.full((T, mat.M), float("nan"), dtype=torch.float32, device=dev)
        q.mul_mat_q4q8(qs, d, xq, xd, y=y)
        torch.cuda.synchronize(dev)
        assert bool(torch.isfinite(y).all()), f"prefill T={T} {mat.name}: unwritten or non-finite outputs"
        rows = np.sort(rng.choice(mat.M, 48, replace=False))
        toks = np.sort(rng.choice(T, 48, replace=False))
        rows[-1] = mat.M - 1
        toks[-1] = T - 1
        qs_o, d_o = oracle.q4_quantize(w[rows])
        xq_o, xd_o, _ = oracle.q8_quantize_rmsnorm(x[toks], g, workloads.RMS_EPS)
        assert np.array_equal(xq.cpu().numpy()[toks], xq_o)
        assert np.array_equal(xd.cpu().numpy()[toks].view(np.uint32), xd_o.view(np.uint32))
        y_o, _ = oracle.mul_mat(qs_o, d_o, xq_o, xd_o, nthreads=NTHREADS, want_y64=False)
        y_s = y.cpu().numpy()[np.ix_(toks, rows)]
        assert_close(y_s, y_o, f"prefill T={T} {mat.name}")


def test_prefill_down_projection_t512_full():
    """The Llama-3-8B down projection (4096 x 14336) at T = 512, on the tiled
    route: every one of the 2M outputs against the oracle (from the oracle's
    own weight codes and activation codes, which the GPU's equal bit for bit),
    and the int32 block sums of one 128-row tile column (all 512 tokens x 448
    blocks) bit for bit."""
    dev = torch.device("cuda:0")
    T, M, K = 512, 4096, 14336
    w = workloads.weight(8, 0, 6, M, K)
    x = workloads.activation(8, 0, 3, T, K)
    g = workloads.norm_weight(8, 0, 3, K)
    qs, d = q.q4_quantize(to_dev(w))
    xq, xd, _ = q.q8_quantize_rmsnorm(to_dev(x), to_dev(g), workloads.RMS_EPS)
    qs_o, d_o = oracle.q4_quantize(w)
    xq_o, xd_o, _ = oracle.q8_quantize_rmsnorm(x, g, workloads.RMS_EPS)
    assert np.array_equal(qs.cpu().numpy(), qs_o) and np.array_equal(d.cpu().numpy().view(np.uint16), d_o)
    assert np.array_equal(xq.cpu().numpy(), xq_o)
    assert np.array_equal(xd.cpu().numpy().view(np.uint32), xd_o.view(np.uint32))
    y = torch.full((T, M), float("nan"), dtype=torch.float32, device=dev)
    q.mul_mat_q4q8(qs, d, xq, xd, y=y)
    torch.cuda.synchronize(dev)
    y = y.cpu().numpy()
    assert np.isfinite(y).all()
    y_o, _ = oracle.mul_mat(qs_o, d_o, xq_o, xd_o, nthreads=NTHREADS, want_y64=False)
    assert_close(y, y_o, "down projection T=512, every output")
    col = slice(1920, 2048)   # one tile column of 128 weight rows
    yb, I = q.mul_mat_q4q8_blocksums(qs[col], d[col], xq, xd)
    torch.cuda.synchronize(dev)
    assert np.array_equal(I.cpu().numpy(), oracle.block_dots(qs_o[col], K, xq_o))
    assert_close(yb.cpu().numpy(), y_o[:, col], "tile column through the block-sum instance")
