"""GPU parity of the folded-in prologue product (mul_mat_q4q8_rmsnorm) and of
grouped streaming launches (mul_mat_q4q8_group) against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import assert_close, to_dev

pytestmark = pytest.mark.gpu

q = pytest.importorskip("block_quantized_matmul_q8_amd")


def _weights(seed, layer, matrix, M, K):
    w = workloads.weight(seed, layer, matrix, M, K)
    qs, d = oracle.q4_quantize(w)
    return qs, d


def _ref(qs, d, x, g, no_norm=False):
    xq, xd, _ = oracle.q8_quantize_rmsnorm(x, g, workloads.RMS_EPS, no_norm=no_norm)
    y, _ = oracle.mul_mat(qs, d, xq, xd, nthreads=16, want_y64=False)
    return y


@pytest.mark.parametrize("M,K,B", [(1, 32, 1), (7, 64, 1), (256, 512, 1), (130, 1408, 2), (1000, 2048, 1),
                                   (300, 4096, 3), (64, 8192, 1), (200, 14336, 1), (96, 2048, 4),
                                   (40, 8192, 2)])
def test_fused_single(M, K, B):
    qs, d = _weights(41, 0, M % 5, M, K)
    x = workloads.activation(41, 0, 0, B, K)
    g = workloads.norm_weight(41, 0, 0, K)
    y = q.mul_mat_q4q8_rmsnorm(to_dev(qs), to_dev(d.view(np.int16)), to_dev(x), to_dev(g), workloads.RMS_EPS)
    torch.cuda.synchronize()
    assert_close(y.cpu().numpy(), _ref(qs, d, x, g), f"M={M} K={K} B={B}")


@pytest.mark.parametrize("M,K,B,raw", [(256, 512, 1, False), (130, 1408, 2, False), (1000, 2048, 1, False),
                                       (300, 4096, 3, False), (64, 8192, 1, False), (200, 14336, 1, False),
                                       (96, 2048, 4, False), (77, 2048, 1, True), (40, 8192, 2, True)])
def test_fused_codes_equal_standalone_prologue(M, K, B, raw):
    """The folded-in prologue produces the codes of the standalone prologue
    bit for bit: with identical codes the product kernel does identical
    arithmetic in both modes, so the outputs must agree bit for bit.  The
    exceptions are one column with K > 8192 and two with K > 4096, where the
    plain product splits K over waves while the folded form keeps K in one
    wave, and three or more columns, where the plain product may run the
    multi-column MFMA kernel: there the two fp32 sums differ in rounding
    order and both are held to the oracle instead."""
    qs, d = _weights(44, 0, M % 5, M, K)
    x = workloads.activation(44, 0, 1, B, K) * np.float32(2.5)
    g = workloads.norm_weight(44, 0, 1, K)
    qs_d, d_d, x_d = to_dev(qs), to_dev(d.view(np.int16)), to_dev(x)
    g_d = None if raw else to_dev(g)
    flags = q.Q8_NO_NORM if raw else 0
    y_f = q.mul_mat_q4q8_rmsnorm(qs_d, d_d, x_d, g_d, workloads.RMS_EPS, flags=flags)
    xq, xd, _ = q.q8_quantize_rmsnorm(x_d, g_d, workloads.RMS_EPS, flags=flags)
    y_u = q.mul_mat_q4q8(qs_d, d_d, xq, xd)
    torch.cuda.synchronize()
    plain_mfma = "gemv_mfma_kernel" in q.q4q8_last_kernel()
    if (B == 1 and K > 8192) or (B == 2 and K > 4096) or plain_mfma:
        ref = _ref(qs, d, x, None if raw else g, no_norm=raw)
        assert_close(y_f.cpu().numpy(), ref, f"folded M={M} K={K}")
        assert_close(y_u.cpu().numpy(), ref, f"plain M={M} K={K}")
    else:
        assert np.array_equal(y_f.cpu().numpy().view(np.uint32), y_u.cpu().numpy().view(np.uint32))
    xq_o, _, _ = oracle.q8_quantize_rmsnorm(x, None if raw else g, workloads.RMS_EPS, no_norm=raw)
    assert np.array_equal(xq.cpu().numpy(), xq_o)


def test_fused_no_norm_and_special_rows(hand_examples):
    M, K = 48, 1408
    qs, d = _weights(42, 0, 0, M, K)
    x = workloads.activation(42, 0, 0, 3, K) * np.float32(4.0)
    x[1] = 0.0                      # all-zero row: codes 0, output 0
    y = q.mul_mat_q4q8_rmsnorm(to_dev(qs), to_dev(d.view(np.int16)), to_dev(x), None, 0.0, flags=q.Q8_NO_NORM)
    torch.cuda.synchronize()
    ref = _ref(qs, d, x, None, no_norm=True)
    assert_close(y.cpu().numpy(), ref)
    assert np.all(y.cpu().numpy()[1] == 0.0)
    # hand example E5 through the folded-in prologue: y = -15.999921 exactly
    e5 = hand_examples["E5"]
    w = np.array([[-8 + (j % 16) for j in range(32)]], np.float32)
    qs1, d1 = oracle.q4_quantize(w)
    y1 = q.mul_mat_q4q8_rmsnorm(to_dev(qs1), to_dev(d1.view(np.int16)), to_dev(np.ones((1, 32), np.float32)),
                                to_dev(np.ones(32, np.float32)), 1e-5)
    torch.cuda.synchronize()
    assert int(y1.cpu().numpy().view(np.uint32)[0, 0]) == int(e5["y_bits"], 16)


@pytest.mark.parametrize("B", [1, 2, 3, 4, 8])
def test_group_mixed(B):
    """Products of different blocking classes (K in one wave or split over
    waves) and all activation modes in one group."""
    dev = torch.device("cuda:0")
    specs = [(512, 2048, "q8"), (130, 1408, "norm"), (64, 8192, "norm"), (300, 4096, "raw"),
             (1, 32, "q8"), (2048, 2048, "norm"), (33, 14336, "q8"), (70, 16384, "norm"),
             (20, 16416, "raw")]
    problems, refs = [], []
    for i, (M, K, mode) in enumerate(specs):
        if K > 16384 and B > 2:
            continue                # beyond the streaming kernel's register blocking for B > 2
        qs, d = _weights(43, 1, i, M, K)
        x = workloads.activation(43, 1, i, B, K)
        g = workloads.norm_weight(43, 1, i, K)
        y = torch.full((B, M), float("nan"), dtype=torch.float32, device=dev)
        p = {"qs": to_dev(qs), "d": to_dev(d.view(np.int16)), "y": y}
        if mode == "q8":
            xq, xd, _ = oracle.q8_quantize_rmsnorm(x, g, workloads.RMS_EPS)
            p.update(xq=to_dev(xq), xd=to_dev(xd))
            ref, _ = oracle.mul_mat(qs, d, xq, xd, nthreads=16, want_y64=False)
        elif mode == "norm":
            p.update(x=to_dev(x), g=to_dev(g), eps=workloads.RMS_EPS)
            ref = _ref(qs, d, x, g)
        else:
            p.update(x=to_dev(x), flags=q.Q8_NO_NORM)
            ref = _ref(qs, d, x, None, no_norm=True)
        problems.append(p)
        refs.append(ref)
    grp = q.Group(problems, B=B)
    assert grp.plan.n_prologue == sum(1 for p in problems if "x" in p)
    for rep in range(2):          # the same device table launched twice
        for p in problems:
            p["y"].fill_(float("nan"))
        grp()
        torch.cuda.synchronize()
        for p, ref in zip(problems, refs):
            assert_close(p["y"].cpu().numpy(), ref, f"rep {rep} M={p['qs'].shape[0]}")
    # the group's prologue pass gives the codes of q8_quantize_rmsnorm and
    # the streaming pass runs the single-product arithmetic, so the outputs
    # agree bit for bit with the two standalone calls -- where both take the
    # same streaming kernel: a single product of B = 5..8 columns with rows of
    # four or more whole 128-byte segments takes the multi-column one, a group only when
    # every product can (grp.plan.mfma_columns)
    group_mfma = "gemv_mfma_kernel" in q.q4q8_last_kernel()
    assert group_mfma == bool(grp.plan.mfma_columns)
    for p, ref in zip(problems, refs):
        if "x" in p:
            raw = p.get("flags", 0) == q.Q8_NO_NORM
            xq, xd, _ = q.q8_quantize_rmsnorm(p["x"], None if raw else p["g"], workloads.RMS_EPS,
                                              flags=p.get("flags", 0))
        else:
            xq, xd = p["xq"], p["xd"]
        single = q.mul_mat_q4q8(p["qs"], p["d"], xq, xd)
        torch.cuda.synchronize()
        if ("gemv_mfma_kernel" in q.q4q8_last_kernel()) == group_mfma:
            assert np.array_equal(single.cpu().numpy().view(np.uint32), p["y"].cpu().numpy().view(np.uint32))
        else:
            assert_close(single.cpu().numpy(), ref, "single call")


@pytest.mark.parametrize("k_max", [32768, 32800])
def test_one_column_group_at_the_instance_boundary(k_max):
    """One-column groups whose largest K is 32768 take the instance built
    without the 8-block classes (K split over 2 or 4 waves above 8192); one
    more block takes the full instance.  Both mix every smaller class and must
    match the oracle, and each product must equal its single-product call bit
    for bit."""
    dev = torch.device("cuda:0")
    specs = [(257, 32), (96, 1024), (130, 2048), (75, 4096), (300, 6144), (64, 8192), (40, 8224),
             (33, 14336), (21, 16416), (17, k_max)]
    problems, refs = [], []
    for i, (M, K) in enumerate(specs):
        qs, d = _weights(46, 0, i, M, K)
        x = workloads.activation(46, 0, i, 1, K)
        g = workloads.norm_weight(46, 0, i, K)
        xq, xd, _ = oracle.q8_quantize_rmsnorm(x, g, workloads.RMS_EPS)
        y = torch.full((1, M), float("nan"), dtype=torch.float32, device=dev)
        problems.append({"qs": to_dev(qs), "d": to_dev(d.view(np.int16)), "xq": to_dev(xq), "xd": to_dev(xd),
                         "y": y})
        refs.append(oracle.mul_mat(qs, d, xq, xd, nthreads=16, want_y64=False)[0])
    grp = q.Group(problems, B=1)
    assert grp.plan.max_k == k_max
    grp()
    torch.cuda.synchronize()
    for p, ref in zip(problems, refs):
        assert_close(p["y"].cpu().numpy(), ref, f"k_max={k_max} M={p['qs'].shape[0]}")
        single = q.mul_mat_q4q8(p["qs"], p["d"], p["xq"], p["xd"])
        torch.cuda.synchronize()
        assert np.array_equal(single.cpu().numpy().view(np.uint32), p["y"].cpu().numpy().view(np.uint32))


def test_group_full_llama_1b_layer_in_a_graph():
    """One Llama-3.2-1B layer (seven matrices, four activation rows with their
    own norm weights) as one group with the prologue folded in, captured in a
    HIP graph and replayed; every replay matches the oracle."""
    dev = torch.device("cuda:0")
    layer = workloads.LLAMA_3_2_1B
    xs = {s: workloads.activation(0, 3, s, 1, K) for s, K in workloads.slot_k(layer).items()}
    gs = {s: workloads.norm_weight(0, 3, s, K) for s, K in workloads.slot_k(layer).items()}
    xs_d = {s: to_dev(v) for s, v in xs.items()}
    gs_d = {s: to_dev(v) for s, v in gs.items()}
    problems, refs = [], []
    for mi, m in enumerate(layer):
        qs, d = _weights(0, 3, mi, m.M, m.K)
        y = torch.zeros((1, m.M), dtype=torch.float32, device=dev)
        problems.append({"qs": to_dev(qs), "d": to_dev(d.view(np.int16)), "y": y, "x": xs_d[m.slot],
                         "g": gs_d[m.slot], "eps": workloads.RMS_EPS})
        refs.append(_ref(qs, d, xs[m.slot], gs[m.slot]))
    grp = q.Group(problems, B=1)
    assert grp.plan.n_prologue == 4           # Q/K/V share a row, gate/up another
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        grp()                       # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        grp()
    for rep in range(3):
        for p in problems:
            p["y"].zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for p, ref, m in zip(problems, refs, layer):
            assert_close(p["y"].cpu().numpy(), ref, f"replay {rep} {m.name}")


@pytest.mark.parametrize("B", [1, 2, 4, 8])
def test_group_full_llama_8b_layer(B):
    """One Llama-3-8B layer at full shape as one grouped call with fp32 rows
    (prologue pass, then the streaming pass; K = 14336 is split over waves
    for B > 1), every output against the oracle."""
    dev = torch.device("cuda:0")
    layer = workloads.LLAMA_3_8B
    xs = {s: workloads.activation(5, 0, s, B, K) for s, K in workloads.slot_k(layer).items()}
    gs = {s: workloads.norm_weight(5, 0, s, K) for s, K in workloads.slot_k(layer).items()}
    xs_d = {s: to_dev(v) for s, v in xs.items()}
    gs_d = {s: to_dev(v) for s, v in gs.items()}
    problems, refs = [], []
    for mi, m in enumerate(layer):
        qs, d = _weights(5, 0, mi, m.M, m.K)
        y = torch.full((B, m.M), float("nan"), dtype=torch.float32, device=dev)
        problems.append({"qs": to_dev(qs), "d": to_dev(d.view(np.int16)), "y": y, "x": xs_d[m.slot],
                         "g": gs_d[m.slot], "eps": workloads.RMS_EPS})
        refs.append(_ref(qs, d, xs[m.slot], gs[m.slot]))
    grp = q.Group(problems, B=B)
    grp()
    torch.cuda.synchronize()
    for p, ref, m in zip(problems, refs, layer):
        assert_close(p["y"].cpu().numpy(), ref, f"B={B} {m.name}")


@pytest.mark.parametrize("B", [9, 130, 300])
def test_group_tiled_mixed(B):
    """B > 8 takes the tiled MFMA route: ragged products with Q8 planes and
    fp32 rows in one launch; every output against the oracle, and bit for bit
    against the single-product calls (the same tile arithmetic)."""
    dev = torch.device("cuda:0")
    specs = [(200, 1408, "norm"), (130, 4096, "q8"), (64, 2080, "raw"), (257, 512, "norm")]
    problems, refs = [], []
    for i, (M, K, mode) in enumerate(specs):
        qs, d = _weights(47, 2, i, M, K)
        x = workloads.activation(47, 2, i, B, K)
        g = workloads.norm_weight(47, 2, i, K)
        y = torch.full((B, M), float("nan"), dtype=torch.float32, device=dev)
        p = {"qs": to_dev(qs), "d": to_dev(d.view(np.int16)), "y": y}
        if mode == "q8":
            xq, xd, _ = oracle.q8_quantize_rmsnorm(x, g, workloads.RMS_EPS)
            p.update(xq=to_dev(xq), xd=to_dev(xd))
            ref, _ = oracle.mul_mat(qs, d, xq, xd, nthreads=16, want_y64=False)
        elif mode == "norm":
            p.update(x=to_dev(x), g=to_dev(g), eps=workloads.RMS_EPS)
            ref = _ref(qs, d, x, g)
        else:
            p.update(x=to_dev(x), flags=q.Q8_NO_NORM)
            ref = _ref(qs, d, x, None, no_norm=True)
        problems.append(p)
        refs.append(ref)
    grp = q.Group(problems, B=B)
    q.q4q8_dispatch_counts(reset=True)
    grp()
    torch.cuda.synchronize()
    assert q.q4q8_dispatch_counts(reset=True)["gemm"] == 1
    for p, ref in zip(problems, refs):
        assert_close(p["y"].cpu().numpy(), ref, f"B={B} M={p['qs'].shape[0]}")
        if "x" in p:
            raw = p.get("flags", 0) == q.Q8_NO_NORM
            xq, xd, _ = q.q8_quantize_rmsnorm(p["x"], None if raw else p["g"], workloads.RMS_EPS,
                                              flags=p.get("flags", 0))
        else:
            xq, xd = p["xq"], p["xd"]
        single = q.mul_mat_q4q8(p["qs"], p["d"], xq, xd)
        torch.cuda.synchronize()
        assert np.array_equal(single.cpu().numpy().view(np.uint32), p["y"].cpu().numpy().view(np.uint32))


@pytest.mark.parametrize("T", [512, 2048])
def test_group_tiled_prefill_layer_sampled(T):
    """A Llama-3-8B-shaped prefill layer (T tokens, all seven matrices, fp32
    rows through the prologue pass) as one grouped tiled launch, the launch
    the benchmark times.  Every output must be written (y starts as NaN); the
    oracle recomputes 40 sampled rows x 40 sampled tokens of each matrix,
    including the last row and token, and at T = 512 every output of the down
    projection (4096 x 14336)."""
    dev = torch.device("cuda:0")
    layer = workloads.LLAMA_3_8B
    rng = np.random.default_rng(T + 1)
    xs = {s: workloads.activation(6, 0, s, T, K) for s, K in workloads.slot_k(layer).items()}
    gs = {s: workloads.norm_weight(6, 0, s, K) for s, K in workloads.slot_k(layer).items()}
    xs_d = {s: to_dev(v) for s, v in xs.items()}
    gs_d = {s: to_dev(v) for s, v in gs.items()}
    problems, ws = [], []
    for mi, m in enumerate(layer):
        w = workloads.weight(6, 0, mi, m.M, m.K)
        qs, d = q.q4_quantize(to_dev(w))
        y = torch.full((T, m.M), float("nan"), dtype=torch.float32, device=dev)
        problems.append({"qs": qs, "d": d, "y": y, "x": xs_d[m.slot], "g": gs_d[m.slot],
                         "eps": workloads.RMS_EPS})
        ws.append(w)
    grp = q.Group(problems, B=T)
    grp()
    torch.cuda.synchronize()
    for p, m in zip(problems, layer):
        assert bool(torch.isfinite(p["y"]).all()), f"T={T} {m.name}: unwritten or non-finite outputs"
    for p, w, m in zip(problems, ws, layer):
        rows = np.sort(rng.choice(m.M, 40, replace=False))
        toks = np.sort(rng.choice(T, 40, replace=False))
        rows[-1], toks[-1] = m.M - 1, T - 1
        qs_o, d_o = oracle.q4_quantize(w[rows])
        xq_o, xd_o, _ = oracle.q8_quantize_rmsnorm(xs[m.slot][toks], gs[m.slot], workloads.RMS_EPS)
        y_o, _ = oracle.mul_mat(qs_o, d_o, xq_o, xd_o, nthreads=16, want_y64=False)
        y_s = p["y"].cpu().numpy()[np.ix_(toks, rows)]
        assert_close(y_s, y_o, f"T={T} {m.name}")
        if T == 512 and m.name == "down":
            qs_f, d_f = oracle.q4_quantize(w)
            xq_f, xd_f, _ = oracle.q8_quantize_rmsnorm(xs[m.slot], gs[m.slot], workloads.RMS_EPS)
            y_f, _ = oracle.mul_mat(qs_f, d_f, xq_f, xd_f, nthreads=16, want_y64=False)
            assert_close(p["y"].cpu().numpy(), y_f, f"T={T} down, every output")


def test_full_decode_step_sampled():
    """The benchmark's headline launch as it is timed: all 16 Llama-3.2-1B
    layers (112 products, 64 fp32 activation rows with their norm weights) as
    one grouped call, weights drawn on the device as in the benchmark.  Every
    output must be written (y starts as NaN); the oracle recomputes 12 sampled
    rows of every product (the last row included) from the same weights and
    rows."""
    import bench
    dev = torch.device("cuda:0")
    model = bench.DecodeModel(workloads.LLAMA_3_2_1B, 16, 1, 0, dev)
    step, _ = bench.decode_1b_groups(model)
    for m in (mm for layer in model.mats for mm in layer):
        m["y"].fill_(float("nan"))
    step()
    torch.cuda.synchronize()
    for m in (mm for layer in model.mats for mm in layer):
        assert bool(torch.isfinite(m["y"]).all()), f"{m['name']}: unwritten or non-finite outputs"
    rng = np.random.default_rng(7)
    for l in range(model.n_layers):
        acts = {s: (x.cpu().numpy(), g.cpu().numpy()) for s, (x, g) in model.acts[l].items()}
        for m in model.mats[l]:
            rows = np.sort(rng.choice(m["M"], 12, replace=False))
            rows[-1] = m["M"] - 1
            qs = m["qs"].cpu().numpy()[rows]
            d = m["d"].cpu().numpy().view(np.uint16)[rows]
            x, g = acts[m["slot"]]
            y_o = _ref(qs, d, x, g)
            assert_close(m["y"].cpu().numpy()[:, rows], y_o, f"layer {l} {m['name']}")


_PROLOGUE_CASES = ([(1, K) for K in (32, 96, 1408, 2048, 8192, 8224, 14336, 32768, 32800)] +
                   [(3, K) for K in (96, 2048, 8192, 8224, 14336)] +
                   [(8, K) for K in (96, 2048, 8192, 8224, 14336, 32768)] +
                   [(9, K) for K in (2048, 14336)])


@pytest.mark.parametrize("raw", [False, True])
@pytest.mark.parametrize("B,K", _PROLOGUE_CASES)
def test_group_prologue_planes_bit_exact(B, K, raw):
    """The grouped prologue pass's own Q8 planes (read out of the group's
    workspace, where the first fp32 input's codes [B][K] start at offset 0 and
    its scales [B][K/32] at the next 16-byte boundary) equal the oracle's bit
    for bit: the 1024-thread forms for B <= 8 (four lanes per block up to K =
    8192, one lane per block up to 32768, the LDS tree beyond) and the
    256-thread form above; zero rows, tiny rows and a lone spike included."""
    print(f"[group prologue] B={B} K={K} raw={raw}", flush=True)
    x = workloads.activation(48, B, K % 97, B, K) * np.float32(1.7)
    if B >= 3:
        x[1] = 0.0
        x[2] *= np.float32(1e-20)
        x[0, K // 3] = np.float32(3000.0)
    g = workloads.norm_weight(48, 0, K % 89, K)
    M = 16
    qs, d = _weights(48, 0, 0, M, K)
    y = torch.full((B, M), float("nan"), device="cuda:0")
    p = {"qs": to_dev(qs), "d": to_dev(d.view(np.int16)), "y": y, "x": to_dev(x)}
    if raw:
        p["flags"] = q.Q8_NO_NORM
    else:
        p.update(g=to_dev(g), eps=workloads.RMS_EPS)
    grp = q.Group([p], B=B)
    assert grp.plan.n_prologue == 1
    grp.workspace.fill_(0xA5)
    grp()
    torch.cuda.synchronize()
    ws = grp.workspace.cpu().numpy()
    off = (B * K + 15) // 16 * 16
    xq = ws[:B * K].view(np.int8).reshape(B, K)
    xd = ws[off:off + B * (K // 32) * 4].view(np.uint32).reshape(B, K // 32)
    xq_o, xd_o, _ = oracle.q8_quantize_rmsnorm(x, None if raw else g, workloads.RMS_EPS, no_norm=raw)
    assert np.array_equal(xq, xq_o)
    assert np.array_equal(xd, xd_o.view(np.uint32))
    y_o, _ = oracle.mul_mat(qs, d, xq_o, xd_o, nthreads=16, want_y64=False)
    assert np.isfinite(y.cpu().numpy()).all()
    assert_close(y.cpu().numpy(), y_o, f"B={B} K={K}")


@pytest.mark.parametrize("B", [1, 3, 8])
def test_group_prologue_packed_rows_mixed(B):
    """A decode group's prologue pass over fp32 inputs of different K (one
    32-block to 14336), raw rows beside normalised ones: every input's planes,
    read out of the workspace, equal the oracle's bit for bit, and the outputs
    the oracle's product."""
    print(f"[packed prologue] B={B}", flush=True)
    ks = [2048, 2048, 1024, 96, 8192, 4096, 4096, 14336, 32, 2048]
    M = 16
    probs, refs, layout = [], [], []
    off = 0
    for i, K in enumerate(ks):
        raw = i % 3 == 1
        x = workloads.activation(49, B, i, B, K) * np.float32(1.3)
        if B >= 3:
            x[1] = 0.0
        g = workloads.norm_weight(49, 0, i, K)
        qs, d = _weights(49, 0, i, M, K)
        y = torch.full((B, M), float("nan"), device="cuda:0")
        p = {"qs": to_dev(qs), "d": to_dev(d.view(np.int16)), "y": y, "x": to_dev(x)}
        if raw:
            p["flags"] = q.Q8_NO_NORM
        else:
            p.update(g=to_dev(g), eps=workloads.RMS_EPS)
        probs.append(p)
        xq_o, xd_o, _ = oracle.q8_quantize_rmsnorm(x, None if raw else g, workloads.RMS_EPS, no_norm=raw)
        refs.append((qs, d, xq_o, xd_o))
        xd_off = off + (B * K + 15) // 16 * 16
        layout.append((off, xd_off, K))
        off = xd_off + (B * (K // 32) * 4 + 15) // 16 * 16
    grp = q.Group(probs, B=B)
    assert grp.plan.n_prologue == len(ks)
    grp.workspace.fill_(0xA5)
    grp()
    torch.cuda.synchronize()
    ws = grp.workspace.cpu().numpy()
    for i, ((qs, d, xq_o, xd_o), (xo, xdo, K), p) in enumerate(zip(refs, layout, probs)):
        xq = ws[xo:xo + B * K].view(np.int8).reshape(B, K)
        xd = ws[xdo:xdo + B * (K // 32) * 4].view(np.uint32).reshape(B, K // 32)
        assert np.array_equal(xq, xq_o), f"input {i} K={K}"
        assert np.array_equal(xd, xd_o.view(np.uint32)), f"input {i} K={K}"
        y_o, _ = oracle.mul_mat(qs, d, xq_o, xd_o, nthreads=16, want_y64=False)
        assert np.isfinite(p["y"].cpu().numpy()).all()
        assert_close(p["y"].cpu().numpy(), y_o, f"input {i} K={K}")


@pytest.mark.parametrize("B", [4, 8])
def test_group_eight_llama_8b_layers(B):
    """The Llama-3-8B decode step as the benchmark launches it: eight layers'
    56 products in one grouped call with fp32 rows (the layers share one set of
    weights; each has its own activation rows and outputs), so B = 8 takes the
    multi-column kernel with the windows of all eight layers packed into
    workgroup bins (products split over several records) and B = 4 the lane
    kernel.  Every output is written and finite and equals the single call on
    the same planes bit for bit; sampled rows of every product match the
    oracle."""
    print(f"[eight 8B layers] B={B}", flush=True)
    dev = torch.device("cuda:0")
    layer = workloads.LLAMA_3_8B
    weights = [_weights(5, 0, mi, m.M, m.K) for mi, m in enumerate(layer)]
    weights_d = [(to_dev(qs), to_dev(d.view(np.int16))) for qs, d in weights]
    problems, meta = [], []
    for l in range(8):
        xs = {s: workloads.activation(6, l, s, B, K) for s, K in workloads.slot_k(layer).items()}
        gs = {s: workloads.norm_weight(6, l, s, K) for s, K in workloads.slot_k(layer).items()}
        xs_d = {s: to_dev(v) for s, v in xs.items()}
        gs_d = {s: to_dev(v) for s, v in gs.items()}
        for mi, m in enumerate(layer):
            y = torch.full((B, m.M), float("nan"), dtype=torch.float32, device=dev)
            problems.append({"qs": weights_d[mi][0], "d": weights_d[mi][1], "y": y, "x": xs_d[m.slot],
                             "g": gs_d[m.slot], "eps": workloads.RMS_EPS})
            meta.append((l, mi, m, xs[m.slot], gs[m.slot]))
    grp = q.Group(problems, B=B)
    assert bool(grp.plan.mfma_columns) == (B == 8)
    if B == 8:
        assert grp.plan.n_records > len(problems)      # products split over several records
    grp()
    torch.cuda.synchronize()
    rng = np.random.default_rng(60 + B)
    for p, (l, mi, m, x, g) in zip(problems, meta):
        tag = f"B={B} layer {l} {m.name}"
        y = p["y"].cpu().numpy()
        assert np.isfinite(y).all(), tag
        xq, xd, _ = q.q8_quantize_rmsnorm(p["x"], p["g"], workloads.RMS_EPS)
        single = q.mul_mat_q4q8(p["qs"], p["d"], xq, xd)
        torch.cuda.synchronize()
        assert np.array_equal(single.cpu().numpy().view(np.uint32), y.view(np.uint32)), tag
        rows = np.unique(np.concatenate([[0, m.M - 1], rng.integers(0, m.M, 14)]))
        qs, d = weights[mi]
        xq_o, xd_o, _ = oracle.q8_quantize_rmsnorm(x, g, workloads.RMS_EPS)
        y_o, _ = oracle.mul_mat(qs[rows], d[rows], xq_o, xd_o, nthreads=16, want_y64=False)
        assert_close(y[:, rows], y_o, tag)


def test_group_multicolumn_in_hip_graph():
    """The packed multi-column route (B = 8) captured in a HIP graph: the
    prologue pass and the streaming launch over a group whose products are
    split over workgroup bins.  Replayed five times with eager work on the
    same buffers in between; every replay equals the eager launch bit for
    bit."""
    B = 8
    dev = torch.device("cuda:0")
    specs = [(4096, 4096, 0), (1024, 4096, 0), (2816, 2048, 1), (2048, 8192, 2), (1000, 1024, 3)]
    problems = []
    for i, (M, K, slot) in enumerate(specs):
        qs, d = _weights(50, 0, i, M, K)
        x = workloads.activation(50, 0, slot, B, K)
        g = workloads.norm_weight(50, 0, slot, K)
        y = torch.full((B, M), float("nan"), dtype=torch.float32, device=dev)
        problems.append({"qs": to_dev(qs), "d": to_dev(d.view(np.int16)), "y": y, "x": to_dev(x), "g": to_dev(g),
                         "eps": workloads.RMS_EPS})
    grp = q.Group(problems, B=B)
    assert grp.plan.mfma_columns == 1 and grp.plan.n_records > len(problems)
    grp()
    torch.cuda.synchronize()
    eager = [p["y"].clone() for p in problems]
    assert all(torch.isfinite(e).all() for e in eager)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        grp()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        grp()
    for rep in range(5):
        for p in problems:
            p["y"].fill_(float("nan"))
        grp.workspace.fill_(0x5A)          # eager work on the prologue planes between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for p, e in zip(problems, eager):
            assert torch.equal(p["y"].view(torch.int32), e.view(torch.int32)), f"replay {rep}"


def test_group_tiled_in_hip_graph():
    """The tiled route (B = 300: the 256-thread prologue pass, then one tiled
    MFMA launch) captured in a HIP graph and replayed three times with eager
    work on the same buffers in between; every replay equals the eager launch
    bit for bit."""
    B = 300
    dev = torch.device("cuda:0")
    specs = [(300, 4096), (130, 1408), (257, 2048)]
    problems = []
    for i, (M, K) in enumerate(specs):
        qs, d = _weights(51, 0, i, M, K)
        x = workloads.activation(51, 0, i, B, K)
        g = workloads.norm_weight(51, 0, i, K)
        y = torch.full((B, M), float("nan"), dtype=torch.float32, device=dev)
        problems.append({"qs": to_dev(qs), "d": to_dev(d.view(np.int16)), "y": y, "x": to_dev(x), "g": to_dev(g),
                         "eps": workloads.RMS_EPS})
    grp = q.Group(problems, B=B)
    grp()
    torch.cuda.synchronize()
    eager = [p["y"].clone() for p in problems]
    assert all(torch.isfinite(e).all() for e in eager)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        grp()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        grp()
    for rep in range(3):
        for p in problems:
            p["y"].fill_(float("nan"))
        grp.workspace.fill_(0x3C)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for p, e in zip(problems, eager):
            assert torch.equal(p["y"].view(torch.int32), e.view(torch.int32)), f"replay {rep}"
