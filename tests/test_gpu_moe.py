"""GPU parity of mul_mat_id_q4q8 (expert-routed product) against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import assert_close, to_dev

pytestmark = pytest.mark.gpu

q = pytest.importorskip("block_quantized_matmul_q8_amd")


def _experts(seed, E, M, K):
    w = np.stack([workloads.weight(seed, 0, e, M, K) for e in range(E)])
    qs, d = oracle.q4_quantize(w.reshape(E * M, K))
    return w, qs.reshape(E, M, K // 2), d.reshape(E, M, K // 32)


def _acts(seed, T, S, K):
    x = workloads.activation(seed, 1, S, T * S, K)
    g = workloads.norm_weight(seed, 1, S, K)
    xq, xd, _ = oracle.q8_quantize_rmsnorm(x, g, workloads.RMS_EPS)
    return xq.reshape(T, S, K), xd.reshape(T, S, K // 32)


def _gpu(qs, d, xq, xd, ids):
    y = q.mul_mat_id_q4q8(to_dev(qs), to_dev(d.view(np.int16)), to_dev(xq), to_dev(xd), to_dev(ids))
    torch.cuda.synchronize()
    return y.cpu().numpy()


def _check_rows(y, y_o, ids, E):
    for t in range(ids.shape[0]):
        for s in range(ids.shape[1]):
            if 0 <= ids[t, s] < E:
                assert_close(y[t, s], y_o[t, s], f"t={t} s={s}")
            else:
                assert np.all(np.isnan(y[t, s]))


@pytest.mark.parametrize("mode", ["broadcast", "per_slot"])
@pytest.mark.parametrize("E,M,K,T,top_k", [(6, 40, 1408, 5, 3), (9, 130, 512, 11, 4), (3, 7, 32, 2, 2)])
def test_small(mode, E, M, K, T, top_k):
    S = 1 if mode == "broadcast" else top_k
    _, qs, d = _experts(31, E, M, K)
    xq, xd = _acts(31, T, S, K)
    ids = workloads.expert_ids(31, T, E, top_k)
    y = _gpu(qs, d, xq, xd, ids)
    y_o = oracle.mul_mat_id(qs, d, xq, xd, ids, nthreads=8)
    _check_rows(y, y_o, ids, E)


def test_bad_ids_give_nan_rows():
    E, M, K, T, top_k = 4, 24, 256, 6, 2
    _, qs, d = _experts(32, E, M, K)
    xq, xd = _acts(32, T, 1, K)
    ids = workloads.expert_ids(32, T, E, top_k)
    ids[0, 1] = E
    ids[3, 0] = -7
    ids[5, 1] = 1 << 30
    y = _gpu(qs, d, xq, xd, ids)
    y_o = oracle.mul_mat_id(qs, d, xq, xd, ids)
    _check_rows(y, y_o, ids, E)


@pytest.mark.parametrize("E", [40, 900])
def test_routing_in_launch_and_separate(E):
    """Small routings run inside every workgroup of the streaming launch;
    larger ones (here 900 experts) take the separate routing launch.  Both,
    on ids that select the same experts (plus invalid ids), against the
    oracle."""
    M, K, T, top_k = 70, 512, 9, 4
    _, qs40, d40 = _experts(37, 40, M, K)
    qs = np.zeros((E, M, K // 2), np.uint8)
    d = np.zeros((E, M, K // 32), np.uint16)
    qs[:40], d[:40] = qs40, d40
    xq, xd = _acts(37, T, top_k, K)
    ids = workloads.expert_ids(37, T, 40, top_k)
    ids[2, 1] = E
    ids[6, 3] = -1
    y = _gpu(qs, d, xq, xd, ids)
    y_o = oracle.mul_mat_id(qs, d, xq, xd, ids, nthreads=8)
    _check_rows(y, y_o, ids, E)


def test_single_expert_reduces_to_mul_mat():
    E, M, K, T = 1, 96, 1408, 7
    _, qs, d = _experts(33, E, M, K)
    xq, xd = _acts(33, T, 1, K)
    ids = np.zeros((T, 1), np.int32)
    y = _gpu(qs, d, xq, xd, ids)
    y_mm = q.mul_mat_q4q8(to_dev(qs[0]), to_dev(d[0].view(np.int16)), to_dev(xq[:, 0]), to_dev(xd[:, 0]))
    torch.cuda.synchronize()
    y_o, _ = oracle.mul_mat(qs[0], d[0], xq[:, 0], xd[:, 0])
    assert_close(y[:, 0], y_o)
    assert_close(y_mm.cpu().numpy(), y_o)


def test_full_moe_decode():
    """The MoE decode workload at full shape: 64 experts, gate/up 1408 x 2048
    fed by each token's row (shared by its 8 slots), down 2048 x 1408 fed by one
    row per (token, slot); 16 tokens, top-8 ids uniform without replacement."""
    cfg = workloads.MOE
    ids = workloads.expert_ids(0, cfg.T, cfg.E, cfg.top_k)
    for name, M, K, S in (("gate", cfg.ffn, cfg.hidden, 1), ("up", cfg.ffn, cfg.hidden, 1),
                          ("down", cfg.hidden, cfg.ffn, cfg.top_k)):
        _, qs, d = _experts(0 if name != "up" else 1, cfg.E, M, K)
        xq, xd = _acts(0, cfg.T, S, K)
        y = _gpu(qs, d, xq, xd, ids)
        y_o = oracle.mul_mat_id(qs, d, xq, xd, ids, nthreads=16)
        assert_close(y, y_o, name)


@pytest.mark.parametrize("E,M,K,T,top_k,S", [
    (2, 70, 512, 20, 1, 1),        # ~10 pairs per expert: two passes of up to 8 pairs
    (3, 33, 4096, 9, 2, 2),        # K band 4096, one row per (token, slot)
    (4, 20, 8224, 6, 3, 1),        # K band 16384 (split over waves), ragged block count
    (5, 48, 7168, 13, 5, 5),       # K band 8192
])
def test_expert_loads_and_k_bands(E, M, K, T, top_k, S):
    _, qs, d = _experts(34, E, M, K)
    xq, xd = _acts(34, T, S, K)
    ids = workloads.expert_ids(34, T, E, top_k)
    y = _gpu(qs, d, xq, xd, ids)
    y_o = oracle.mul_mat_id(qs, d, xq, xd, ids, nthreads=8)
    _check_rows(y, y_o, ids, E)


@pytest.mark.parametrize("mode", ["broadcast", "per_slot"])
@pytest.mark.parametrize("K", [1408, 1440, 1536, 1024, 96])
def test_short_rows_every_width(mode, K):
    """Rows of at most 48 blocks (K <= 1536) take 16 lanes per row and 3
    blocks per lane, in passes of at most four routed pairs: experts with 1,
    2, 3 and 6 pairs (widths 1, 2, 4, then 4 + 2), 77 rows (a partial last
    window), block counts below and at 48."""
    E, M, T, top_k = 4, 77, 6, 2
    S = 1 if mode == "broadcast" else top_k
    _, qs, d = _experts(38, E, M, K)
    xq, xd = _acts(38, T, S, K)
    ids = np.array([[3, 2], [3, 2], [3, 2], [3, 1], [3, 1], [3, 0]], np.int32)
    y = _gpu(qs, d, xq, xd, ids)
    y_o = oracle.mul_mat_id(qs, d, xq, xd, ids, nthreads=8)
    _check_rows(y, y_o, ids, E)


def test_many_bad_ids():
    """Half of the pairs carry ids outside [0, E): their rows are NaN, the
    others are computed as usual."""
    E, M, K, T, top_k = 5, 40, 1408, 12, 4
    _, qs, d = _experts(35, E, M, K)
    xq, xd = _acts(35, T, 1, K)
    ids = workloads.expert_ids(35, T, E, top_k)
    ids[::2, :] = -1
    ids[1, 3] = E + 3
    y = _gpu(qs, d, xq, xd, ids)
    y_o = oracle.mul_mat_id(qs, d, xq, xd, ids, nthreads=8)
    _check_rows(y, y_o, ids, E)


def test_full_moe_stacked_gate_up():
    """The benchmark's routed call as it is timed: gate and up of all 64
    experts stacked into one [E][2 * 1408][2048] tensor, 16 tokens, top-8."""
    cfg = workloads.MOE
    ids = workloads.expert_ids(0, cfg.T, cfg.E, cfg.top_k)
    _, qs, d = _experts(2, cfg.E, 2 * cfg.ffn, cfg.hidden)
    xq, xd = _acts(2, cfg.T, 1, cfg.hidden)
    y = _gpu(qs, d, xq, xd, ids)
    y_o = oracle.mul_mat_id(qs, d, xq, xd, ids, nthreads=16)
    assert_close(y, y_o, "stacked gate/up")


def _sum_gpu(y, w):
    out = q.moe_expert_sum_f32(to_dev(y), None if w is None else to_dev(w))
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("T,top_k,M", [(16, 8, 2048), (3, 1, 5), (7, 5, 300), (1, 64, 257), (2, 3, 70000)])
def test_expert_sum_bit_exact(T, top_k, M):
    g = np.random.default_rng(40 + top_k)
    y = (g.standard_normal((T, top_k, M)) * np.exp(g.uniform(-20, 20, size=(T, top_k, 1)))).astype(np.float32)
    y[0, 0, :3] = [0.0, -0.0, 1e-45]
    w = workloads.expert_weights(40, T, top_k)
    for wv in (w, None):
        out = _sum_gpu(y, wv)
        ref = oracle.moe_expert_sum(y, wv)
        assert np.array_equal(out.view(np.uint32), ref.view(np.uint32))


def test_expert_sum_of_routed_down_projection():
    """The MoE down projection as the benchmark runs it (64 experts of
    2048 x 1408, 16 tokens, top-8, one row per (token, slot)), followed by
    the weighted expert-plane sum; a bad id makes its token's sum NaN."""
    cfg = workloads.MOE
    ids = workloads.expert_ids(0, cfg.T, cfg.E, cfg.top_k)
    ids[5, 2] = cfg.E
    _, qs, d = _experts(3, cfg.E, cfg.hidden, cfg.ffn)
    xq, xd = _acts(3, cfg.T, cfg.top_k, cfg.ffn)
    w = workloads.expert_weights(0, cfg.T, cfg.top_k)
    y = q.mul_mat_id_q4q8(to_dev(qs), to_dev(d.view(np.int16)), to_dev(xq), to_dev(xd), to_dev(ids))
    out = q.moe_expert_sum_f32(y, to_dev(w))
    torch.cuda.synchronize()
    y, out = y.cpu().numpy(), out.cpu().numpy()
    # bit-exact against the chain over the GPU's own planes
    assert np.array_equal(out.view(np.uint32), oracle.moe_expert_sum(y, w).view(np.uint32))
    # and within tolerance of the oracle end to end (rows without the bad id)
    y_o = oracle.mul_mat_id(qs, d, xq, xd, ids, nthreads=16)
    out_o = oracle.moe_expert_sum(y_o, w)
    assert np.all(np.isnan(out[5])) and np.all(np.isnan(out_o[5]))
    keep = [t for t in range(cfg.T) if t != 5]
    assert_close(out[keep], out_o[keep], "expert sum of the down projection")


def test_moe_chain_gate_up_swiglu_down_sum():
    """A whole routed FFN on the MoE shape: stacked gate/up routed product ->
    SwiGLU -> Q8 of every (token, slot) row -> routed down product -> weighted
    expert sum.  Each GPU stage is checked against the oracle stage applied to
    the GPU's own input (codes bit-exact, fp32 outputs within tolerance), and
    the end result against the oracle chain."""
    cfg = workloads.MOE
    ids = workloads.expert_ids(1, cfg.T, cfg.E, cfg.top_k)
    w = workloads.expert_weights(1, cfg.T, cfg.top_k)
    _, qs_gu, d_gu = _experts(4, cfg.E, 2 * cfg.ffn, cfg.hidden)
    _, qs_dn, d_dn = _experts(5, cfg.E, cfg.hidden, cfg.ffn)
    xq, xd = _acts(4, cfg.T, 1, cfg.hidden)
    y_gu = q.mul_mat_id_q4q8(to_dev(qs_gu), to_dev(d_gu.view(np.int16)), to_dev(xq), to_dev(xd), to_dev(ids))
    rows = y_gu.view(cfg.T * cfg.top_k, 2 * cfg.ffn)
    hq, hd, _ = q.q8_quantize_swiglu(rows[:, :cfg.ffn], rows[:, cfg.ffn:])
    y_dn = q.mul_mat_id_q4q8(to_dev(qs_dn), to_dev(d_dn.view(np.int16)), hq.view(cfg.T, cfg.top_k, cfg.ffn),
                             hd.view(cfg.T, cfg.top_k, cfg.ffn // 32), to_dev(ids))
    out = q.moe_expert_sum_f32(y_dn, to_dev(w))
    torch.cuda.synchronize()
    y_gu_h = y_gu.cpu().numpy()
    # SwiGLU codes bit-exact on the GPU's own gate/up planes
    g_h = y_gu_h[:, :, :cfg.ffn].reshape(-1, cfg.ffn).copy()
    u_h = y_gu_h[:, :, cfg.ffn:].reshape(-1, cfg.ffn).copy()
    oq, od, _ = oracle.q8_quantize_swiglu(g_h, u_h)
    assert np.array_equal(hq.cpu().numpy(), oq) and np.array_equal(hd.cpu().numpy(), od)
    # the end-to-end chain against the oracle chain
    y_gu_o = oracle.mul_mat_id(qs_gu, d_gu, xq, xd, ids, nthreads=16)
    assert_close(y_gu_h, y_gu_o, "gate/up")
    g_o = y_gu_o[:, :, :cfg.ffn].reshape(-1, cfg.ffn).copy()
    u_o = y_gu_o[:, :, cfg.ffn:].reshape(-1, cfg.ffn).copy()
    hq_o, hd_o, _ = oracle.q8_quantize_swiglu(g_o, u_o)
    y_dn_o = oracle.mul_mat_id(qs_dn, d_dn, hq_o.reshape(cfg.T, cfg.top_k, cfg.ffn),
                               hd_o.reshape(cfg.T, cfg.top_k, cfg.ffn // 32), ids, nthreads=16)
    out_o = oracle.moe_expert_sum(y_dn_o, w)
    # the GPU's gate/up differ from the oracle's by fp32 summation order, which
    # can move a Q8 code by one step; the end result is compared normwise with
    # the quantisation-level tolerance of one extra Q8 rounding (2^-8 relative)
    err = np.abs(out.cpu().numpy().astype(np.float64) - out_o).max() / np.abs(out_o).max()
    assert err < 2e-3, err


@pytest.mark.parametrize("E", [64, 900])
def test_routed_call_in_hip_graph(E):
    """A routed call captured in a HIP graph (routing inside the streaming
    launch for 64 experts, its own launch for 900) and replayed three times,
    the workspace overwritten with garbage between replays: every replay
    equals the eager call bit for bit, so the routing keeps nothing from an
    earlier call."""
    M, K, T, top_k = 96, 1408, 16, 8
    _, qs40, d40 = _experts(39, 40, M, K)
    qs = np.zeros((E, M, K // 2), np.uint8)
    d = np.zeros((E, M, K // 32), np.uint16)
    qs[:40], d[:40] = qs40, d40
    xq, xd = _acts(39, T, top_k, K)
    ids = workloads.expert_ids(39, T, 40, top_k)
    ids[3, 2] = E                                   # one invalid id: a NaN row
    args = [to_dev(qs), to_dev(d.view(np.int16)), to_dev(xq), to_dev(xd), to_dev(ids)]
    ws = torch.empty(q.mul_mat_id_q4q8_workspace(E, T, top_k), dtype=torch.uint8, device="cuda:0")
    y = torch.empty((T, top_k, M), dtype=torch.float32, device="cuda:0")
    q.mul_mat_id_q4q8(*args, y=y, ws=ws)
    torch.cuda.synchronize()
    eager = y.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        q.mul_mat_id_q4q8(*args, y=y, ws=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        q.mul_mat_id_q4q8(*args, y=y, ws=ws)
    for rep in range(3):
        y.fill_(-1.0)
        ws.fill_(0xC3)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), eager.view(torch.int32)), f"replay {rep}"
    y_o = oracle.mul_mat_id(qs, d, xq, xd, ids, nthreads=8)
    _check_rows(eager.cpu().numpy(), y_o, ids, E)
