"""The allocation-free routed entry point (mul_mat_id_q4q8_noalloc) against
mul_mat_id_q4q8 with a caller workspace: bit-identical outputs on two calls in
a row on the same device scratch, the second with a smaller input, both with
routings large enough to take the separate routing launch (the one that keeps
its results in the workspace) and a few invalid ids (NaN rows)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import to_dev

pytestmark = pytest.mark.gpu

q = pytest.importorskip("block_quantized_matmul_q8_amd")


def _case(seed, E, M, K, T, top_k, slots):
    w = workloads.weight(seed, 0, 0, E * M, K)
    qs, d = oracle.q4_quantize(w)
    x = workloads.activation(seed, 0, 1, T * slots, K)
    g = workloads.norm_weight(seed, 0, 1, K)
    xq, xd, _ = oracle.q8_quantize_rmsnorm(x, g, workloads.RMS_EPS)
    ids = workloads.expert_ids(seed, T, E, top_k)
    ids[0, 0] = E + 3          # invalid ids -> NaN rows
    ids[T - 1, top_k - 1] = -1
    return (to_dev(qs.reshape(E, M, K // 2)), to_dev(d.view(np.int16).reshape(E, M, K // 32)),
            to_dev(xq.reshape(T, slots, K)), to_dev(xd.reshape(T, slots, K // 32)), to_dev(ids))


def test_noalloc_equals_workspace_call_twice():
    dev = torch.device("cuda:0")
    # E = 512 experts, 64 tokens x top-8: 4107 routing ints, above the 4096 that
    # the streaming launch routes in LDS, so the routing lives in the scratch;
    # then a smaller call in the widest K band (separate routing launch too).
    for seed, E, M, K, T, top_k, slots in ((31, 512, 32, 2048, 64, 8, 8), (32, 48, 64, 16384, 8, 4, 1)):
        qs, d, xq, xd, ids = _case(seed, E, M, K, T, top_k, slots)
        y_ref = q.mul_mat_id_q4q8(qs, d, xq, xd, ids)
        y = torch.full((T, top_k, M), 7.0, dtype=torch.float32, device=dev)
        q.mul_mat_id_q4q8_noalloc(qs, d, xq, xd, ids, y)
        torch.cuda.synchronize(dev)
        a, b = y.cpu().numpy(), y_ref.cpu().numpy()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"E={E} K={K}: outputs differ"
        assert np.isnan(a[0, 0]).all() and np.isnan(a[T - 1, top_k - 1]).all()
        assert np.isfinite(a[1]).all()


def test_noalloc_rejects_bad_arguments():
    L = q.lib()
    import ctypes
    v = ctypes.c_void_p
    assert L.mul_mat_id_q4q8_noalloc(v(256), v(256), 0, 4, 64, v(256), v(256), 1, v(256), 1, 1, v(256),
                                     None) == q.Q4Q8_E_ARG
    assert "E = 0" in q.q4q8_last_error()
