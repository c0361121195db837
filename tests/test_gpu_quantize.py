"""GPU parity of the quantisation kernels against the oracle: bit-exact codes,
scales and code sums (Q4 weight planes; fused RMSNorm * g -> Q8 prologue)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import f16_bits, f32_bits, to_dev

pytestmark = pytest.mark.gpu

q = pytest.importorskip("block_quantized_matmul_q8_amd")


@pytest.mark.parametrize("M,K", [(1, 32), (3, 64), (256, 512), (129, 1408), (2048, 2048), (64, 14336)])
def test_q4_quantize_bit_exact(M, K):
    w = workloads.weight(11, M, K % 97, M, K)
    if M >= 3:
        w[1, :32] = 0.0                                   # all-zero block
        w[2, :32] = [-8 + (j % 16) for j in range(32)]    # hand example E1
        w[0, :32] = np.float32(1e-3) * w[0, :32]
    qs, d = q.q4_quantize(to_dev(w))
    qs_o, d_o = oracle.q4_quantize(w)
    assert np.array_equal(qs.cpu().numpy(), qs_o)
    assert np.array_equal(f16_bits(d), d_o)


def test_q4_quantize_hand_examples(hand_examples):
    rows = [np.array([-8 + (j % 16) for j in range(32)], np.float32),
            np.array(hand_examples["E2a"]["w"], np.float32),
            np.array(hand_examples["E2b"]["w"], np.float32),
            np.zeros(32, np.float32)]
    qs, d = q.q4_quantize(to_dev(np.stack(rows)))
    qs = qs.cpu().numpy()
    d = f16_bits(d)
    assert qs[0].tolist() == hand_examples["E1"]["qs"] and d[0, 0] == 0x3C00
    assert qs[1].tolist() == hand_examples["E2a"]["qs"] and d[1, 0] == 0x3C00
    assert qs[2].tolist() == hand_examples["E2b"]["qs"] and d[2, 0] == 0xBC00
    assert np.all(qs[3] == hand_examples["E3"]["q4_qs_byte"]) and d[3, 0] == 0


def test_e7_reciprocal_multiply_on_gpu(hand_examples):
    """E7: the GPU quantisers take id = fl(1 / d) and then fl(w * id), as the
    oracle does; a dividing kernel would give code 1 (Q4) and -127 (Q8, Q8_0)
    at j = 1.  The block sits among random blocks so that it is one block of a
    longer row (and of several rows) as well."""
    e7 = hand_examples["E7"]
    w = workloads.weight(14, 0, 0, 3, 96)
    w[0, 32:64] = e7["q4_w"]
    w[2, :32] = e7["q4_w"]
    qs, d = q.q4_quantize(to_dev(w))
    qs, d = qs.cpu().numpy(), f16_bits(d)
    assert qs[0, 16:32].tolist() == e7["q4_qs"] and qs[2, :16].tolist() == e7["q4_qs"]
    assert d[0, 1] == int(e7["q4_d_bits"], 16) and d[2, 0] == int(e7["q4_d_bits"], 16)
    qs_o, d_o = oracle.q4_quantize(w)
    assert np.array_equal(qs, qs_o) and np.array_equal(d, d_o)

    v = workloads.activation(14, 1, 0, 2, 96)
    v[1, 64:] = e7["q8_v"]
    xq, xd, xs = q.q8_quantize_rmsnorm(to_dev(v), None, 0.0, flags=q.Q8_NO_NORM, want_xs=True)
    xq, xd, xs = xq.cpu().numpy(), xd.cpu().numpy(), xs.cpu().numpy()
    assert xq[1, 64:].tolist() == e7["q8_codes"] and float(xd[1, 2]) == e7["q8_d"] and int(xs[1, 2]) == e7["q8_sum"]
    o = oracle.q8_quantize_rmsnorm(v, None, 0.0, no_norm=True)
    assert np.array_equal(xq, o[0]) and np.array_equal(xd.view(np.uint32), o[1].view(np.uint32))

    qw, dw = q.q8_0_quantize(to_dev(v))
    qw, dw = qw.cpu().numpy(), f16_bits(dw)
    assert qw[1, 64:].tolist() == e7["q8_codes"] and dw[1, 2] == int(e7["q8_0_d_bits"], 16)
    qw_o, dw_o = oracle.q8w_quantize(v)
    assert np.array_equal(qw, qw_o) and np.array_equal(dw, dw_o)


def test_e8_codes_from_fp32_scale_on_gpu(hand_examples):
    """E8: the Q4 and Q8_0 weight quantisers take their codes from the fp32
    scale and store fp16(d); codes from the fp16 scale would be 12 (Q4) and
    4 (Q8_0) at j = 1."""
    e8 = hand_examples["E8"]
    w = workloads.weight(15, 0, 0, 2, 64)
    w[1, 32:] = e8["q4_w"]
    qs, d = q.q4_quantize(to_dev(w))
    qs, d = qs.cpu().numpy(), f16_bits(d)
    assert qs[1, 16:].tolist() == e8["q4_qs"] and d[1, 1] == int(e8["q4_d_bits"], 16)
    w[1, 32:] = e8["q8_0_w"]
    qw, dw = q.q8_0_quantize(to_dev(w))
    qw, dw = qw.cpu().numpy(), f16_bits(dw)
    assert qw[1, 32:].tolist() == e8["q8_0_codes"] and dw[1, 1] == int(e8["q8_0_d_bits"], 16)


def test_q4_quantize_wide_range_and_subnormal_scales():
    """Scales that round to fp16 subnormals and to large fp16 values."""
    g = np.random.default_rng(5)
    w = g.standard_normal((8, 256), dtype=np.float32)
    w[0] *= np.float32(1e-6)
    w[1] *= np.float32(3e-5)
    w[2] *= np.float32(1e4)
    qs, d = q.q4_quantize(to_dev(w))
    qs_o, d_o = oracle.q4_quantize(w)
    assert np.array_equal(qs.cpu().numpy(), qs_o)
    assert np.array_equal(f16_bits(d), d_o)


@pytest.mark.parametrize("B,K", [(1, 32), (5, 512), (3, 1408), (4, 2048), (2, 8192), (3, 8224), (1, 14336),
                                 (2, 16384), (2, 16416), (2048, 4096), (16, 131072)])
def test_q8_rmsnorm_bit_exact(B, K):
    x = workloads.activation(12, B % 89, K % 83, B, K)
    gw = workloads.norm_weight(12, 0, K % 83, K)
    if B >= 3:
        x[1] = 0.0                    # all-zero row
        x[2, : K // 2] *= np.float32(1e-3)
    xq, xd, xs = q.q8_quantize_rmsnorm(to_dev(x), to_dev(gw), workloads.RMS_EPS, want_xs=True)
    xq_o, xd_o, xs_o = oracle.q8_quantize_rmsnorm(x, gw, workloads.RMS_EPS)
    assert np.array_equal(xq.cpu().numpy(), xq_o)
    assert np.array_equal(f32_bits(xd), xd_o.view(np.uint32))
    assert np.array_equal(xs.cpu().numpy(), xs_o)


def test_q8_rmsnorm_hand_examples(hand_examples):
    for key in ("E5", "E6"):
        ex = hand_examples[key]
        x = np.full((1, ex["K"]), ex["x"], np.float32)
        gw = np.full(ex["K"], ex["g"], np.float32)
        xq, xd, _ = q.q8_quantize_rmsnorm(to_dev(x), to_dev(gw), ex["eps"])
        assert int(f32_bits(xd)[0, 0]) == int(ex["xd_bits"], 16), key
        assert np.all(xq.cpu().numpy() == ex["code"]), key


def test_q8_no_norm_flag(hand_examples):
    e4 = hand_examples["E4"]
    v = np.array([e4["v"]], np.float32)
    xq, xd, xs = q.q8_quantize_rmsnorm(to_dev(v), None, 0.0, flags=q.Q8_NO_NORM, want_xs=True)
    assert xq.cpu().numpy()[0].tolist() == e4["codes"]
    assert float(xd.cpu().numpy()[0, 0]) == e4["d"] and int(xs.cpu().numpy()[0, 0]) == e4["sum"]
    x = workloads.activation(13, 0, 0, 7, 1408) * np.float32(3.0)
    xq, xd, xs = q.q8_quantize_rmsnorm(to_dev(x), None, 0.0, flags=q.Q8_NO_NORM, want_xs=True)
    o = oracle.q8_quantize_rmsnorm(x, None, 0.0, no_norm=True)
    assert np.array_equal(xq.cpu().numpy(), o[0])
    assert np.array_equal(f32_bits(xd), o[1].view(np.uint32))
    assert np.array_equal(xs.cpu().numpy(), o[2])


def test_prologue_empty_batch():
    import torch
    x = torch.empty((0, 64), dtype=torch.float32, device="cuda:0")
    g = torch.ones(64, dtype=torch.float32, device="cuda:0")
    xq, xd, _ = q.q8_quantize_rmsnorm(x, g, 1e-5)
    assert xq.shape == (0, 64) and xd.shape == (0, 2)


@pytest.mark.parametrize("B,K", [(1, 32), (3, 2048), (8, 4096), (2, 8224), (2, 16384), (2, 16416), (1, 131072)])
@pytest.mark.parametrize("per_row", [False, True])
def test_q8_rmsnorm_add_bit_exact(B, K, per_row):
    """RMS_NORM + MUL + ADD -> Q8: codes, scales and code sums equal the
    oracle bit for bit, for a shared [K] addend and one addend row per row,
    in both the register form (K <= 16384) and the LDS-tree form."""
    x = workloads.activation(50, 1, 0, B, K)
    g = workloads.norm_weight(50, 1, 0, K)
    a = workloads.activation(50, 2, 0, B, K)
    if not per_row:
        a = a[0].copy()
    xq, xd, xs = q.q8_quantize_rmsnorm_add(to_dev(x), to_dev(g), to_dev(a), workloads.RMS_EPS, want_xs=True)
    torch.cuda.synchronize()
    oq, od, os_ = oracle.q8_quantize_rmsnorm_add(x, g, a, workloads.RMS_EPS)
    assert np.array_equal(xq.cpu().numpy(), oq)
    assert np.array_equal(xd.cpu().numpy().view(np.uint32), od.view(np.uint32))
    assert np.array_equal(xs.cpu().numpy(), os_)


def _swiglu_inputs(seed, B, F):
    # gates spread over silu's whole range: both clamps of the exponential,
    # the saturated region and small values
    gate = (workloads.activation(seed, 3, 0, B, F) * np.float32(12.0)).astype(np.float32)
    gate[0, :8] = [0.0, -0.0, 17.0, -17.0, 88.0, -88.0, 200.0, -200.0]
    up = workloads.activation(seed, 4, 0, B, F)
    return gate, up


@pytest.mark.parametrize("B,F", [(1, 32), (8, 1408), (3, 2048), (1, 14336), (128, 1408)])
@pytest.mark.parametrize("stacked", [False, True])
def test_q8_swiglu_bit_exact(B, F, stacked):
    """SwiGLU -> Q8: codes, scales and code sums equal the oracle bit for bit,
    from separate gate / up planes and from one stacked [B][2F] buffer."""
    gate, up = _swiglu_inputs(60, B, F)
    if stacked:
        buf = to_dev(np.concatenate([gate, up], axis=1))
        g_dev, u_dev = buf[:, :F], buf[:, F:]
    else:
        g_dev, u_dev = to_dev(gate), to_dev(up)
    xq, xd, xs = q.q8_quantize_swiglu(g_dev, u_dev, want_xs=True)
    torch.cuda.synchronize()
    oq, od, os_ = oracle.q8_quantize_swiglu(gate, up)
    assert np.array_equal(xq.cpu().numpy(), oq)
    assert np.array_equal(xd.cpu().numpy().view(np.uint32), od.view(np.uint32))
    assert np.array_equal(xs.cpu().numpy(), os_)
