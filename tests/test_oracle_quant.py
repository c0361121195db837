"""Pins of the oracle's Q4 / Q8 quantisers and the RMSNorm prologue.

Pinned against: the hand-derived examples in tests/golden/hand_examples.json
(E1-E8), closed-form round-trip error bounds derived from the block rule,
closed forms for constant rows, and an fp64 RMS normalisation within the
fp32 error bound of the fixed reduction order.
"""
import os

import numpy as np
import pytest

import oracle
import workloads

U = 2.0 ** -24  # fp32 unit roundoff


def _h(s):
    return int(s, 16)


# ----------------------------------------------------------------------------- Q4

def test_q4_hand_examples(hand_examples):
    e1 = hand_examples["E1"]
    w = np.array([[-8 + (j % 16) for j in range(32)]], dtype=np.float32)
    qs, d = oracle.q4_quantize(w)
    assert int(d[0, 0]) == _h(e1["d_bits"])
    assert qs[0].tolist() == e1["qs"]
    assert oracle.q4_unpack_codes(qs, 32)[0].tolist() == e1["codes"]
    for key in ("E2a", "E2b"):
        ex = hand_examples[key]
        w = np.array([ex["w"]], dtype=np.float32)
        qs, d = oracle.q4_quantize(w)
        assert int(d[0, 0]) == _h(ex["d_bits"]), key
        assert qs[0].tolist() == ex["qs"], key
        assert oracle.q4_unpack_codes(qs, 32)[0].tolist() == ex["codes"], key
        deq = oracle.dequantize_q4(qs, d, 32)[0, :8]
        assert deq.tolist() == ex["dequant_first8"], key


def test_q4_zero_block(hand_examples):
    e3 = hand_examples["E3"]
    w = np.zeros((3, 64), dtype=np.float32)
    w[1, 32:] = np.linspace(-1, 1, 32, dtype=np.float32)  # one non-zero block
    w[2, :32] = -0.0
    qs, d = oracle.q4_quantize(w)
    assert int(d[0, 0]) == int(d[0, 1]) == int(d[1, 0]) == int(d[2, 0]) == _h(e3["q4_d_bits"])
    assert np.all(qs[0] == e3["q4_qs_byte"]) and np.all(qs[1, :16] == e3["q4_qs_byte"])
    assert np.all(qs[2, :16] == e3["q4_qs_byte"])


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_q4_round_trip_bound(seed):
    """Closed-form bound.  With d the fp32 scale and d16 = fp16(d):
    unclamped codes satisfy |w - (q-8) d16| <= |d| (1/2 + 2^-8 + 2^-19);
    the clamped top code (q = 15) satisfies <= |d| (1 + 2^-8 + 2^-19)."""
    g = np.random.default_rng(seed)
    M, K = 64, 1024
    w = (g.standard_normal((M, K), dtype=np.float32) * np.float32(0.02))
    w[0, :32] *= np.float32(1e3)                        # wide dynamic range
    w[1, :32] = np.float32(0.0); w[1, 5] = np.float32(-3e-3)  # single spike
    qs, d = oracle.q4_quantize(w)
    q = oracle.q4_unpack_codes(qs, K).astype(np.int64)
    assert q.min() >= 0 and q.max() <= 15
    d16 = oracle.f16_bits_to_f32(d).astype(np.float64)
    dd = np.repeat(d16, 32, axis=1) / (1 - 2.0 ** -11)   # |d32| <= |d16| / (1 - 2^-11)
    err = np.abs(w.astype(np.float64) - (q - 8) * np.repeat(d16, 32, axis=1))
    lim_half = np.abs(dd) * (0.5 + 2.0 ** -8 + 2.0 ** -19)
    lim_one = np.abs(dd) * (1.0 + 2.0 ** -8 + 2.0 ** -19)
    assert np.all(err[q <= 14] <= lim_half[q <= 14])
    assert np.all(err <= lim_one)
    # the first extreme element of each block maps to code 0 (value -8 d)
    wb = w.reshape(M, -1, 32)
    first = np.argmax(np.abs(wb) == np.abs(wb).max(axis=2, keepdims=True), axis=2)
    qb = q.reshape(M, -1, 32)
    assert np.all(np.take_along_axis(qb, first[..., None], axis=2) == 0)


# ----------------------------------------------------------------------------- Q8

def test_q8_hand_example(hand_examples):
    e4 = hand_examples["E4"]
    v = np.array([e4["v"]], dtype=np.float32)
    xq, xd, xs = oracle.q8_quantize(v)
    assert xq[0].tolist() == e4["codes"]
    assert float(xd[0, 0]) == e4["d"]
    assert int(xs[0, 0]) == e4["sum"]
    # the no-norm flag of the fused entry takes the same path
    xq2, xd2, xs2 = oracle.q8_quantize_rmsnorm(v, None, 1e-5, no_norm=True)
    assert np.array_equal(xq, xq2) and np.array_equal(xd, xd2) and np.array_equal(xs, xs2)


def test_q8_zero_block(hand_examples):
    e3 = hand_examples["E3"]
    v = np.zeros((1, 64), dtype=np.float32)
    v[0, 40] = 1.0
    xq, xd, xs = oracle.q8_quantize(v)
    assert float(xd[0, 0]) == e3["q8_d"] and np.all(xq[0, :32] == e3["q8_code"]) and xs[0, 0] == 0
    assert xq[0, 40] == 127


@pytest.mark.parametrize("seed", [0, 1])
def test_q8_round_trip_bound(seed):
    """|v - q d| <= d (1/2 + 2^-16); codes in [-127, 127]; xs = sum of codes;
    the block maximum maps to +-127."""
    g = np.random.default_rng(seed)
    v = g.standard_normal((16, 2048), dtype=np.float32)
    v[0] *= np.float32(1e-30)
    v[1] *= np.float32(1e20)
    xq, xd, xs = oracle.q8_quantize(v)
    dd = np.repeat(xd.astype(np.float64), 32, axis=1)
    err = np.abs(v.astype(np.float64) - xq.astype(np.float64) * dd)
    assert np.all(err <= dd * (0.5 + 2.0 ** -16))
    assert np.abs(xq.astype(np.int64)).max() <= 127
    assert np.array_equal(xs, xq.reshape(16, -1, 32).astype(np.int32).sum(axis=2))
    vb = np.abs(v.reshape(16, -1, 32))
    amax_idx = np.argmax(vb, axis=2)
    qb = np.abs(xq.reshape(16, -1, 32).astype(np.int64))
    assert np.all(np.take_along_axis(qb, amax_idx[..., None], axis=2) == 127)


# ----------------------------------------------------------------------------- RMSNorm

def test_rmsnorm_hand_examples(hand_examples):
    for key in ("E5", "E6"):
        ex = hand_examples[key]
        x = np.full((1, ex["K"]), ex["x"], dtype=np.float32)
        g = np.full(ex["K"], ex["g"], dtype=np.float32)
        _, s = oracle.rmsnorm(x, ex["eps"])
        assert int(s.view(np.uint32)[0]) == _h(ex["s_bits"]), key
        xq, xd, xs = oracle.q8_quantize_rmsnorm(x, g, ex["eps"])
        assert int(xd.view(np.uint32)[0, 0]) == _h(ex["xd_bits"]), key
        assert np.all(xq == ex["code"]), key
    assert int(oracle.q8_quantize_rmsnorm(np.ones((1, 32), np.float32), np.ones(32, np.float32),
                                          1e-5)[2][0, 0]) == hand_examples["E5"]["code_sum"]


@pytest.mark.parametrize("c", [0.25, 1.0, 3.0, -7.5, 1e-3])
@pytest.mark.parametrize("K", [32, 96, 2048, 1408])
def test_rmsnorm_constant_row_closed_form(c, K):
    """A constant row c has s = 1/sqrt(c^2 + eps) exactly in real arithmetic;
    the fp32 chain (exact squares of a constant with a power-of-two count are
    not guaranteed, so allow the fp32 bound of the fixed reduction)."""
    eps = 1e-5
    x = np.full((1, K), c, dtype=np.float32)
    _, s = oracle.rmsnorm(x, eps)
    exact = 1.0 / np.sqrt(np.float64(np.float32(c)) ** 2 + np.float64(np.float32(eps)))
    nb = K // 32
    n_ops = 32 + int(np.ceil(np.log2(nb))) + 4
    assert abs(float(s[0]) - exact) <= n_ops * U * exact


@pytest.mark.parametrize("K", [32, 512, 1408, 2048, 4096, 14336])
def test_rmsnorm_vs_fp64(K):
    """Random rows: the fp32 scale lies within the forward error bound of its
    reduction (32 sequential adds + ceil(log2 nb) tree levels + 4 ops) of the
    fp64 value."""
    eps = 1e-5
    x = workloads.activation(0, 0, 0, 8, K)
    x[1] *= np.float32(1e-3)
    x[2] *= np.float32(30.0)
    _, s = oracle.rmsnorm(x, eps)
    x64 = x.astype(np.float64)
    s64 = 1.0 / np.sqrt((x64 * x64).mean(axis=1) + np.float64(np.float32(eps)))
    nb = K // 32
    n_ops = 32 + int(np.ceil(np.log2(nb))) + 4
    assert np.all(np.abs(s.astype(np.float64) - s64) <= n_ops * U * s64)


def test_reduction_order_is_the_stated_tree():
    """The result depends on the stated order: check a row crafted so that the
    block-tree sum differs from a plain left-to-right fp32 sum."""
    K = 128  # nb = 4: tree ((p0 + p1) + (p2 + p3))
    x = np.zeros((1, K), dtype=np.float32)
    x[0, 0] = np.float32(4096.0)          # p0 = 2^24, p1 = 0
    x[0, 64] = np.float32(1.0)            # p2 = 1
    x[0, 96] = np.float32(1.0)            # p3 = 1
    _, s = oracle.rmsnorm(x, 0.0)
    # tree: (2^24 + 0) + (1 + 1) = 2^24 + 2 (exact); a left-to-right sum would
    # give ((2^24 + 1) -> 2^24) + 1 -> 2^24 (ties to even) instead.
    ssq_tree = np.float32(2.0 ** 24 + 2.0)
    mean = np.float32(ssq_tree / np.float32(K))
    expect = np.float32(1.0) / np.sqrt(mean)
    ssq_seq = np.float32(2.0 ** 24)
    other = np.float32(1.0) / np.sqrt(np.float32(ssq_seq / np.float32(K)))
    assert expect != other
    assert s[0] == expect


@pytest.mark.parametrize("K", [64, 1408, 4096])
def test_fused_equals_unfused(K):
    """q8_quantize_rmsnorm == rmsnorm -> multiply by g -> q8_quantize, bit for bit
    (the fusion of RMS_NORM+MUL must not change the result)."""
    x = workloads.activation(0, 1, 0, 5, K)
    g = workloads.norm_weight(0, 1, 0, K)
    t, _ = oracle.rmsnorm(x, 1e-5)
    v = oracle.mul_rows(t, g)
    a = oracle.q8_quantize(v)
    b = oracle.q8_quantize_rmsnorm(x, g, 1e-5)
    for u, w in zip(a, b):
        assert np.array_equal(u, w)


def test_golden_rmsnorm_examples_rederived_exactly(hand_examples):
    """The stored E5 / E6 values follow from the stated fp32 steps carried out
    on exact rationals (tests/golden/derive_hand_examples.py), independently
    of the oracle."""
    import importlib.util
    path = os.path.join(os.path.dirname(__file__), "golden", "derive_hand_examples.py")
    spec = importlib.util.spec_from_file_location("derive_hand_examples", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    for name, xv in (("E5", 1), ("E6", 2)):
        r = mod.constant_row(xv)
        assert mod.bits(r["s"]) == hand_examples[name]["s_bits"]
        assert mod.bits(r["d"]) == hand_examples[name]["xd_bits"]
        assert r["v_times_id"] == hand_examples[name]["code"]
    assert mod.bits(mod.e5_y(mod.constant_row(1)["d"], hand_examples["E5"]["I"])) == hand_examples["E5"]["y_bits"]


def _derive_module():
    import importlib.util
    path = os.path.join(os.path.dirname(__file__), "golden", "derive_hand_examples.py")
    spec = importlib.util.spec_from_file_location("derive_hand_examples", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_golden_e7_rederived_exactly(hand_examples):
    """E7's stored codes follow from the reciprocal-multiply rule on exact
    rationals, and a plain division gives the other stored codes: the block
    really separates the two readings."""
    mod = _derive_module()
    e7 = hand_examples["E7"]
    r = mod.e7_blocks()
    assert float(r["q4"]["d"]) == 7.0 and float(r["q8"]["d"]) == e7["q8_d"]
    assert r["q4"]["codes"] == e7["q4_codes"] and r["q4"]["codes_if_divided"] == e7["q4_codes_if_divided"]
    assert r["q8"]["codes"] == e7["q8_codes"] and r["q8"]["codes_if_divided"] == e7["q8_codes_if_divided"]
    assert e7["q4_codes"] != e7["q4_codes_if_divided"] and e7["q8_codes"] != e7["q8_codes_if_divided"]


def test_e7_reciprocal_multiply_not_divide(hand_examples):
    """The block rules take id = fl(1 / d) and then fl(w * id), not fl(w / d):
    Q4, Q8 (through the no-norm flag) and Q8_0 codes of E7 equal the
    reciprocal-multiply codes (a dividing oracle fails here)."""
    e7 = hand_examples["E7"]
    qs, d = oracle.q4_quantize(np.array([e7["q4_w"]], dtype=np.float32))
    assert int(d[0, 0]) == _h(e7["q4_d_bits"])
    assert qs[0].tolist() == e7["q4_qs"]
    assert oracle.q4_unpack_codes(qs, 32)[0].tolist() == e7["q4_codes"]
    v = np.array([e7["q8_v"]], dtype=np.float32)
    for xq, xd, xs in (oracle.q8_quantize(v), oracle.q8_quantize_rmsnorm(v, None, 1e-5, no_norm=True)):
        assert xq[0].tolist() == e7["q8_codes"] and float(xd[0, 0]) == e7["q8_d"] and int(xs[0, 0]) == e7["q8_sum"]
    qw, dw = oracle.q8w_quantize(v)
    assert qw[0].tolist() == e7["q8_codes"] and int(dw[0, 0]) == _h(e7["q8_0_d_bits"])


def test_golden_e8_rederived_exactly(hand_examples):
    """E8's stored codes follow from the fp32 scale on exact rationals, and
    codes from the stored fp16 scale would be the other stored codes."""
    mod = _derive_module()
    e8 = hand_examples["E8"]
    r = mod.e8_blocks()
    for name, key_w in (("q4", "q4"), ("q8_0", "q8_0")):
        assert r[name]["codes"] == e8[f"{key_w}_codes"], name
        assert r[name]["codes_if_from_f16"] == e8[f"{key_w}_codes_if_from_f16"], name
        assert e8[f"{key_w}_codes"] != e8[f"{key_w}_codes_if_from_f16"], name
        assert mod.bits(r[name]["d"]) == "0x3dcccccd"
        assert float(r[name]["d16"]) == float(np.uint16(int(e8[f"{key_w}_d_bits"], 16)).view(np.float16))


def test_e8_codes_from_fp32_scale(hand_examples):
    """The Q4 and Q8_0 weight rules take their codes from the fp32 scale and
    store fp16(d) beside them (an oracle that quantised with the stored fp16
    scale fails here)."""
    e8 = hand_examples["E8"]
    qs, d = oracle.q4_quantize(np.array([e8["q4_w"]], dtype=np.float32))
    assert int(d[0, 0]) == _h(e8["q4_d_bits"]) and qs[0].tolist() == e8["q4_qs"]
    assert oracle.q4_unpack_codes(qs, 32)[0].tolist() == e8["q4_codes"]
    qw, dw = oracle.q8w_quantize(np.array([e8["q8_0_w"]], dtype=np.float32))
    assert qw[0].tolist() == e8["q8_0_codes"] and int(dw[0, 0]) == _h(e8["q8_0_d_bits"])


def test_block_partial_sums_are_sequential():
    """Within a block the squares are summed left to right in fp32: for
    x = [4096, 1, 1, 1, 0 x 28] the sequential sum is 2^24 (each + 1 ties to
    even), where a pairwise order would give 2^24 + 2; s follows in closed
    form from ssq = 2^24 with numpy's correctly rounded fp32 ops."""
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, :4] = [4096.0, 1.0, 1.0, 1.0]
    _, s = oracle.rmsnorm(x, 0.0)
    mean = np.float32(np.float32(2.0 ** 24) / np.float32(32.0))
    expect = np.float32(1.0) / np.sqrt(mean)
    other = np.float32(1.0) / np.sqrt(np.float32(np.float32(2.0 ** 24 + 2.0) / np.float32(32.0)))
    assert expect != other
    assert s[0] == expect


# --- RMS_NORM + MUL + ADD -> Q8 ---------------------------------------------

@pytest.mark.parametrize("K", [32, 1408, 4096])
def test_norm_add_zero_addend_is_rmsnorm(K):
    """A zero addend leaves RMS_NORM+MUL -> Q8 unchanged, bit for bit."""
    x = workloads.activation(4, 1, 0, 3, K)
    g = workloads.norm_weight(4, 1, 0, K)
    a = np.zeros(K, dtype=np.float32)
    for u, w in zip(oracle.q8_quantize_rmsnorm_add(x, g, a, 1e-5), oracle.q8_quantize_rmsnorm(x, g, 1e-5)):
        assert np.array_equal(u, w)


@pytest.mark.parametrize("K", [64, 2048])
def test_norm_add_equals_unfused(K):
    """Fused RMS_NORM+MUL+ADD == rmsnorm -> multiply by g -> an fp32 add (numpy's
    IEEE single add) -> q8_quantize, bit for bit, for one addend per row and one
    shared addend."""
    x = workloads.activation(5, 1, 0, 4, K)
    g = workloads.norm_weight(5, 1, 0, K)
    a_rows = workloads.activation(5, 2, 0, 4, K)
    t, _ = oracle.rmsnorm(x, 1e-5)
    v = oracle.mul_rows(t, g)
    for a in (a_rows, a_rows[1]):
        ref = oracle.q8_quantize((v + a).astype(np.float32))
        got = oracle.q8_quantize_rmsnorm_add(x, g, a, 1e-5)
        for u, w in zip(got, ref):
            assert np.array_equal(u, w)


def test_norm_add_hand_example(hand_examples):
    """E5 (K = 32, x = 1, g = 1, eps = 1e-5: s = 1 - 84 * 2^-24) with the
    addend -s on the first 16 elements and 0.25 on the last 16.  The ADD comes
    after the norm and the MUL: the first half cancels exactly to 0, the second
    half is s + 0.25 = 1.25 - 42 * 2^-23 (exact).  So codes are 0 and 127, and
    d = fl(v / 127).  Adding before the norm would give entirely different
    codes."""
    e5 = hand_examples["E5"]
    s = np.uint32(int(e5["s_bits"], 16)).view(np.float32)
    a = np.concatenate([np.full(16, -s, dtype=np.float32), np.full(16, 0.25, dtype=np.float32)])
    xq, xd, xs = oracle.q8_quantize_rmsnorm_add(np.ones((1, 32), np.float32), np.ones(32, np.float32), a, 1e-5)
    v = np.float32(1.25 - 42 * 2.0 ** -23)
    assert np.float32(s) + np.float32(0.25) == v                  # the sum is exact
    assert xq[0, :16].tolist() == [0] * 16 and xq[0, 16:].tolist() == [127] * 16
    assert xd[0, 0] == np.float32(v) / np.float32(127.0) and xs[0, 0] == 16 * 127


def test_norm_add_shared_addend_equals_repeated_rows():
    K, B = 512, 3
    x = workloads.activation(6, 1, 0, B, K)
    g = workloads.norm_weight(6, 1, 0, K)
    a = workloads.activation(6, 2, 0, 1, K)[0]
    for u, w in zip(oracle.q8_quantize_rmsnorm_add(x, g, a, 1e-5),
                    oracle.q8_quantize_rmsnorm_add(x, g, np.tile(a, (B, 1)), 1e-5)):
        assert np.array_equal(u, w)
