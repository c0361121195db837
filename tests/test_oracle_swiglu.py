"""Pins of the oracle's SwiGLU -> Q8 producer and its fixed fp32 exponential.

Pinned against: the fp64 exponential (numpy, on the exact fp32 inputs) over a
dense sample of the algorithm's domain, exact values at 0 and at the domain's
ends, the fp64 silu formula, silu's closed forms (silu(+-0) = +-0, silu(g) = g
once exp(-g) < 2^-24, -0 once exp(-g) overflows the domain), the unfused chain
(silu, then numpy's IEEE fp32 multiply, then Q8) and the special case up = 1,
gate >= 17 that reduces to the plain Q8 quantiser.
"""
import numpy as np
import pytest

import oracle
import workloads


def _ulps(got, ref):
    ref32 = np.abs(ref).astype(np.float32)
    return np.abs(got.astype(np.float64) - ref) / np.spacing(ref32).astype(np.float64)


def test_exp_q_accuracy_over_the_domain():
    t = np.concatenate([np.linspace(-17, 88, 1_000_001, dtype=np.float32),
                        np.arange(-17, 89, dtype=np.float32)])
    err = _ulps(oracle.exp_q(t), np.exp(t.astype(np.float64)))
    assert err.max() <= 1.5


def test_exp_q_special_values():
    v = oracle.exp_q(np.array([0.0, -0.0, 88.0, 88.001, 1e30, -17.0, -17.001, -1e30, np.nan], np.float32))
    assert v[0] == 1.0 and v[1] == 1.0
    assert np.isfinite(v[2]) and v[3] == np.inf and v[4] == np.inf
    assert v[5] > 0 and v[6] == 0.0 and v[7] == 0.0 and np.isnan(v[8])


def test_silu_closed_forms_and_accuracy():
    s = oracle.silu(np.array([0.0, -0.0, 17.0, 20.5, 1e6, -88.01, -1e6], np.float32))
    assert s[0] == 0.0 and not np.signbit(s[0]) and s[1] == 0.0 and np.signbit(s[1])
    assert s[2] == np.float32(17.0) and s[3] == np.float32(20.5) and s[4] == np.float32(1e6)
    assert s[5] == 0.0 and np.signbit(s[5]) and s[6] == 0.0 and np.signbit(s[6])
    g = np.linspace(-30, 30, 200_001, dtype=np.float32)
    ref = g.astype(np.float64) / (1.0 + np.exp(-g.astype(np.float64)))
    keep = np.abs(ref) > 1e-30
    assert _ulps(oracle.silu(g)[keep], ref[keep]).max() <= 3.0


@pytest.mark.parametrize("F", [32, 1408, 14336])
def test_swiglu_q8_equals_unfused(F):
    gate = workloads.activation(7, 1, 0, 3, F)
    up = workloads.activation(7, 2, 0, 3, F)
    h = (oracle.silu(gate) * up).astype(np.float32)       # numpy fp32 multiply, one rounding
    for u, w in zip(oracle.q8_quantize_swiglu(gate, up), oracle.q8_quantize(h)):
        assert np.array_equal(u, w)


def test_swiglu_q8_reduces_to_q8_for_saturated_gates():
    g = np.random.default_rng(8)
    gate = g.uniform(17, 400, size=(2, 64)).astype(np.float32)
    for u, w in zip(oracle.q8_quantize_swiglu(gate, np.ones_like(gate)), oracle.q8_quantize(gate)):
        assert np.array_equal(u, w)
