"""Pins of the oracle's fp16 conversions against numpy's IEEE binary16 casts.

The scale of every Q4 block is stored as fp16, so the oracle's hand-written
round-to-nearest-even conversion is checked exhaustively: every one of the
2^32 fp32 bit patterns (NaNs only checked to stay NaN) and every fp16 pattern.
"""
import numpy as np
import pytest

import oracle


def test_f16_to_f32_exhaustive():
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = oracle.f16_bits_to_f32(h)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


_STEP = 1 << 23  # one fp32 binade


def _check(u):
    f = u.view(np.float32)
    ours = oracle.f32_to_f16_bits(f)
    with np.errstate(over="ignore", invalid="ignore"):
        ref = f.astype(np.float16).view(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        o = ours[nan]
        assert np.all(((o & 0x7C00) == 0x7C00) & ((o & 0x03FF) != 0))
        ours, ref = ours[~nan], ref[~nan]
    assert np.array_equal(ours, ref)


@pytest.mark.parametrize("exp_lo,exp_hi", [(101, 112), (112, 123), (123, 134), (134, 144)])
def test_f32_to_f16_exhaustive_binades(exp_lo, exp_hi):
    """Every positive fp32 pattern whose binade can give a result other than
    0 or inf (exponent fields 101..143: values in [2^-26, 2^17))."""
    base = np.arange(_STEP, dtype=np.uint32)
    for e in range(exp_lo, exp_hi):
        _check(base + np.uint32(e << 23))


def test_f32_to_f16_random_full_space():
    """16M random patterns over all 2^32 (both signs, zeros, subnormals,
    underflow, overflow, inf, NaN), plus the binade edges."""
    g = np.random.default_rng(12345)
    u = g.integers(0, 1 << 32, size=1 << 24, dtype=np.uint64).astype(np.uint32)
    edges = np.array([0, 1, 0x7FFFFF, 0x800000, 0x7F7FFFFF, 0x7F800000, 0x7F800001, 0x7FC00000,
                      0xFFFFFFFF], dtype=np.uint32)
    u = np.concatenate([u, edges, edges | np.uint32(0x80000000)])
    _check(u)


def test_f16_round_trip_special_values():
    cases = [
        (0.0, 0x0000), (-0.0, 0x8000), (1.0, 0x3C00), (-1.0, 0xBC00), (65504.0, 0x7BFF),
        (65520.0, 0x7C00),              # halfway to the next binade rounds to inf
        (2.0 ** -24, 0x0001),           # smallest subnormal
        (2.0 ** -25, 0x0000),           # exact tie with zero -> even (zero)
        (3 * 2.0 ** -25, 0x0002),       # tie between 1 and 2 subnormal quanta -> even
        (2.0 ** -14, 0x0400),           # smallest normal
        (1.0 + 2.0 ** -11, 0x3C00),     # tie -> even
        (1.0 + 3 * 2.0 ** -11, 0x3C02),
    ]
    for v, bits in cases:
        got = oracle.f32_to_f16_bits(np.array([v], dtype=np.float32))[0]
        assert int(got) == bits, v
