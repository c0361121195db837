"""The Q8 coders on the GPU round with fl(t + copysign(0.5 - 2^-25, t))
truncated instead of roundf(t) (halves away from zero, the rule the oracle
applies).  This pins the identity on the CPU with numpy's float32 addition
(round to nearest even, as the GPU's): every float in [1/8, 4) and a
sample of the smaller ones, every float
within 2^12 ulps of each half-integer and integer up to 256 (the codes' range
and its neighbourhood), both signs, and the binades where the spacing reaches
1/2 and 1.  (An exhaustive run over all floats in [0, 2^24], 1.27e9 values,
found no mismatch either; it takes about a minute, too long for this suite.)
The GPU kernels themselves are held to the oracle's roundf codes bit for bit
by the prologue tests."""
import numpy as np

C = np.float32(0.49999997)


def _check(t):
    t = np.asarray(t, dtype=np.float32)
    got = np.trunc((t + np.copysign(C, t)).astype(np.float32)).astype(np.float64)
    tt = t.astype(np.float64)
    ref = np.copysign(np.floor(np.abs(tt) + 0.5), tt)
    bad = np.flatnonzero(got != ref)
    assert bad.size == 0, (t[bad[:5]], got[bad[:5]], ref[bad[:5]])


def test_constant_is_the_float_below_one_half():
    assert C == np.float32(0.5) - np.float32(2.0 ** -25)
    assert np.nextafter(C, np.float32(1)) == np.float32(0.5)


def test_small_values_exhaustive():
    lo, hi = np.array([0.125, 4.0], dtype=np.float32).view(np.uint32)
    t = np.arange(lo, hi, dtype=np.uint32).view(np.float32)
    _check(t)
    _check(-t)
    tiny = np.arange(0, lo, 997, dtype=np.uint32).view(np.float32)
    _check(tiny)
    _check(-tiny)


def test_neighbourhoods_of_halves_and_integers():
    centres = np.arange(0, 513, dtype=np.float32) / np.float32(2)
    bits = centres.view(np.uint32).astype(np.int64)
    offs = np.arange(-4096, 4097, dtype=np.int64)
    t = (bits[:, None] + offs[None, :]).ravel()
    t = t[(t >= 0) & (t < 0x7F800000)].astype(np.uint32).view(np.float32)
    _check(t)
    _check(-t)


def test_binades_with_half_and_unit_spacing():
    for lo in (2.0 ** 22, 2.0 ** 23, 2.0 ** 24):
        b = np.array([lo], dtype=np.float32).view(np.uint32)[0]
        t = np.arange(b - 70000, b + 70000, dtype=np.uint32).view(np.float32)
        _check(t)
        _check(-t)
