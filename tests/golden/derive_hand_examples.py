"""Exact re-derivation of the hand examples E5, E6 and E7 stored in
hand_examples.json.

Each fp32 operation of the prologue (mean = ssq / K, mean + eps, sqrt, 1 / r,
x * s, amax / 127, 1 / d, v * id) and of the block rules (m / -8, 1 / d,
w * id, + 8.5) is carried out on exact rationals and rounded once to the
nearest binary32 value (ties to even), so the values follow from the stated
definitions alone.  Neither the oracle nor the GPU library is used.  Run as a
script to print the values.

E7 tells the reciprocal-multiply reading of the block rules (id = fl(1 / d),
then fl(w * id)) from a plain division fl(w / d): its blocks put the two on
opposite sides of a rounding boundary, so the codes differ.  E8 tells codes
taken from the fp32 scale (the reading) from codes taken from the stored
fp16 scale, for the Q4 and the Q8_0 weight rules.
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction


def round_f32(q: Fraction) -> Fraction:
    """Nearest binary32 value to the exact rational q (normal range), ties to even."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = math.floor(math.log2(a.numerator) - math.log2(a.denominator))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp = Fraction(2) ** (e - 23)
    n = a / ulp
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * ulp


def sqrt_f32(q: Fraction) -> Fraction:
    """Nearest binary32 value to sqrt(q) for a positive rational q."""
    c = round_f32(Fraction(math.sqrt(q.numerator / q.denominator)))
    e = math.floor(math.log2(c.numerator) - math.log2(c.denominator))
    ulp = Fraction(2) ** (e - 23)
    cands = [c + k * ulp for k in range(-4, 5)]
    # the nearest float to sqrt(q) is the candidate whose rounding interval
    # holds sqrt(q): compare squares against q exactly
    best = min(cands, key=lambda t: abs(t * t - q))
    lo, hi = best - ulp / 2, best + ulp / 2
    assert lo * lo <= q <= hi * hi
    return best


def round_f16(q: Fraction) -> Fraction:
    """Nearest binary16 value to q (normal range), ties to even."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = 0
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    assert e >= -14, "subnormal binary16 not handled"
    ulp = Fraction(2) ** (e - 10)
    n = a / ulp
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * ulp


def bits(q: Fraction) -> str:
    return "0x%08x" % struct.unpack("<I", struct.pack("<f", float(q)))[0]


def constant_row(x: int, K: int = 32, eps: float = 1e-5):
    """RMSNorm * g -> Q8 of a row of K equal values x with g = 1."""
    e = round_f32(Fraction(eps))
    ssq = Fraction(x * x * K)  # every partial sum is an exact small integer
    mean = round_f32(ssq / K)
    r = sqrt_f32(round_f32(mean + e))
    s = round_f32(1 / r)
    v = round_f32(x * s)
    d = round_f32(v / 127)
    inv = round_f32(1 / d)
    code = round_f32(v * inv)
    return {"s": s, "v": v, "d": d, "v_times_id": code}


def e5_y(d: Fraction, I: int = -2032) -> Fraction:
    """y = fl(I * fl(f32(d_w) * d_x)) with d_w = 1."""
    return round_f32(I * round_f32(Fraction(1) * d))


def _trunc(q: Fraction) -> int:
    """Truncation toward zero."""
    return int(q)  # int() of a Fraction truncates toward zero


def q4_block(w, recip: bool = True, codes_from_f16: bool = False):
    """Q4 rule on one block of exact fp32 values w (Fractions): d = fl(m / -8)
    with m the first element of largest magnitude; codes
    clamp(trunc(fl(fl(w * fl(1 / d)) + 8.5)), 0, 15), or with fl(w / d) in
    place of the reciprocal product when recip is False, or from the fp16
    scale in place of d when codes_from_f16 is True."""
    amax, m = Fraction(0), Fraction(0)
    for v in w:
        if abs(v) > amax:
            amax, m = abs(v), v
    if amax == 0:
        return Fraction(0), [8] * len(w)
    d = round_f32(m / -8)
    if codes_from_f16:
        d = round_f16(d)
    inv = round_f32(1 / d)
    codes = []
    for v in w:
        t = round_f32(v * inv) if recip else round_f32(v / d)
        u = round_f32(t + Fraction(17, 2))
        codes.append(min(15, max(0, _trunc(u))))
    return d, codes


def q8_block(v, recip: bool = True, codes_from_f16: bool = False):
    """Q8 rule on one block of exact fp32 values v: d = fl(amax / 127); codes
    roundf(fl(v * fl(1 / d))) (halves away from zero) clamped to +-127, or with
    fl(v / d) when recip is False, or from fp16(d) when codes_from_f16 is True
    (the Q8_0 weight rule stores fp16(d))."""
    amax = max(abs(x) for x in v)
    if amax == 0:
        return Fraction(0), [0] * len(v)
    d = round_f32(amax / 127)
    if codes_from_f16:
        d = round_f16(d)
    inv = round_f32(1 / d)
    codes = []
    for x in v:
        t = round_f32(x * inv) if recip else round_f32(x / d)
        a = abs(t)
        r = _trunc(a + Fraction(1, 2))  # floor(|t| + 1/2): halves away from zero
        codes.append(max(-127, min(127, r if t >= 0 else -r)))
    return d, codes


def e7_blocks():
    """The E7 blocks: Q4 w = [-56, -52.5, 0 x 30] (d = 7, fl(1 / 7) rounds up,
    so fl(-52.5 * id) = -7.5 - 2^-21 and the code is 0, where -52.5 / 7 = -7.5
    exactly gives 1); Q8 (and Q8_0) v = [5207, -5186.5, 0 x 30] (d = 41,
    fl(1 / 41) rounds down, so fl(-5186.5 * id) = -126.5 + 2^-17 and the code
    is -126, where -5186.5 / 41 = -126.5 exactly gives -127)."""
    w = [Fraction(-56), Fraction(-105, 2)] + [Fraction(0)] * 30
    v = [Fraction(5207), Fraction(-10373, 2)] + [Fraction(0)] * 30
    out = {}
    for name, fn, blk in (("q4", q4_block, w), ("q8", q8_block, v)):
        d, codes = fn(blk, True)
        d_div, codes_div = fn(blk, False)
        assert d == d_div
        out[name] = {"d": d, "codes": codes, "codes_if_divided": codes_div}
    return out


def e8_blocks():
    """The E8 blocks, codes from the fp32 scale d = 0.1f: Q4 w = [-0.8, 0.34995,
    0 x 30] (fp16(d) = 0.0999755859375 would move w / d from 3.4995 to 3.5004,
    across the rounding boundary of 3.5); Q8_0 w = [12.7, 0.349995, 0 x 30]
    (3.49995 against 3.5008)."""
    def f32(x: str) -> Fraction:
        return Fraction(struct.unpack("<f", struct.pack("<f", float(x)))[0])
    w = [f32("-0.8"), f32("0.34995")] + [Fraction(0)] * 30
    v = [f32("12.7"), f32("0.349995")] + [Fraction(0)] * 30
    out = {}
    for name, fn, blk in (("q4", q4_block, w), ("q8_0", q8_block, v)):
        d, codes = fn(blk)
        _, codes16 = fn(blk, codes_from_f16=True)
        out[name] = {"d": d, "d16": round_f16(d), "codes": codes, "codes_if_from_f16": codes16}
    return out


if __name__ == "__main__":
    for xv in (1, 2):
        r = constant_row(xv)
        print(f"x={xv}: s {bits(r['s'])} xd {bits(r['d'])} v*id {float(r['v_times_id'])}")
    print("E5 y", bits(e5_y(constant_row(1)["d"])))
    for name, r in e7_blocks().items():
        print(f"E7 {name}: d {float(r['d'])} codes {r['codes'][:4]} if divided {r['codes_if_divided'][:4]}")
    for name, r in e8_blocks().items():
        print(f"E8 {name}: d {bits(r['d'])} fp16 {float(r['d16'])} codes {r['codes'][:3]} "
              f"if from fp16 {r['codes_if_from_f16'][:3]}")
