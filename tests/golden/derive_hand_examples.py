"""Exact re-derivation of the RMSNorm hand examples E5 and E6 stored in
hand_examples.json.

Each fp32 operation of the prologue (mean = ssq / K, mean + eps, sqrt, 1 / r,
x * s, amax / 127, 1 / d, v * id) is carried out on exact rationals and
rounded once to the nearest binary32 value (ties to even), so the values
follow from the stated definitions alone.  Neither the oracle nor the GPU
library is used.  Run as a script to print the values.
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


if __name__ == "__main__":
    for xv in (1, 2):
        r = constant_row(xv)
        print(f"x={xv}: s {bits(r['s'])} xd {bits(r['d'])} v*id {float(r['v_times_id'])}")
    print("E5 y", bits(e5_y(constant_row(1)["d"])))
