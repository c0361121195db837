"""A second, independent reading of the Q4 x Q8 arithmetic, in numpy.

TEST INFRASTRUCTURE ONLY.  It is written from the block rules and the product
contract as stated (the Q4-weight x Q8-activation convention that the page
"GGML：Backend 抽象与硬件加速" holds every backend to, sections "Metal 与
Vulkan：默认路径和生成路径" and "硬件选择怎样映射到本栈"; the RMS_NORM+MUL and
RMS_NORM+MUL+ADD fusions of "llama.cpp b10909：Metal后端融合表重构..."; the
MoE routing and GLU ops of "llama.cpp b10981发布：OpenVINO后端优化有状态解码与
GPU MoE推理"), not from the C oracle's source: whole-array numpy operations
where the C code loops, numpy's own float16 cast for the stored scales, and
float64 where an integer decision needs the exact value.  The tests require it
to agree with the C oracle bit for bit, so a slip in either shows.

Every float32 step is one numpy float32 operation (numpy rounds each one to
nearest and never fuses a multiply with an add), so a rule written
fl(a * b + c) is two operations here.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32
QK = 32


def f16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> fp16 bit patterns, numpy's cast (round to nearest even)."""
    return np.asarray(x, dtype=F32).astype(np.float16).view(np.uint16)


def f16_value(h: np.ndarray) -> np.ndarray:
    return np.asarray(h, dtype=np.uint16).view(np.float16).astype(F32)


def _round_half_away(r: np.ndarray) -> np.ndarray:
    """C roundf of float32 values, decided on exact float64 values."""
    a = np.abs(r.astype(np.float64))
    return np.copysign(np.floor(a + 0.5), r.astype(np.float64))


def _blocks(a: np.ndarray) -> np.ndarray:
    rows, K = a.shape
    return a.reshape(rows, K // QK, QK)


def q4_quantize(w: np.ndarray):
    """Q4 block rule.  Per block: amax = max |w|; m = the element of lowest
    index whose magnitude is amax; d = fl(m / -8); codes from the fp32 d:
    q = trunc(fl(fl(w * fl(1/d)) + 8.5)) clamped to [0, 15]; an all-zero block
    has d = +0 and every code 8.  Stored: fp16(d) and the codes packed two per
    byte, code j low and code j + 16 high."""
    w = np.ascontiguousarray(w, dtype=F32)
    M, K = w.shape
    b = _blocks(w)
    mag = np.abs(b)
    amax = mag.max(axis=2)
    first = np.argmax(mag == amax[..., None], axis=2)
    m = np.take_along_axis(b, first[..., None], axis=2)[..., 0]
    zero = amax == 0
    d = np.where(zero, F32(0), m / F32(-8)).astype(F32)
    with np.errstate(divide="ignore", invalid="ignore"):
        inv = (F32(1) / np.where(zero, F32(1), d)).astype(F32)
        t = (b * inv[..., None]).astype(F32)
        t = (t + F32(8.5)).astype(F32)
    q = np.clip(np.trunc(t.astype(np.float64)), 0, 15)
    q = np.where(zero[..., None], 8, q).astype(np.uint8)
    packed = (q[:, :, :16] | (q[:, :, 16:] << 4)).astype(np.uint8)
    return packed.reshape(M, K // 2), f16_bits(d)


def q4_codes(qs: np.ndarray) -> np.ndarray:
    """Unpacked Q4 codes u8 [M][K] of packed qs u8 [M][K/2]."""
    M, half = qs.shape
    b = qs.reshape(M, half // 16, 16)
    return np.concatenate([b & 0xF, b >> 4], axis=2).reshape(M, half * 2)


def q8_quantize(v: np.ndarray):
    """Q8 block rule: amax = max |v|; d = fl(amax / 127) (fp32, stored as is);
    q = roundf(fl(v * fl(1/d))) clamped to [-127, 127]; an all-zero block has
    d = 0 and codes 0.  Also the int32 sum of each block's codes."""
    v = np.ascontiguousarray(v, dtype=F32)
    B, K = v.shape
    b = _blocks(v)
    amax = np.abs(b).max(axis=2)
    d = (amax / F32(127)).astype(F32)
    zero = d == 0
    with np.errstate(divide="ignore", invalid="ignore"):
        inv = (F32(1) / np.where(zero, F32(1), d)).astype(F32)
        r = (b * inv[..., None]).astype(F32)
    q = np.clip(_round_half_away(r), -127, 127)
    q = np.where(zero[..., None], 0, q).astype(np.int8)
    return q.reshape(B, K), d, q.astype(np.int32).sum(axis=2).astype(np.int32)


def rms_scale(x: np.ndarray, eps: float) -> np.ndarray:
    """RMS scale per row: the squares of each 32-block summed one after the
    other in index order, the block sums added pairwise over a power-of-two
    list padded with zeros, mean = fl(sum / K), s = fl(1 / fl(sqrt(fl(mean + eps))))."""
    x = np.ascontiguousarray(x, dtype=F32)
    B, K = x.shape
    b = _blocks(x)
    sq = (b * b).astype(F32)
    p = np.zeros((B, K // QK), dtype=F32)
    for j in range(QK):
        p = (p + sq[:, :, j]).astype(F32)
    n = 1
    while n < p.shape[1]:
        n *= 2
    p = np.concatenate([p, np.zeros((B, n - p.shape[1]), dtype=F32)], axis=1)
    while p.shape[1] > 1:
        p = (p[:, 0::2] + p[:, 1::2]).astype(F32)
    mean = (p[:, 0] / F32(K)).astype(F32)
    root = np.sqrt((mean + F32(eps)).astype(F32)).astype(F32)
    return (F32(1) / root).astype(F32)


def rmsnorm_mul(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """v = fl(fl(x * s) * g): the norm and the weight multiply, each its own op."""
    s = rms_scale(x, eps)
    return ((x.astype(F32) * s[:, None]).astype(F32) * g.astype(F32)[None, :]).astype(F32)


def q8_quantize_rmsnorm(x, g, eps, no_norm=False):
    v = np.asarray(x, dtype=F32) if no_norm else rmsnorm_mul(x, g, eps)
    return q8_quantize(v)


def q8_quantize_rmsnorm_add(x, g, a, eps):
    """v = fl(fl(fl(x * s) * g) + a), then the Q8 rule; a is one [K] addend
    for every row or a [B][K] addend per row."""
    v = rmsnorm_mul(x, g, eps)
    a = np.asarray(a, dtype=F32)
    return q8_quantize((v + (a[None, :] if a.ndim == 1 else a)).astype(F32))


def block_dots(qs: np.ndarray, xq: np.ndarray) -> np.ndarray:
    """Exact integer block dots I [B][M][K/32] = sum_j (q4 - 8) * q8."""
    w = q4_codes(qs).astype(np.int64) - 8
    M, K = w.shape
    B = xq.shape[0]
    wb = w.reshape(M, K // QK, QK)
    xb = xq.astype(np.int64).reshape(B, K // QK, QK)
    return np.einsum("mkj,bkj->bmk", wb, xb).astype(np.int32)


def scale_accumulate(I: np.ndarray, dw_bits: np.ndarray, xd: np.ndarray) -> np.ndarray:
    """y[b][m] = fp32 sum over blocks in ascending order of
    fl(float(I) * fl(f32(d_w) * d_x)), starting from 0."""
    B, M, nb = I.shape
    dw = f16_value(dw_bits)                     # [M][nb]
    dd = (dw[None, :, :] * xd.astype(F32)[:, None, :]).astype(F32)
    t = (I.astype(F32) * dd).astype(F32)
    acc = np.zeros((B, M), dtype=F32)
    for kb in range(nb):
        acc = (acc + t[:, :, kb]).astype(F32)
    return acc


def mul_mat(qs, d, xq, xd):
    return scale_accumulate(block_dots(qs, xq), d, xd)


def mul_mat_id(qs, d, xq, xd, ids):
    """y[t][s] = mul_mat(expert ids[t][s], activation row (t, s) or (t, 0));
    an id outside [0, E) gives a row of NaNs."""
    E, M, _ = qs.shape
    T, n_x_slots, _ = xq.shape
    top_k = ids.shape[1]
    y = np.empty((T, top_k, M), dtype=F32)
    for t in range(T):
        for s in range(top_k):
            e = int(ids[t, s])
            r = s if n_x_slots == top_k else 0
            if 0 <= e < E:
                y[t, s] = mul_mat(qs[e], d[e], xq[t, r:r + 1], xd[t, r:r + 1])[0]
            else:
                y[t, s] = np.nan
    return y


def q8w_quantize(w: np.ndarray):
    """Q8_0 weights: the Q8 rule with the scale stored as fp16 and the codes
    taken from the fp32 scale."""
    q, d, _ = q8_quantize(w)
    return q, f16_bits(d)


def mul_mat_q8w(qw, d, xq, xd):
    M, K = qw.shape
    B = xq.shape[0]
    wb = qw.astype(np.int64).reshape(M, K // QK, QK)
    xb = xq.astype(np.int64).reshape(B, K // QK, QK)
    I = np.einsum("mkj,bkj->bmk", wb, xb).astype(np.int32)
    return scale_accumulate(I, d, xd)


def moe_expert_sum(y: np.ndarray, w: np.ndarray | None = None) -> np.ndarray:
    """out[t] = ((v_0 + v_1) + v_2) + ..., v_s = fl(w[t][s] * y[t][s]) (or y)."""
    y = np.asarray(y, dtype=F32)
    v = y if w is None else (np.asarray(w, dtype=F32)[:, :, None] * y).astype(F32)
    out = v[:, 0].copy()
    for s in range(1, y.shape[1]):
        out = (out + v[:, s]).astype(F32)
    return out


# fixed fp32 exponential of the SwiGLU prologue: reduction by ln 2 split in two
# constants, a degree-7 Taylor polynomial in Horner form, exact scaling by 2^n
_L2E = np.array([0x3FB8AA3B], dtype=np.uint32).view(F32)[0]
_LN2_HI = np.array([0x3F317200], dtype=np.uint32).view(F32)[0]
_LN2_LO = np.array([0x35BFBE8E], dtype=np.uint32).view(F32)[0]


def exp_q(t: np.ndarray) -> np.ndarray:
    import math

    t = np.asarray(t, dtype=F32)
    with np.errstate(over="ignore", invalid="ignore"):
        n = np.rint((t * _L2E).astype(F32)).astype(F32)
        n = np.clip(np.nan_to_num(n, nan=0.0), -25, 127).astype(F32)
        r = ((t - (n * _LN2_HI).astype(F32)).astype(F32) - (n * _LN2_LO).astype(F32)).astype(F32)
        c = np.full(t.shape, F32(1.0 / math.factorial(7)), dtype=F32)
        for k in range(6, 0, -1):
            c = ((c * r).astype(F32) + F32(1.0 / math.factorial(k))).astype(F32)
        p = ((c * r).astype(F32) + F32(1)).astype(F32)
        e = np.ldexp(p, n.astype(np.int32)).astype(F32)
    e = np.where(t > 88, F32(np.inf), e)
    e = np.where(t < -17, F32(0), e)
    return np.where(np.isnan(t), F32(np.nan), e).astype(F32)


def q8_quantize_swiglu(gate, up):
    """h = fl(silu(gate) * up), silu(g) = fl(g / fl(1 + exp_q(-g))), then Q8."""
    gate = np.asarray(gate, dtype=F32)
    up = np.asarray(up, dtype=F32)
    with np.errstate(over="ignore"):
        den = (F32(1) + exp_q((-gate).astype(F32))).astype(F32)
        silu = (gate / den).astype(F32)
    return q8_quantize((silu * up).astype(F32))
