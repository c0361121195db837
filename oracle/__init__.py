"""Q4-weight x Q8-activation oracle (ctypes wrapper over ``q4q8_oracle.c``).

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import this package.  The
product library never calls it and has no CPU fallback to it.

Every function takes and returns numpy arrays in the plane layouts described
in ``q4q8_oracle.h``.  The C library is compiled with gcc by ``build()``
(``oracle/build.py``); it is built on first use if missing.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .build import LIB_PATH, build

_lib = None

_c_f32p = ctypes.POINTER(ctypes.c_float)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    # Q4Q8_ORACLE_LIB: another build of the same source (the sanitizer build
    # that the test suite runs in a child process)
    path = os.environ.get("Q4Q8_ORACLE_LIB", LIB_PATH)
    if path == LIB_PATH and not os.path.exists(LIB_PATH):
        build()
    lib = ctypes.CDLL(path)
    vp, i64, f32, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int
    lib.orc_f32_to_f16.argtypes = [f32]
    lib.orc_f32_to_f16.restype = ctypes.c_uint16
    lib.orc_f16_to_f32.argtypes = [ctypes.c_uint16]
    lib.orc_f16_to_f32.restype = f32
    lib.orc_f32_to_f16_array.argtypes = [vp, i64, vp]
    lib.orc_f16_to_f32_array.argtypes = [vp, i64, vp]
    lib.orc_q4_quantize.argtypes = [vp, i64, i64, vp, vp]
    lib.orc_q4_unpack_codes.argtypes = [vp, i64, i64, vp]
    lib.orc_rmsnorm.argtypes = [vp, i64, i64, f32, vp, vp]
    lib.orc_mul_rows.argtypes = [vp, i64, i64, vp, vp]
    lib.orc_q8_quantize.argtypes = [vp, i64, i64, vp, vp, vp]
    lib.orc_q8_quantize_rmsnorm.argtypes = [vp, i64, i64, vp, f32, i32, vp, vp, vp]
    lib.orc_block_dots.argtypes = [vp, i64, i64, vp, i64, vp]
    lib.orc_mul_mat.argtypes = [vp, vp, i64, i64, vp, vp, i64, vp, vp]
    lib.orc_mul_mat_mt.argtypes = [vp, vp, i64, i64, vp, vp, i64, vp, vp, i32]
    lib.orc_mul_mat_id.argtypes = [vp, vp, i64, i64, i64, vp, vp, i64, vp, i64, i64, vp, i32]
    lib.orc_moe_expert_sum.argtypes = [vp, vp, i64, i64, i64, vp]
    lib.orc_q8_quantize_rmsnorm_add.argtypes = [vp, i64, i64, vp, vp, i64, f32, vp, vp, vp]
    lib.orc_q8w_quantize.argtypes = [vp, i64, i64, vp, vp]
    lib.orc_block_dots_q8w.argtypes = [vp, i64, i64, vp, i64, vp]
    lib.orc_mul_mat_q8w_mt.argtypes = [vp, vp, i64, i64, vp, vp, i64, vp, vp, i32]
    lib.orc_silu_array.argtypes = [vp, i64, vp]
    lib.orc_exp_q_array.argtypes = [vp, i64, vp]
    lib.orc_q8_quantize_swiglu.argtypes = [vp, vp, i64, i64, i64, vp, vp, vp]
    for name in ("orc_f32_to_f16_array", "orc_f16_to_f32_array", "orc_q4_quantize",
                 "orc_q4_unpack_codes", "orc_rmsnorm", "orc_mul_rows", "orc_q8_quantize",
                 "orc_q8_quantize_rmsnorm", "orc_block_dots", "orc_mul_mat", "orc_mul_mat_mt",
                 "orc_mul_mat_id", "orc_moe_expert_sum", "orc_q8_quantize_rmsnorm_add",
                 "orc_silu_array", "orc_exp_q_array", "orc_q8_quantize_swiglu", "orc_q8w_quantize",
                 "orc_block_dots_q8w", "orc_mul_mat_q8w_mt"):
        getattr(lib, name).restype = None
    _lib = lib
    return lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    a = np.asarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return np.ascontiguousarray(a)


def _check_k(K):
    if K <= 0 or K % 32:
        raise ValueError(f"K must be a positive multiple of 32, got {K}")


def f32_to_f16_bits(x) -> np.ndarray:
    x = _c(np.asarray(x, dtype=np.float32), np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().orc_f32_to_f16_array(_p(x), x.size, _p(out))
    return out


def f16_bits_to_f32(h) -> np.ndarray:
    h = _c(np.asarray(h, dtype=np.uint16), np.uint16)
    out = np.empty(h.shape, dtype=np.float32)
    _load().orc_f16_to_f32_array(_p(h), h.size, _p(out))
    return out


def q4_quantize(w):
    """W f32 [M][K] -> (qs u8 [M][K/2], d u16 [M][K/32])."""
    w = _c(w, np.float32)
    M, K = w.shape
    _check_k(K)
    qs = np.empty((M, K // 2), dtype=np.uint8)
    d = np.empty((M, K // 32), dtype=np.uint16)
    _load().orc_q4_quantize(_p(w), M, K, _p(qs), _p(d))
    return qs, d


def q4_unpack_codes(qs, K):
    qs = _c(qs, np.uint8)
    M = qs.shape[0]
    q = np.empty((M, K), dtype=np.uint8)
    _load().orc_q4_unpack_codes(_p(qs), M, K, _p(q))
    return q


def rmsnorm(x, eps):
    """x f32 [B][K] -> (x * s [B][K], s [B])."""
    x = _c(x, np.float32)
    B, K = x.shape
    _check_k(K)
    out = np.empty_like(x)
    s = np.empty(B, dtype=np.float32)
    _load().orc_rmsnorm(_p(x), B, K, np.float32(eps), _p(out), _p(s))
    return out, s


def mul_rows(v, g):
    v = _c(v, np.float32)
    g = _c(g, np.float32)
    B, K = v.shape
    out = np.empty_like(v)
    _load().orc_mul_rows(_p(v), B, K, _p(g), _p(out))
    return out


def q8_quantize(v):
    """v f32 [B][K] -> (xq i8 [B][K], xd f32 [B][K/32], xs i32 [B][K/32])."""
    v = _c(v, np.float32)
    B, K = v.shape
    _check_k(K)
    xq = np.empty((B, K), dtype=np.int8)
    xd = np.empty((B, K // 32), dtype=np.float32)
    xs = np.empty((B, K // 32), dtype=np.int32)
    _load().orc_q8_quantize(_p(v), B, K, _p(xq), _p(xd), _p(xs))
    return xq, xd, xs


def q8_quantize_rmsnorm(x, g, eps, no_norm=False):
    """Fused RMSNorm -> x g -> Q8.  Returns (xq, xd, xs)."""
    x = _c(x, np.float32)
    B, K = x.shape
    _check_k(K)
    g = None if g is None else _c(g, np.float32)
    if not no_norm and (g is None or g.shape != (K,)):
        raise ValueError("g must be f32 [K] unless no_norm")
    xq = np.empty((B, K), dtype=np.int8)
    xd = np.empty((B, K // 32), dtype=np.float32)
    xs = np.empty((B, K // 32), dtype=np.int32)
    _load().orc_q8_quantize_rmsnorm(_p(x), B, K, _p(g), np.float32(eps), int(bool(no_norm)),
                                    _p(xq), _p(xd), _p(xs))
    return xq, xd, xs


def q8_quantize_rmsnorm_add(x, g, a, eps):
    """RMS_NORM + MUL + ADD -> Q8: x f32 [B][K], g f32 [K], a f32 [K] (one
    addend for every row) or [B][K] (one per row).  Returns xq i8 [B][K],
    xd f32 [B][K/32], xs i32 [B][K/32]."""
    x = _c(x, np.float32)
    g = _c(g, np.float32)
    a = _c(a, np.float32)
    B, K = x.shape
    _check_k(K)
    if g.shape != (K,) or a.shape not in ((K,), (B, K)):
        raise ValueError("shape mismatch")
    stride = 0 if a.ndim == 1 else K
    xq = np.empty((B, K), dtype=np.int8)
    xd = np.empty((B, K // 32), dtype=np.float32)
    xs = np.empty((B, K // 32), dtype=np.int32)
    _load().orc_q8_quantize_rmsnorm_add(_p(x), B, K, _p(g), _p(a), stride, float(eps), _p(xq), _p(xd), _p(xs))
    return xq, xd, xs


def exp_q(t):
    """The fixed fp32 exponential of the SwiGLU prologue (see the header)."""
    t = np.ascontiguousarray(np.asarray(t, dtype=np.float32))
    out = np.empty_like(t)
    _load().orc_exp_q_array(_p(t), t.size, _p(out))
    return out


def silu(g):
    """silu(g) = g / (1 + exp_q(-g)), fp32, elementwise."""
    g = np.ascontiguousarray(np.asarray(g, dtype=np.float32))
    out = np.empty_like(g)
    _load().orc_silu_array(_p(g), g.size, _p(out))
    return out


def q8_quantize_swiglu(gate, up):
    """SwiGLU -> Q8: gate, up f32 [B][F] -> (xq i8 [B][F], xd f32 [B][F/32],
    xs i32 [B][F/32]) of h = fl(silu(gate) * up)."""
    gate = _c(gate, np.float32)
    up = _c(up, np.float32)
    if gate.shape != up.shape or gate.ndim != 2:
        raise ValueError("shape mismatch")
    B, F = gate.shape
    _check_k(F)
    xq = np.empty((B, F), dtype=np.int8)
    xd = np.empty((B, F // 32), dtype=np.float32)
    xs = np.empty((B, F // 32), dtype=np.int32)
    _load().orc_q8_quantize_swiglu(_p(gate), _p(up), B, F, F, _p(xq), _p(xd), _p(xs))
    return xq, xd, xs


def block_dots(qs, K, xq):
    """Exact per-block int32 dots I [B][M][K/32]."""
    qs = _c(qs, np.uint8)
    xq = _c(xq, np.int8)
    M = qs.shape[0]
    B = xq.shape[0]
    _check_k(K)
    out = np.empty((B, M, K // 32), dtype=np.int32)
    _load().orc_block_dots(_p(qs), M, K, _p(xq), B, _p(out))
    return out


def mul_mat(qs, d, xq, xd, nthreads=1, want_y64=True):
    """y f32 [B][M] (and the fp64 sum of the same terms, or None)."""
    qs = _c(qs, np.uint8)
    d = _c(d, np.uint16)
    xq = _c(xq, np.int8)
    xd = _c(xd, np.float32)
    M = qs.shape[0]
    K = qs.shape[1] * 2
    B = xq.shape[0]
    _check_k(K)
    if d.shape != (M, K // 32) or xq.shape != (B, K) or xd.shape != (B, K // 32):
        raise ValueError("shape mismatch")
    y = np.empty((B, M), dtype=np.float32)
    y64 = np.empty((B, M), dtype=np.float64) if want_y64 else None
    lib = _load()
    if nthreads == 1:
        lib.orc_mul_mat(_p(qs), _p(d), M, K, _p(xq), _p(xd), B, _p(y), _p(y64))
    else:
        lib.orc_mul_mat_mt(_p(qs), _p(d), M, K, _p(xq), _p(xd), B, _p(y), _p(y64), int(nthreads))
    return y, y64


def mul_mat_id(qs, d, xq, xd, ids, nthreads=1):
    """Expert-routed product.  qs u8 [E][M][K/2], d u16 [E][M][K/32],
    xq i8 [T][n_x_slots][K], xd f32 [T][n_x_slots][K/32], ids i32 [T][top_k]
    -> y f32 [T][top_k][M] (NaN rows for ids outside [0, E))."""
    qs = _c(qs, np.uint8)
    d = _c(d, np.uint16)
    xq = _c(xq, np.int8)
    xd = _c(xd, np.float32)
    ids = _c(ids, np.int32)
    E, M, half = qs.shape
    K = half * 2
    T, n_x_slots, K2 = xq.shape
    top_k = ids.shape[1]
    _check_k(K)
    if K2 != K or ids.shape[0] != T or n_x_slots not in (1, top_k):
        raise ValueError("shape mismatch")
    y = np.empty((T, top_k, M), dtype=np.float32)
    _load().orc_mul_mat_id(_p(qs), _p(d), E, M, K, _p(xq), _p(xd), n_x_slots, _p(ids), T, top_k,
                           _p(y), int(nthreads))
    return y


def moe_expert_sum(y, w=None):
    """Expert-plane sum: y f32 [T][top_k][M], w f32 [T][top_k] or None ->
    out f32 [T][M], the in-order chain of fp32 products and sums."""
    y = _c(y, np.float32)
    T, top_k, M = y.shape
    if top_k < 1:
        raise ValueError("top_k must be >= 1")
    if w is not None:
        w = _c(w, np.float32)
        if w.shape != (T, top_k):
            raise ValueError("shape mismatch")
    out = np.empty((T, M), dtype=np.float32)
    _load().orc_moe_expert_sum(_p(y), _p(w), T, top_k, M, _p(out))
    return out


def q8w_quantize(w):
    """Q8_0 weights: w f32 [M][K] -> (qw i8 [M][K], d u16 [M][K/32])."""
    w = _c(w, np.float32)
    M, K = w.shape
    _check_k(K)
    qw = np.empty((M, K), dtype=np.int8)
    d = np.empty((M, K // 32), dtype=np.uint16)
    _load().orc_q8w_quantize(_p(w), M, K, _p(qw), _p(d))
    return qw, d


def block_dots_q8w(qw, xq):
    """Exact block sums sum_j qw_j x_j: int32 [B][M][K/32]."""
    qw = _c(qw, np.int8)
    xq = _c(xq, np.int8)
    M, K = qw.shape
    B = xq.shape[0]
    _check_k(K)
    I = np.empty((B, M, K // 32), dtype=np.int32)
    _load().orc_block_dots_q8w(_p(qw), M, K, _p(xq), B, _p(I))
    return I


def mul_mat_q8w(qw, d, xq, xd, nthreads=1, want_y64=True):
    """Q8_0 W [M][K] times Q8 x [B][K] -> (y f32 [B][M], y64 f64 [B][M] or None)."""
    qw = _c(qw, np.int8)
    d = _c(d, np.uint16)
    xq = _c(xq, np.int8)
    xd = _c(xd, np.float32)
    M, K = qw.shape
    B = xq.shape[0]
    _check_k(K)
    if d.shape != (M, K // 32) or xq.shape != (B, K) or xd.shape != (B, K // 32):
        raise ValueError("shape mismatch")
    y = np.empty((B, M), dtype=np.float32)
    y64 = np.empty((B, M), dtype=np.float64) if want_y64 else None
    _load().orc_mul_mat_q8w_mt(_p(qw), _p(d), M, K, _p(xq), _p(xd), B, _p(y), _p(y64), int(nthreads))
    return y, y64


def dequantize_q8w(qw, d):
    """fp64 dequantised Q8_0 weights (q * f32(d)) [M][K] (exact in fp64)."""
    return qw.astype(np.float64) * np.repeat(f16_bits_to_f32(d).astype(np.float64), 32, axis=1)


def dequantize_q4(qs, d, K):
    """fp64 dequantised weights ((q - 8) * f32(d)) [M][K] (exact in fp64)."""
    q = q4_unpack_codes(qs, K).astype(np.float64) - 8.0
    dw = f16_bits_to_f32(d).astype(np.float64)
    return q * np.repeat(dw, 32, axis=1)


def dequantize_q8(xq, xd):
    """fp64 dequantised activations (q * d) [B][K] (exact in fp64)."""
    return xq.astype(np.float64) * np.repeat(xd.astype(np.float64), 32, axis=1)
