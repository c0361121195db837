"""Python binding of the MI355X Q4 x Q8 library (``libq4q8.so``, C ABI in
``include/q4q8.h``).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI.  PyTorch provides device memory and streams.  There
is no CPU fallback: if the library is not built this module raises on import
of the library (``lib()``), and a failed call raises ``Q4Q8Error``.

The functions take torch CUDA (HIP) tensors in the plane layouts of the header:
    qs u8 [M][K/2], d int16/uint16 [M][K/32] (fp16 bits), xq i8 [B][K],
    xd f32 [B][K/32], y f32 [B][M].
Outputs are allocated with torch when not passed in.  Calls are enqueued on
``stream`` (default: the current torch stream of the tensors' device) and
return without synchronising.
"""
from __future__ import annotations

import ctypes
import os

import torch

from .build import LIB_PATH

Q4Q8_OK = 0
Q4Q8_E_ARG = -1
Q4Q8_E_ALIGN = -2
Q4Q8_E_ARCH = -3
Q4Q8_E_LAUNCH = -4
Q4Q8_E_UNSUPPORTED = -5

Q8_NO_NORM = 1
WEIGHTS_Q8_0 = 2  # Q4Q8_WEIGHTS_Q8_0: a group product with Q8_0 weights

PATH_AUTO = 0
PATH_GEMV = 1
PATH_GEMM = 2
PATH_GEMV_LANES = 3

QK = 32


class Q4Q8Error(RuntimeError):
    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn} failed with status {status}: {message}")
        self.status = status


class GemvDesc(ctypes.Structure):
    """q4q8_gemv_desc of include/q4q8.h."""
    _fields_ = [("qs", ctypes.c_void_p), ("d", ctypes.c_void_p), ("M", ctypes.c_int64), ("K", ctypes.c_int64),
                ("xq", ctypes.c_void_p), ("xd", ctypes.c_void_p), ("x", ctypes.c_void_p), ("g", ctypes.c_void_p),
                ("eps", ctypes.c_float), ("flags", ctypes.c_uint32), ("y", ctypes.c_void_p)]


class GroupPlan(ctypes.Structure):
    """q4q8_group_plan of include/q4q8.h."""
    _fields_ = [("magic", ctypes.c_uint32), ("B", ctypes.c_int32), ("n_records", ctypes.c_int32),
                ("n_prologue", ctypes.c_int32), ("n_windows", ctypes.c_int64), ("max_k", ctypes.c_int64),
                ("map_offset", ctypes.c_int64), ("prologue_offset", ctypes.c_int64),
                ("table_bytes", ctypes.c_int64), ("workspace_bytes", ctypes.c_int64),
                ("weight_formats", ctypes.c_int32), ("max_prologue_k", ctypes.c_int32),
                ("mfma_columns", ctypes.c_int32), ("mfma_grid", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load ``libq4q8.so`` (built in-tree by ``__graft_entry__.build()``)."""
    global _lib
    if _lib is not None:
        return _lib
    # Q4Q8_LIB: another build of the same sources (the host-sanitizer build
    # that the test suite loads in a child process)
    path = os.environ.get("Q4Q8_LIB", LIB_PATH)
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run __graft_entry__.build() first")
    L = ctypes.CDLL(path)
    vp, i64, i32, u32, f32, sz = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_uint32,
                                  ctypes.c_float, ctypes.c_size_t)
    L.q4q8_last_error.restype = ctypes.c_char_p
    L.q4q8_last_error.argtypes = []
    L.q4q8_version.restype = i32
    L.q4q8_version.argtypes = []
    L.q4q8_last_kernel.restype = ctypes.c_char_p
    L.q4q8_last_kernel.argtypes = []
    L.q4_quantize.argtypes = [vp, i64, i64, vp, vp, vp]
    L.q8_quantize_rmsnorm.argtypes = [vp, i64, i64, vp, f32, u32, vp, vp, vp, vp]
    L.mul_mat_q4q8.argtypes = [vp, vp, i64, i64, vp, vp, i64, vp, vp]
    L.mul_mat_q4q8_blocksums.argtypes = [vp, vp, i64, i64, vp, vp, i64, vp, vp, vp]
    L.mul_mat_id_q4q8_workspace.argtypes = [i64, i64, i64]
    L.mul_mat_id_q4q8_workspace.restype = sz
    L.mul_mat_id_q4q8.argtypes = [vp, vp, i64, i64, i64, vp, vp, i64, vp, i64, i64, vp, vp, sz, vp]
    L.mul_mat_id_q4q8_noalloc.argtypes = [vp, vp, i64, i64, i64, vp, vp, i64, vp, i64, i64, vp, vp]
    L.mul_mat_q4q8_rmsnorm.argtypes = [vp, vp, i64, i64, vp, vp, f32, u32, i64, vp, vp]
    L.moe_expert_sum_f32.argtypes = [vp, vp, i64, i64, i64, vp, vp]
    L.q8_quantize_rmsnorm_add.argtypes = [vp, i64, i64, vp, vp, i64, f32, vp, vp, vp, vp]
    L.q8_quantize_swiglu.argtypes = [vp, vp, i64, i64, i64, vp, vp, vp, vp]
    L.q8_0_quantize.argtypes = [vp, i64, i64, vp, vp, vp]
    L.mul_mat_q8_0_q8.argtypes = [vp, vp, i64, i64, vp, vp, i64, vp, vp]
    L.mul_mat_q8_0_q8_blocksums.argtypes = [vp, vp, i64, i64, vp, vp, i64, vp, vp, vp]
    L.q4q8_group_build.argtypes = [ctypes.POINTER(GemvDesc), ctypes.c_int32, i64, vp, sz, vp, sz,
                                   ctypes.POINTER(GroupPlan)]
    L.mul_mat_q4q8_group.argtypes = [vp, ctypes.POINTER(GroupPlan), vp]
    L.q4q8_set_path.argtypes = [i32]
    L.q4q8_dispatch_counts.argtypes = [ctypes.POINTER(ctypes.c_uint64), i32]
    for name in ("q4_quantize", "q8_quantize_rmsnorm", "mul_mat_q4q8", "mul_mat_q4q8_blocksums",
                 "mul_mat_id_q4q8", "mul_mat_id_q4q8_noalloc", "q4q8_set_path", "q4q8_dispatch_counts", "mul_mat_q4q8_rmsnorm",
                 "q4q8_group_build", "mul_mat_q4q8_group", "moe_expert_sum_f32", "q8_quantize_rmsnorm_add",
                 "q8_quantize_swiglu", "q8_0_quantize", "mul_mat_q8_0_q8", "mul_mat_q8_0_q8_blocksums"):
        getattr(L, name).restype = i32
    _lib = L
    return L


def _check(fn: str, status: int) -> None:
    if status != Q4Q8_OK:
        raise Q4Q8Error(fn, status, lib().q4q8_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _need(t, name, dtypes, ndim=None, contiguous=True):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor, got {t.device}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


_F16_BITS = (torch.int16, torch.uint16) if hasattr(torch, "uint16") else (torch.int16,)


def q4_quantize(w, qs=None, d=None, stream=None):
    """fp32 W [M][K] -> (qs u8 [M][K/2], d int16 [M][K/32] fp16 bits)."""
    _need(w, "w", (torch.float32,), 2)
    M, K = w.shape
    if qs is None:
        qs = torch.empty((M, K // 2), dtype=torch.uint8, device=w.device)
    if d is None:
        d = torch.empty((M, max(K // QK, 0)), dtype=torch.int16, device=w.device)
    _need(qs, "qs", (torch.uint8,))
    _need(d, "d", _F16_BITS)
    if qs.numel() != M * (K // 2) or d.numel() != M * (K // QK):
        raise ValueError("qs / d shape does not match w")
    _check("q4_quantize", lib().q4_quantize(_ptr(w), M, K, _ptr(qs), _ptr(d), _stream(stream, w.device)))
    return qs, d


def q8_quantize_rmsnorm(x, g, eps, flags=0, xq=None, xd=None, xs=None, want_xs=False, stream=None):
    """fp32 x [B][K] (and g [K]) -> (xq i8 [B][K], xd f32 [B][K/32], xs i32 [B][K/32] or None)."""
    _need(x, "x", (torch.float32,), 2)
    B, K = x.shape
    if g is not None:
        _need(g, "g", (torch.float32,), 1)
    if xq is None:
        xq = torch.empty((B, K), dtype=torch.int8, device=x.device)
    if xd is None:
        xd = torch.empty((B, K // QK), dtype=torch.float32, device=x.device)
    if xs is None and want_xs:
        xs = torch.empty((B, K // QK), dtype=torch.int32, device=x.device)
    _need(xq, "xq", (torch.int8,))
    _need(xd, "xd", (torch.float32,))
    if xs is not None:
        _need(xs, "xs", (torch.int32,))
    if xq.numel() != B * K or xd.numel() != B * (K // QK):
        raise ValueError("xq / xd shape does not match x")
    _check("q8_quantize_rmsnorm",
           lib().q8_quantize_rmsnorm(_ptr(x), B, K, _ptr(g), ctypes.c_float(eps), flags, _ptr(xq), _ptr(xd),
                                     _ptr(xs), _stream(stream, x.device)))
    return xq, xd, xs


def q8_quantize_rmsnorm_add(x, g, a, eps, xq=None, xd=None, xs=None, want_xs=False, stream=None):
    """RMS_NORM + MUL + ADD -> Q8: x f32 [B][K], g f32 [K], a f32 [K] (one
    addend for every row) or [B][K] -> (xq i8 [B][K], xd f32 [B][K/32],
    xs i32 [B][K/32] or None)."""
    _need(x, "x", (torch.float32,), 2)
    _need(g, "g", (torch.float32,), 1)
    _need(a, "a", (torch.float32,))
    B, K = x.shape
    if tuple(a.shape) == (K,):
        stride = 0
    elif tuple(a.shape) == (B, K):
        stride = K
    else:
        raise ValueError("a must be [K] or [B][K]")
    for t, name in ((x, "x"), (g, "g"), (a, "a")):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if xq is None:
        xq = torch.empty((B, K), dtype=torch.int8, device=x.device)
    if xd is None:
        xd = torch.empty((B, K // QK), dtype=torch.float32, device=x.device)
    if xs is None and want_xs:
        xs = torch.empty((B, K // QK), dtype=torch.int32, device=x.device)
    _need(xq, "xq", (torch.int8,))
    _need(xd, "xd", (torch.float32,))
    if xs is not None:
        _need(xs, "xs", (torch.int32,))
    if xq.numel() != B * K or xd.numel() != B * (K // QK):
        raise ValueError("xq / xd shape does not match x")
    _check("q8_quantize_rmsnorm_add",
           lib().q8_quantize_rmsnorm_add(_ptr(x), B, K, _ptr(g), _ptr(a), stride, ctypes.c_float(eps), _ptr(xq),
                                         _ptr(xd), _ptr(xs), _stream(stream, x.device)))
    return xq, xd, xs


def q8_quantize_swiglu(gate, up, xq=None, xd=None, xs=None, want_xs=False, stream=None):
    """SwiGLU -> Q8: gate, up f32 [B][F] views with unit element stride and the
    same row stride (e.g. the two halves of a stacked [B][2F] gate|up buffer)
    -> (xq i8 [B][F], xd f32 [B][F/32], xs i32 [B][F/32] or None)."""
    _need(gate, "gate", (torch.float32,), 2, contiguous=False)
    _need(up, "up", (torch.float32,), 2, contiguous=False)
    if tuple(gate.shape) != tuple(up.shape):
        raise ValueError("gate and up shapes differ")
    B, F = gate.shape
    if gate.stride(1) != 1 or up.stride(1) != 1 or (B > 1 and gate.stride(0) != up.stride(0)):
        raise ValueError("gate and up need unit element stride and one common row stride")
    row_stride = gate.stride(0) if B > 1 else F
    if xq is None:
        xq = torch.empty((B, F), dtype=torch.int8, device=gate.device)
    if xd is None:
        xd = torch.empty((B, F // QK), dtype=torch.float32, device=gate.device)
    if xs is None and want_xs:
        xs = torch.empty((B, F // QK), dtype=torch.int32, device=gate.device)
    _need(xq, "xq", (torch.int8,))
    _need(xd, "xd", (torch.float32,))
    if xs is not None:
        _need(xs, "xs", (torch.int32,))
    if xq.numel() != B * F or xd.numel() != B * (F // QK):
        raise ValueError("xq / xd shape does not match gate")
    _check("q8_quantize_swiglu",
           lib().q8_quantize_swiglu(_ptr(gate), _ptr(up), B, F, row_stride, _ptr(xq), _ptr(xd), _ptr(xs),
                                    _stream(stream, gate.device)))
    return xq, xd, xs


def _matmul_shapes(qs, d, xq, xd):
    _need(qs, "qs", (torch.uint8,), 2)
    _need(d, "d", _F16_BITS, 2)
    _need(xq, "xq", (torch.int8,), 2)
    _need(xd, "xd", (torch.float32,), 2)
    M, half = qs.shape
    K = 2 * half
    B = xq.shape[0]
    if xq.shape[1] != K or d.shape != (M, K // QK) or xd.shape != (B, K // QK):
        raise ValueError(f"shape mismatch: qs {tuple(qs.shape)} d {tuple(d.shape)} xq {tuple(xq.shape)} "
                         f"xd {tuple(xd.shape)}")
    return M, K, B


def mul_mat_q4q8(qs, d, xq, xd, y=None, stream=None):
    """y f32 [B][M] = Q4 W [M][K] times Q8 x [B][K] (per column)."""
    M, K, B = _matmul_shapes(qs, d, xq, xd)
    if y is None:
        y = torch.empty((B, M), dtype=torch.float32, device=qs.device)
    _need(y, "y", (torch.float32,))
    if y.numel() != B * M:
        raise ValueError("y shape does not match")
    _check("mul_mat_q4q8", lib().mul_mat_q4q8(_ptr(qs), _ptr(d), M, K, _ptr(xq), _ptr(xd), B, _ptr(y),
                                              _stream(stream, qs.device)))
    return y


def mul_mat_q4q8_blocksums(qs, d, xq, xd, y=None, I=None, stream=None):
    """As mul_mat_q4q8, also returning the exact block sums I i32 [B][M][K/32]."""
    M, K, B = _matmul_shapes(qs, d, xq, xd)
    if y is None:
        y = torch.empty((B, M), dtype=torch.float32, device=qs.device)
    if I is None:
        I = torch.empty((B, M, K // QK), dtype=torch.int32, device=qs.device)
    _need(y, "y", (torch.float32,))
    _need(I, "I", (torch.int32,))
    _check("mul_mat_q4q8_blocksums",
           lib().mul_mat_q4q8_blocksums(_ptr(qs), _ptr(d), M, K, _ptr(xq), _ptr(xd), B, _ptr(y), _ptr(I),
                                        _stream(stream, qs.device)))
    return y, I


def q8_0_quantize(w, qw=None, d=None, stream=None):
    """fp32 W [M][K] -> Q8_0 planes (qw i8 [M][K], d int16 [M][K/32] fp16 bits)."""
    _need(w, "w", (torch.float32,), 2)
    M, K = w.shape
    if qw is None:
        qw = torch.empty((M, K), dtype=torch.int8, device=w.device)
    if d is None:
        d = torch.empty((M, max(K // QK, 0)), dtype=torch.int16, device=w.device)
    _need(qw, "qw", (torch.int8,))
    _need(d, "d", _F16_BITS)
    if qw.numel() != M * K or d.numel() != M * (K // QK):
        raise ValueError("qw / d shape does not match w")
    _check("q8_0_quantize", lib().q8_0_quantize(_ptr(w), M, K, _ptr(qw), _ptr(d), _stream(stream, w.device)))
    return qw, d


def _matmul_shapes_q8_0(qw, d, xq, xd):
    _need(qw, "qw", (torch.int8,), 2)
    _need(d, "d", _F16_BITS, 2)
    _need(xq, "xq", (torch.int8,), 2)
    _need(xd, "xd", (torch.float32,), 2)
    M, K = qw.shape
    B = xq.shape[0]
    if xq.shape[1] != K or d.shape != (M, K // QK) or xd.shape != (B, K // QK):
        raise ValueError(f"shape mismatch: qw {tuple(qw.shape)} d {tuple(d.shape)} xq {tuple(xq.shape)} "
                         f"xd {tuple(xd.shape)}")
    return M, K, B


def mul_mat_q8_0_q8(qw, d, xq, xd, y=None, stream=None):
    """y f32 [B][M] = Q8_0 W [M][K] times Q8 x [B][K] (per column)."""
    M, K, B = _matmul_shapes_q8_0(qw, d, xq, xd)
    if y is None:
        y = torch.empty((B, M), dtype=torch.float32, device=qw.device)
    _need(y, "y", (torch.float32,))
    if y.numel() != B * M:
        raise ValueError("y shape does not match")
    _check("mul_mat_q8_0_q8", lib().mul_mat_q8_0_q8(_ptr(qw), _ptr(d), M, K, _ptr(xq), _ptr(xd), B, _ptr(y),
                                                    _stream(stream, qw.device)))
    return y


def mul_mat_q8_0_q8_blocksums(qw, d, xq, xd, y=None, I=None, stream=None):
    """As mul_mat_q8_0_q8, also returning the exact block sums I i32 [B][M][K/32]."""
    M, K, B = _matmul_shapes_q8_0(qw, d, xq, xd)
    if y is None:
        y = torch.empty((B, M), dtype=torch.float32, device=qw.device)
    if I is None:
        I = torch.empty((B, M, K // QK), dtype=torch.int32, device=qw.device)
    _need(y, "y", (torch.float32,))
    _need(I, "I", (torch.int32,))
    if y.numel() != B * M or I.numel() != B * M * (K // QK):
        raise ValueError("y / I shape does not match")
    _check("mul_mat_q8_0_q8_blocksums",
           lib().mul_mat_q8_0_q8_blocksums(_ptr(qw), _ptr(d), M, K, _ptr(xq), _ptr(xd), B, _ptr(y), _ptr(I),
                                           _stream(stream, qw.device)))
    return y, I


def mul_mat_q4q8_rmsnorm(qs, d, x, g, eps, flags=0, y=None, stream=None):
    """y f32 [B][M] = Q4 W [M][K] times Q8(RMSNorm(x) * g) for fp32 x [B][K], the
    prologue folded into the product kernel (same codes as q8_quantize_rmsnorm)."""
    _need(qs, "qs", (torch.uint8,), 2)
    _need(d, "d", _F16_BITS, 2)
    _need(x, "x", (torch.float32,), 2)
    if g is not None:
        _need(g, "g", (torch.float32,), 1)
    M, half = qs.shape
    K = 2 * half
    B = x.shape[0]
    if x.shape[1] != K or d.shape != (M, K // QK):
        raise ValueError("shape mismatch")
    if y is None:
        y = torch.empty((B, M), dtype=torch.float32, device=qs.device)
    _need(y, "y", (torch.float32,))
    _check("mul_mat_q4q8_rmsnorm",
           lib().mul_mat_q4q8_rmsnorm(_ptr(qs), _ptr(d), M, K, _ptr(x), _ptr(g), ctypes.c_float(eps), flags, B,
                                      _ptr(y), _stream(stream, qs.device)))
    return y


def q4q8_group_plan(descs, B):
    """Validate descriptors (a sequence of GemvDesc) and return the GroupPlan
    alone (sizes of the table image and of the workspace)."""
    n = len(descs)
    arr = (GemvDesc * n)(*descs)
    plan = GroupPlan()
    _check("q4q8_group_build", lib().q4q8_group_build(arr, n, B, None, 0, None, 0, ctypes.byref(plan)))
    return plan


def q4q8_group_build(descs, B, workspace=None):
    """Validate descriptors and return (table image as a numpy uint8 array,
    GroupPlan); `workspace` is a device uint8 tensor of at least
    plan.workspace_bytes (see q4q8_group_plan), or None when no product takes
    fp32 rows."""
    import numpy as np

    n = len(descs)
    arr = (GemvDesc * n)(*descs)
    plan = q4q8_group_plan(descs, B)
    nbytes = int(plan.table_bytes)
    image = np.zeros(max(nbytes, 16) + 16, dtype=np.uint8)
    off = (-image.ctypes.data) % 16
    image = image[off:off + nbytes]
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        _need(workspace, "workspace", (torch.uint8,))
        ws_ptr, ws_bytes = _ptr(workspace), workspace.numel()
    _check("q4q8_group_build", lib().q4q8_group_build(arr, n, B, ws_ptr, ws_bytes,
                                                      image.ctypes.data_as(ctypes.c_void_p), nbytes,
                                                      ctypes.byref(plan)))
    return image, plan


def mul_mat_q4q8_group(table_dev, plan, stream=None):
    _need(table_dev, "table", (torch.uint8,))
    _check("mul_mat_q4q8_group", lib().mul_mat_q4q8_group(_ptr(table_dev), ctypes.byref(plan),
                                                          _stream(stream, table_dev.device)))


class Group:
    """A list of independent streaming products launched together.

    Each product is given as keyword arguments: qs (Q4 codes) or qw (Q8_0
    codes), d (weight scales), y (output),
    and either xq, xd (Q8 activations) or x with g / eps (fp32 activations
    that the group's prologue pass normalises and quantises; flags=Q8_NO_NORM
    skips the norm).  The tensors must stay alive and in place while the group
    is used; the group owns its device table and workspace.
    """

    def __init__(self, problems, B=1, device=None):
        descs = []
        self._keep = []
        for i, p in enumerate(problems):
            d, y = p["d"], p["y"]
            if p.get("qw") is not None:
                qs = p["qw"]
                _need(qs, f"problems[{i}].qw", (torch.int8,), 2)
                M, K = qs.shape
                wflag = WEIGHTS_Q8_0
            else:
                qs = p["qs"]
                _need(qs, f"problems[{i}].qs", (torch.uint8,), 2)
                M, half = qs.shape
                K = 2 * half
                wflag = 0
            _need(d, f"problems[{i}].d", _F16_BITS, 2)
            _need(y, f"problems[{i}].y", (torch.float32,), 2)
            if tuple(d.shape) != (M, K // 32) or tuple(y.shape) != (B, M):
                raise ValueError(f"problems[{i}]: d must be ({M}, {K // 32}) and y ({B}, {M})")
            desc = GemvDesc(qs=qs.data_ptr(), d=d.data_ptr(), M=M, K=K, y=y.data_ptr(),
                            eps=float(p.get("eps", 0.0)), flags=int(p.get("flags", 0)) | wflag)
            if p.get("xq") is not None:
                _need(p["xq"], f"problems[{i}].xq", (torch.int8,), 2)
                _need(p["xd"], f"problems[{i}].xd", (torch.float32,), 2)
                if tuple(p["xq"].shape) != (B, K) or tuple(p["xd"].shape) != (B, K // 32):
                    raise ValueError(f"problems[{i}]: xq must be ({B}, {K}) and xd ({B}, {K // 32})")
                desc.xq = p["xq"].data_ptr()
                desc.xd = p["xd"].data_ptr()
            else:
                _need(p["x"], f"problems[{i}].x", (torch.float32,), 2)
                if tuple(p["x"].shape) != (B, K):
                    raise ValueError(f"problems[{i}]: x must be ({B}, {K})")
                desc.x = p["x"].data_ptr()
                if p.get("g") is not None:
                    _need(p["g"], f"problems[{i}].g", (torch.float32,), 1)
                    if p["g"].numel() != K:
                        raise ValueError(f"problems[{i}]: g must have {K} elements")
                    desc.g = p["g"].data_ptr()
            descs.append(desc)
            self._keep.append(p)
        dev = device if device is not None else problems[0]["d"].device
        plan = q4q8_group_plan(descs, B)
        self.workspace = None
        if plan.workspace_bytes > 0:
            self.workspace = torch.empty(int(plan.workspace_bytes), dtype=torch.uint8, device=dev)
        image, self.plan = q4q8_group_build(descs, B, self.workspace)
        self.table = torch.from_numpy(image.copy()).to(dev)

    def __call__(self, stream=None):
        mul_mat_q4q8_group(self.table, self.plan, stream)


def mul_mat_id_q4q8_workspace(E, T, top_k) -> int:
    return int(lib().mul_mat_id_q4q8_workspace(E, T, top_k))


def mul_mat_id_q4q8(qs, d, xq, xd, ids, y=None, ws=None, stream=None):
    """Expert-routed product: qs u8 [E][M][K/2], d [E][M][K/32], xq i8 [T][S][K],
    xd f32 [T][S][K/32] (S = 1 or top_k), ids i32 [T][top_k] -> y f32 [T][top_k][M]."""
    _need(qs, "qs", (torch.uint8,), 3)
    _need(d, "d", _F16_BITS, 3)
    _need(xq, "xq", (torch.int8,), 3)
    _need(xd, "xd", (torch.float32,), 3)
    _need(ids, "ids", (torch.int32,), 2)
    E, M, half = qs.shape
    K = 2 * half
    T, S, K2 = xq.shape
    top_k = ids.shape[1]
    if K2 != K or ids.shape[0] != T or d.shape != (E, M, K // QK) or xd.shape != (T, S, K // QK):
        raise ValueError("shape mismatch")
    if y is None:
        y = torch.empty((T, top_k, M), dtype=torch.float32, device=qs.device)
    _need(y, "y", (torch.float32,))
    need = mul_mat_id_q4q8_workspace(E, T, top_k)
    if ws is None:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=qs.device)
    _need(ws, "ws", (torch.uint8,))
    _check("mul_mat_id_q4q8",
           lib().mul_mat_id_q4q8(_ptr(qs), _ptr(d), E, M, K, _ptr(xq), _ptr(xd), S, _ptr(ids), T, top_k, _ptr(y),
                                 _ptr(ws), ws.numel(), _stream(stream, qs.device)))
    return y


NOALLOC_SCRATCH_BYTES = 1 << 20  # Q4Q8_NOALLOC_SCRATCH_BYTES of q4q8.h


def mul_mat_id_q4q8_noalloc(qs, d, xq, xd, ids, y, stream=None):
    """mul_mat_id_q4q8 through the entry point that allocates nothing: the
    routing workspace is the library's per-device scratch (so y must be given;
    calls on one GPU must be ordered on one stream)."""
    _need(qs, "qs", (torch.uint8,), 3)
    _need(d, "d", _F16_BITS, 3)
    _need(xq, "xq", (torch.int8,), 3)
    _need(xd, "xd", (torch.float32,), 3)
    _need(ids, "ids", (torch.int32,), 2)
    _need(y, "y", (torch.float32,))
    E, M, half = qs.shape
    K = 2 * half
    T, S, K2 = xq.shape
    top_k = ids.shape[1]
    if K2 != K or ids.shape[0] != T or d.shape != (E, M, K // QK) or xd.shape != (T, S, K // QK):
        raise ValueError("shape mismatch")
    if y.numel() != T * top_k * M:
        raise ValueError("y shape does not match")
    _check("mul_mat_id_q4q8_noalloc",
           lib().mul_mat_id_q4q8_noalloc(_ptr(qs), _ptr(d), E, M, K, _ptr(xq), _ptr(xd), S, _ptr(ids), T, top_k,
                                         _ptr(y), _stream(stream, qs.device)))
    return y


def moe_expert_sum_f32(y, w=None, out=None, stream=None):
    """Expert-plane sum: y f32 [T][top_k][M] (a mul_mat_id_q4q8 result),
    w f32 [T][top_k] routing weights or None -> out f32 [T][M], the in-order
    chain of fp32 products and sums."""
    _need(y, "y", (torch.float32,), 3)
    T, top_k, M = y.shape
    if w is not None:
        _need(w, "w", (torch.float32,), 2)
        if tuple(w.shape) != (T, top_k):
            raise ValueError("shape mismatch")
    if out is None:
        out = torch.empty((T, M), dtype=torch.float32, device=y.device)
    _need(out, "out", (torch.float32,), 2)
    if tuple(out.shape) != (T, M):
        raise ValueError("shape mismatch")
    for t, name in ((y, "y"), (w, "w"), (out, "out")):
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    _check("moe_expert_sum_f32",
           lib().moe_expert_sum_f32(_ptr(y), _ptr(w), T, top_k, M, _ptr(out), _stream(stream, y.device)))
    return out


def q4q8_set_path(path: int) -> None:
    _check("q4q8_set_path", lib().q4q8_set_path(path))


def q4q8_dispatch_counts(reset: bool = False):
    out = (ctypes.c_uint64 * 4)()
    _check("q4q8_dispatch_counts", lib().q4q8_dispatch_counts(out, int(reset)))
    return {"gemv": out[0], "gemm": out[1], "routed": out[2], "prologue": out[3]}


def q4q8_last_error() -> str:
    return lib().q4q8_last_error().decode()


def q4q8_last_kernel() -> str:
    """Kernel instance that this thread's last library call launched last."""
    return lib().q4q8_last_kernel().decode()


def q4q8_version() -> int:
    return int(lib().q4q8_version())
