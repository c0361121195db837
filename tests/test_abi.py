"""CPU checks of the C-ABI boundary: the library loads, exports every function
declared in include/q4q8.h, and rejects bad calls on the host before any
device work.  Every call below that passes non-null pointers also carries an
invalid argument, so none of them can reach a kernel launch on any machine."""
import ctypes
import os
import re

import pytest

import block_quantized_matmul_q8_amd as q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q4q8.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("q4_quantize", "q8_quantize_rmsnorm", "mul_mat_q4q8", "mul_mat_id_q4q8",
              "mul_mat_id_q4q8_workspace", "q4q8_last_error", "q4q8_set_path",
              "mul_mat_q4q8_blocksums", "q4q8_dispatch_counts", "q4q8_version"):
        assert n in names, n


def test_library_exports_every_declared_symbol():
    L = q.lib()
    for n in declared_functions():
        assert hasattr(L, n), f"{n} declared in q4q8.h but not exported"


def test_binding_has_same_names():
    for n in declared_functions():
        assert callable(getattr(q, n, None)), f"binding lacks {n}"


def test_version():
    assert q.q4q8_version() == 100


def _v(addr):
    return ctypes.c_void_p(addr)


def test_rejects_bad_k_and_dims():
    L = q.lib()
    assert L.mul_mat_q4q8(_v(256), _v(256), 4, 33, _v(256), _v(256), 1, _v(256), None) == q.Q4Q8_E_ARG
    assert "multiple of 32" in q.q4q8_last_error()
    assert L.mul_mat_q4q8(_v(256), _v(256), 4, 0, _v(256), _v(256), 1, _v(256), None) == q.Q4Q8_E_ARG
    assert L.mul_mat_q4q8(_v(256), _v(256), -1, 64, _v(256), _v(256), 1, _v(256), None) == q.Q4Q8_E_ARG
    assert L.mul_mat_q4q8(_v(256), _v(256), 4, 64, _v(256), _v(256), -2, _v(256), None) == q.Q4Q8_E_ARG
    assert L.q4_quantize(_v(256), 4, 48, _v(256), _v(256), None) == q.Q4Q8_E_ARG
    assert L.q8_quantize_rmsnorm(_v(256), 2, 96 + 16, _v(256), ctypes.c_float(1e-5), 0, _v(256), _v(256), None,
                                 None) == q.Q4Q8_E_ARG
    assert L.q8_quantize_rmsnorm(_v(256), 2, 131072 + 32, _v(256), ctypes.c_float(1e-5), 0, _v(256), _v(256),
                                 None, None) == q.Q4Q8_E_ARG


def test_rejects_null_pointers():
    L = q.lib()
    assert L.mul_mat_q4q8(None, _v(256), 4, 64, _v(256), _v(256), 1, _v(256), None) == q.Q4Q8_E_ARG
    assert L.mul_mat_q4q8(_v(256), _v(256), 4, 64, _v(256), _v(256), 1, None, None) == q.Q4Q8_E_ARG
    assert L.q4_quantize(None, 4, 64, _v(256), _v(256), None) == q.Q4Q8_E_ARG
    assert L.q8_quantize_rmsnorm(_v(256), 2, 64, None, ctypes.c_float(1e-5), 0, _v(256), _v(256), None,
                                 None) == q.Q4Q8_E_ARG
    assert L.mul_mat_q4q8_blocksums(_v(256), _v(256), 4, 64, _v(256), _v(256), 1, _v(256), None,
                                    None) == q.Q4Q8_E_ARG


def test_rejects_misaligned_pointers():
    L = q.lib()
    assert L.mul_mat_q4q8(_v(264), _v(256), 4, 64, _v(256), _v(256), 1, _v(256), None) == q.Q4Q8_E_ALIGN
    assert L.mul_mat_q4q8(_v(256), _v(257), 4, 64, _v(256), _v(256), 1, _v(256), None) == q.Q4Q8_E_ALIGN
    assert L.mul_mat_q4q8(_v(256), _v(256), 4, 64, _v(258), _v(256), 1, _v(256), None) == q.Q4Q8_E_ALIGN
    assert L.mul_mat_q4q8(_v(256), _v(256), 4, 64, _v(256), _v(256), 1, _v(258), None) == q.Q4Q8_E_ALIGN
    assert L.q4_quantize(_v(260), 4, 64, _v(256), _v(256), None) == q.Q4Q8_E_ALIGN
    assert L.q8_quantize_rmsnorm(_v(256), 2, 64, _v(256), ctypes.c_float(1e-5), 0, _v(264), _v(256), None,
                                 None) == q.Q4Q8_E_ALIGN


def test_rejects_bad_flags_and_eps():
    L = q.lib()
    assert L.q8_quantize_rmsnorm(_v(256), 2, 64, _v(256), ctypes.c_float(1e-5), 6, _v(256), _v(256), None,
                                 None) == q.Q4Q8_E_ARG
    assert L.q8_quantize_rmsnorm(_v(256), 2, 64, _v(256), ctypes.c_float(-1.0), 0, _v(256), _v(256), None,
                                 None) == q.Q4Q8_E_ARG
    assert L.q8_quantize_rmsnorm(_v(256), 2, 64, _v(256), ctypes.c_float(float("nan")), 0, _v(256), _v(256),
                                 None, None) == q.Q4Q8_E_ARG


def test_mul_mat_id_validation():
    L = q.lib()
    p = _v(256)
    ws = q.mul_mat_id_q4q8_workspace(64, 16, 8)
    assert ws >= 4 * (64 + 1 + 2 * 16 * 8) and ws % 16 == 0
    # n_x_slots neither 1 nor top_k
    assert L.mul_mat_id_q4q8(p, p, 64, 128, 256, p, p, 3, p, 16, 8, p, p, ws, None) == q.Q4Q8_E_ARG
    # top_k out of range, E out of range
    assert L.mul_mat_id_q4q8(p, p, 64, 128, 256, p, p, 1, p, 16, 0, p, p, ws, None) == q.Q4Q8_E_ARG
    assert L.mul_mat_id_q4q8(p, p, 0, 128, 256, p, p, 1, p, 16, 8, p, p, ws, None) == q.Q4Q8_E_ARG
    # workspace too small
    assert L.mul_mat_id_q4q8(p, p, 64, 128, 256, p, p, 1, p, 16, 8, p, p, ws - 16, None) == q.Q4Q8_E_ARG
    # misaligned workspace
    assert L.mul_mat_id_q4q8(p, p, 64, 128, 256, p, p, 1, p, 16, 8, p, _v(260), ws, None) == q.Q4Q8_E_ALIGN
    # null ids
    assert L.mul_mat_id_q4q8(p, p, 64, 128, 256, p, p, 1, None, 16, 8, p, p, ws, None) == q.Q4Q8_E_ARG


def test_empty_problems_are_noops_without_device():
    L = q.lib()
    assert L.mul_mat_q4q8(None, None, 0, 64, None, None, 5, None, None) == q.Q4Q8_OK
    assert L.mul_mat_q4q8(None, None, 7, 64, None, None, 0, None, None) == q.Q4Q8_OK
    assert L.q4_quantize(None, 0, 64, None, None, None) == q.Q4Q8_OK
    assert L.q8_quantize_rmsnorm(None, 0, 64, None, ctypes.c_float(1e-5), 0, None, None, None, None) == q.Q4Q8_OK
    assert L.mul_mat_id_q4q8(None, None, 4, 0, 64, None, None, 1, None, 3, 2, None, None, 0, None) == q.Q4Q8_OK


def test_set_path_and_counters():
    L = q.lib()
    assert L.q4q8_set_path(9) == q.Q4Q8_E_ARG
    assert L.q4q8_dispatch_counts(None, 0) == q.Q4Q8_E_ARG
    q.q4q8_set_path(q.PATH_GEMM)
    q.q4q8_set_path(q.PATH_AUTO)
    c = q.q4q8_dispatch_counts()
    assert set(c) == {"gemv", "gemm", "routed", "prologue"}


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    import block_quantized_matmul_q8_amd as pkg
    monkeypatch.setattr(pkg, "_lib", None)
    monkeypatch.setattr(pkg, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        pkg.lib()


def test_product_never_touches_the_oracle():
    pkg_dir = os.path.join(ROOT, "block_quantized_matmul_q8_amd")
    for dirpath, _, files in os.walk(pkg_dir):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.lower(), f"{f} mentions the oracle"
