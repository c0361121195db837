"""CPU checks of the C-ABI boundary: the library loads, exports every function
declared in include/q4q8.h, and rejects bad calls on the host before any
device work.  Every call below that passes non-null pointers also carries an
invalid argument, so none of them can reach a kernel launch on any machine."""
import ctypes
import os
import re

import numpy as np
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
    for n in ("q4_quantize", "q8_quantize_rmsnorm", "mul_mat_q4q8", "mul_mat_id_q4q8", "moe_expert_sum_f32",
              "q8_quantize_rmsnorm_add", "q8_quantize_swiglu", "q8_0_quantize", "mul_mat_q8_0_q8",
              "mul_mat_q8_0_q8_blocksums",
              "mul_mat_id_q4q8_workspace", "q4q8_last_error", "q4q8_set_path",
              "mul_mat_q4q8_blocksums", "q4q8_dispatch_counts", "q4q8_last_kernel", "q4q8_version"):
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


def test_last_kernel_before_any_launch():
    """No launch on this thread yet (the CPU suite launches nothing)."""
    assert q.q4q8_last_kernel() == ""


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
    # offsets[E + 1] | list[n] | rank[n] | sel[E] | cost prefix[E + 1] | control[4]
    assert ws >= 4 * (64 + 1 + 2 * 16 * 8 + 64 + 65 + 4) and ws % 16 == 0
    # n_x_slots neither 1 nor top_k
    assert L.mul_mat_id_q4q8(p, p, 64, 128, 256, p, p, 3, p, 16, 8, p, p, ws, None) == q.Q4Q8_E_ARG
    # top_k out of range, E out of range
    assert L.mul_mat_id_q4q8(p, p, 64, 128, 256, p, p, 1, p, 16, 0, p, p, ws, None) == q.Q4Q8_E_ARG
    assert L.mul_mat_id_q4q8(p, p, 0, 128, 256, p, p, 1, p, 16, 8, p, p, ws, None) == q.Q4Q8_E_ARG
    ws_big = q.mul_mat_id_q4q8_workspace(4097, 16, 8)
    assert L.mul_mat_id_q4q8(p, p, 4097, 128, 256, p, p, 1, p, 16, 8, p, p, ws_big, None) == q.Q4Q8_E_ARG
    # a schedule whose total cost would overflow int32 is refused before any device call
    ws_4k = q.mul_mat_id_q4q8_workspace(4096, 16, 8)
    assert L.mul_mat_id_q4q8(p, p, 4096, 1 << 30, 256, p, p, 1, p, 16, 8, p, p, ws_4k,
                             None) == q.Q4Q8_E_UNSUPPORTED
    # workspace too small
    assert L.mul_mat_id_q4q8(p, p, 64, 128, 256, p, p, 1, p, 16, 8, p, p, ws - 16, None) == q.Q4Q8_E_ARG
    # misaligned workspace
    assert L.mul_mat_id_q4q8(p, p, 64, 128, 256, p, p, 1, p, 16, 8, p, _v(260), ws, None) == q.Q4Q8_E_ALIGN
    # null ids
    assert L.mul_mat_id_q4q8(p, p, 64, 128, 256, p, p, 1, None, 16, 8, p, p, ws, None) == q.Q4Q8_E_ARG


def test_q8_quantize_rmsnorm_add_validation():
    L = q.lib()
    p = _v(256)
    eps = ctypes.c_float(1e-5)
    assert L.q8_quantize_rmsnorm_add(p, 2, 48, p, p, 0, eps, p, p, None, None) == q.Q4Q8_E_ARG     # K % 32
    assert L.q8_quantize_rmsnorm_add(p, 2, 64, p, p, 32, eps, p, p, None, None) == q.Q4Q8_E_ARG    # stride
    assert L.q8_quantize_rmsnorm_add(p, 2, 64, p, None, 0, eps, p, p, None, None) == q.Q4Q8_E_ARG  # null a
    assert L.q8_quantize_rmsnorm_add(p, 2, 64, p, _v(264), 64, eps, p, p, None, None) == q.Q4Q8_E_ALIGN
    assert L.q8_quantize_rmsnorm_add(p, 2, 64, p, p, 0, ctypes.c_float(-1.0), p, p, None, None) == q.Q4Q8_E_ARG
    assert L.q8_quantize_rmsnorm_add(None, 0, 64, None, None, 0, eps, None, None, None, None) == q.Q4Q8_OK


def test_q8_quantize_swiglu_validation():
    L = q.lib()
    p = _v(256)
    assert L.q8_quantize_swiglu(p, p, 2, 48, 48, p, p, None, None) == q.Q4Q8_E_ARG        # F % 32
    assert L.q8_quantize_swiglu(p, p, 2, 64, 32, p, p, None, None) == q.Q4Q8_E_ARG        # stride < F
    assert L.q8_quantize_swiglu(p, p, 2, 64, 66, p, p, None, None) == q.Q4Q8_E_ARG        # stride % 4
    assert L.q8_quantize_swiglu(p, None, 2, 64, 64, p, p, None, None) == q.Q4Q8_E_ARG
    assert L.q8_quantize_swiglu(p, _v(264), 2, 64, 128, p, p, None, None) == q.Q4Q8_E_ALIGN
    assert L.q8_quantize_swiglu(None, None, 0, 64, 64, None, None, None, None) == q.Q4Q8_OK


def test_moe_expert_sum_validation():
    L = q.lib()
    y, out = _v(256), _v(65536)
    assert L.moe_expert_sum_f32(y, None, 4, 0, 16, out, None) == q.Q4Q8_E_ARG      # top_k < 1
    assert L.moe_expert_sum_f32(y, None, 4, 65, 16, out, None) == q.Q4Q8_E_ARG     # top_k > 64
    assert L.moe_expert_sum_f32(y, None, -1, 2, 16, out, None) == q.Q4Q8_E_ARG
    assert L.moe_expert_sum_f32(None, None, 4, 2, 16, out, None) == q.Q4Q8_E_ARG
    assert L.moe_expert_sum_f32(_v(258), None, 4, 2, 16, out, None) == q.Q4Q8_E_ALIGN
    # out inside y's [T][top_k][M] planes
    assert L.moe_expert_sum_f32(y, None, 4, 2, 16, _v(256 + 64), None) == q.Q4Q8_E_ARG
    assert L.moe_expert_sum_f32(None, None, 0, 2, 16, None, None) == q.Q4Q8_OK      # empty: no device use


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
    assert L.q4q8_set_path(4) == q.Q4Q8_E_ARG
    q.q4q8_set_path(q.PATH_GEMM)
    q.q4q8_set_path(q.PATH_GEMV_LANES)
    q.q4q8_set_path(q.PATH_AUTO)
    c = q.q4q8_dispatch_counts()
    assert set(c) == {"gemv", "gemm", "routed", "prologue"}


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    import block_quantized_matmul_q8_amd as pkg
    monkeypatch.setattr(pkg, "_lib", None)
    monkeypatch.delenv("Q4Q8_LIB", raising=False)
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


def test_struct_layouts_match_the_header(tmp_path):
    """The ctypes mirrors of q4q8_gemv_desc / q4q8_group_plan match the C layout."""
    import subprocess
    src = tmp_path / "sz.c"
    src.write_text('#include "q4q8.h"\n#include <stdio.h>\n#include <stddef.h>\n'
                   'int main(void){printf("%zu %zu %zu %zu %zu\\n", sizeof(q4q8_gemv_desc), sizeof(q4q8_group_plan),'
                   ' offsetof(q4q8_gemv_desc, y), offsetof(q4q8_group_plan, workspace_bytes),'
                   ' offsetof(q4q8_group_plan, weight_formats));'
                   'printf("%zu\\n", offsetof(q4q8_group_plan, mfma_grid));return 0;}\n')
    exe = tmp_path / "sz"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()
    assert int(out[0]) == ctypes.sizeof(q.GemvDesc)
    assert int(out[1]) == ctypes.sizeof(q.GroupPlan)
    assert int(out[2]) == q.GemvDesc.y.offset
    assert int(out[3]) == q.GroupPlan.workspace_bytes.offset
    assert int(out[4]) == q.GroupPlan.weight_formats.offset
    assert int(out[5]) == q.GroupPlan.mfma_grid.offset


def _desc(M=64, K=2048, qs=256, d=256, xq=256, xd=256, x=None, g=None, y=256, flags=0, eps=1e-5):
    return q.GemvDesc(qs=qs, d=d, M=M, K=K, xq=xq, xd=xd, x=x, g=g, y=y, eps=eps, flags=flags)


def _build(descs, B, ws=0, ws_bytes=0):
    """q4q8_group_build through the C ABI with a fake workspace address."""
    n = len(descs)
    arr = (q.GemvDesc * n)(*descs)
    plan = q.GroupPlan()
    st = q.lib().q4q8_group_build(arr, n, B, None, 0, None, 0, ctypes.byref(plan))
    if st != q.Q4Q8_OK:
        raise q.Q4Q8Error("q4q8_group_build", st, q.q4q8_last_error())
    image = np.zeros(int(plan.table_bytes) + 16, np.uint8)
    off = (-image.ctypes.data) % 16
    image = image[off:off + int(plan.table_bytes)]
    st = q.lib().q4q8_group_build(arr, n, B, ctypes.c_void_p(ws) if ws else None, ws_bytes,
                                  image.ctypes.data_as(ctypes.c_void_p), int(plan.table_bytes), ctypes.byref(plan))
    if st != q.Q4Q8_OK:
        raise q.Q4Q8Error("q4q8_group_build", st, q.q4q8_last_error())
    return image, plan


def test_group_build_layout_is_host_only():
    WS = 1 << 20
    ok_q8 = _desc()
    fused = _desc(xq=None, xd=None, x=512, g=768, K=8192)
    same_input = _desc(xq=None, xd=None, x=512, g=768, K=8192, M=32, y=4096)   # shares the prologue job
    other_eps = _desc(xq=None, xd=None, x=512, g=768, K=8192, eps=1e-6, M=8)    # a job of its own
    raw = _desc(xq=None, xd=None, x=512, g=768, K=8192, flags=q.Q8_NO_NORM, M=8)  # g is ignored: own job
    image, plan = _build([ok_q8, fused, _desc(M=0), same_input, other_eps, raw], 1, WS, 3 * 9216)
    # the empty product dropped; a window is 16 rows' worth of 16-byte loads
    # per lane for each of the 4 waves: 64 rows at K = 2048 (one 32-block per
    # lane), 16 rows at K = 8192 (four per lane)
    assert plan.n_records == 5 and plan.B == 1 and plan.n_prologue == 3 and plan.max_k == 8192
    assert plan.max_prologue_k == 8192
    assert plan.n_windows == 1 + 4 + 2 + 1 + 1
    # Q8 planes per job: 8192 codes then 256 fp32 scales, 16-byte aligned
    assert plan.workspace_bytes == 3 * (8192 + 1024)
    assert plan.map_offset == 5 * 96
    assert plan.prologue_offset == (plan.map_offset + 4 * plan.n_windows + 15) // 16 * 16
    assert plan.table_bytes == plan.prologue_offset + 3 * 48
    recs = image[:plan.map_offset].view(np.int32).reshape(5, 24)
    ptrs = image[:plan.map_offset].view(np.int64).reshape(5, 12)
    # record fields: M, K at int32 offsets 14, 15; mode 17; win_begin / n_win at 18, 19
    assert recs[0, 14] == 64 and recs[0, 15] == 2048 and recs[0, 18] == 0 and recs[0, 19] == 1
    assert recs[1, 14] == 64 and recs[1, 15] == 8192 and recs[1, 18] == 1 and recs[1, 19] == 4
    assert (recs[:, 17] == 0).all()           # the streaming pass always reads Q8 planes
    # xq / xd pointers (int64 slots 2, 3) of the products with fp32 rows point at their job's planes
    assert ptrs[0, 2] == 256 and ptrs[0, 3] == 256
    for r, job in ((1, 0), (2, 0), (3, 1), (4, 2)):
        assert ptrs[r, 2] == WS + job * 9216 and ptrs[r, 3] == WS + job * 9216 + 8192
        assert ptrs[r, 4] == 0 and ptrs[r, 5] == 0
    assert image[plan.map_offset:plan.map_offset + 4 * plan.n_windows].view(np.int32).tolist() == \
        [0] + [1] * 4 + [2] * 2 + [3] + [4]
    jobs = image[plan.prologue_offset:].view(np.int64).reshape(3, 6)
    jobs32 = image[plan.prologue_offset:].view(np.int32).reshape(3, 12)
    jobsf = image[plan.prologue_offset:].view(np.float32).reshape(3, 12)
    assert jobs[:, 0].tolist() == [512, 512, 512]
    assert jobs[:, 1].tolist() == [768, 768, 0]                       # raw jobs carry no g
    assert jobs[:, 2].tolist() == [WS, WS + 9216, WS + 2 * 9216]
    assert jobs[:, 3].tolist() == [WS + 8192, WS + 9216 + 8192, WS + 2 * 9216 + 8192]
    assert jobs32[:, 8].tolist() == [8192] * 3 and jobs32[:, 10].tolist() == [0, 0, 1]
    assert jobsf[0, 9] == np.float32(1e-5) and jobsf[1, 9] == np.float32(1e-6)
    # B = 2: planes hold two rows
    _, plan2 = _build([fused], 2, WS, 2 * 8192 + 2 * 1024)
    assert plan2.workspace_bytes == 2 * 8192 + 2 * 1024
    # a group of Q8 products needs no workspace
    _, plan3 = _build([ok_q8], 1)
    assert plan3.workspace_bytes == 0 and plan3.n_prologue == 0


def test_group_build_tiled_layout():
    """B > 8 takes the tiled route: one record per product with
    ceil(M/128) * ceil(B/128) tiles, the long-K products' tiles first."""
    WS = 1 << 20
    a = _desc(M=300, K=2048)
    b = _desc(M=130, K=8192, xq=None, xd=None, x=512, g=768)
    c = _desc(M=128, K=8192, y=4096)
    image, plan = _build([a, b, c], 300, WS, 300 * (8192 + 1024))
    ta, tb, tc = 3 * 3, 2 * 3, 1 * 3
    assert plan.n_records == 3 and plan.B == 300 and plan.n_windows == ta + tb + tc
    recs = image[:plan.map_offset].view(np.int32).reshape(3, 24)
    # records stay in the caller's order; win_begin follows the K-descending work order
    assert recs[:, 19].tolist() == [ta, tb, tc]
    assert recs[1, 18] == 0 and recs[2, 18] == tb and recs[0, 18] == tb + tc
    assert image[plan.map_offset:plan.map_offset + 4 * plan.n_windows].view(np.int32).tolist() == \
        [1] * tb + [2] * tc + [0] * ta
    assert plan.n_prologue == 1 and plan.workspace_bytes == 300 * 8192 + 300 * 256 * 4


def test_group_build_q8_0_records():
    """A Q8_0 product (descriptor flag) carries its weight format in its
    record (int32 offset 20) and, with two loads per block, half the rows per
    window: 32 rows at K = 2048, B = 1, against 64 for Q4."""
    a = _desc(M=64, K=2048)
    b = _desc(M=64, K=2048, flags=q.WEIGHTS_Q8_0, y=4096)
    c = _desc(M=64, K=2048, flags=q.WEIGHTS_Q8_0 | q.Q8_NO_NORM, xq=None, xd=None, x=512, g=None, y=8192)
    image, plan = _build([a, b, c], 1, 1 << 20, 4096)
    recs = image[:plan.map_offset].view(np.int32).reshape(3, 24)
    assert recs[:, 20].tolist() == [0, 1, 1]
    assert recs[:, 19].tolist() == [1, 2, 2] and plan.n_windows == 5
    assert plan.n_prologue == 1 and plan.weight_formats == 3
    # the tiled route keeps the format too
    image, plan = _build([a, b], 300)
    recs = image[:plan.map_offset].view(np.int32).reshape(2, 24)
    assert recs[:, 20].tolist() == [0, 1] and plan.weight_formats == 3
    # uniform groups select the single-format instances
    assert _build([a], 1)[1].weight_formats == 1
    assert _build([b, _desc(M=0, flags=q.WEIGHTS_Q8_0)], 1)[1].weight_formats == 2


def test_group_build_validation_is_host_only():
    bad = [
        ([_desc(K=100)], 1, q.Q4Q8_E_ARG),
        ([_desc(qs=264)], 1, q.Q4Q8_E_ALIGN),
        ([_desc(xq=None, xd=None)], 1, q.Q4Q8_E_ARG),               # neither xq nor x
        ([_desc(xd=None)], 1, q.Q4Q8_E_ARG),                        # xq without xd
        ([_desc(xq=None, xd=None, x=512, g=None)], 1, q.Q4Q8_E_ARG),  # norm without g
        ([_desc(xq=None, xd=None, x=520, g=768)], 1, q.Q4Q8_E_ALIGN),
        ([_desc(flags=4)], 1, q.Q4Q8_E_ARG),
        ([_desc()], 70000, q.Q4Q8_E_UNSUPPORTED),                   # B beyond a grouped launch
        ([_desc(xq=None, xd=None, x=512, g=768, K=262144)], 300, q.Q4Q8_E_ARG),  # fp32 rows too long
        ([_desc(K=131072)], 1, q.Q4Q8_E_UNSUPPORTED),               # K beyond the register blocking
        # K of an odd number of blocks beyond the lane-per-block kernel at B = 8 (the
        # multi-column kernel takes whole block pairs only)
        ([_desc(xq=None, xd=None, x=512, g=768, K=32800)], 8, q.Q4Q8_E_UNSUPPORTED),
    ]
    for descs, B, code in bad:
        with pytest.raises(q.Q4Q8Error) as ei:
            _build(descs, B, 1 << 20, 1 << 20)
        assert ei.value.status == code, (descs[0].K, B)
    fused = [_desc(xq=None, xd=None, x=512, g=768)]
    for ws, nbytes, code in ((0, 0, q.Q4Q8_E_ARG),            # fp32 rows need a workspace
                             (1 << 20, 2048 + 255, q.Q4Q8_E_ARG),  # too small
                             ((1 << 20) + 8, 4096, q.Q4Q8_E_ALIGN)):
        with pytest.raises(q.Q4Q8Error) as ei:
            _build(fused, 1, ws, nbytes)
        assert ei.value.status == code


def test_group_prologue_lds_sized_by_prologue_inputs_only():
    """A tiled group mixing an fp32-row product (K = 4096) with a Q8-plane
    product of very long K: the prologue pass quantises only the former, so
    its LDS is sized by max_prologue_k = 4096, not by max_k (2^20 here would
    ask for several hundred KiB of LDS and fail the whole call)."""
    big = _desc(K=1 << 20, M=16)
    rows = _desc(xq=None, xd=None, x=512, g=768, K=4096, M=128)
    _, plan = _build([big, rows], 64, 1 << 20, 1 << 20)
    assert plan.max_k == 1 << 20 and plan.max_prologue_k == 4096 and plan.n_prologue == 1
    _, plan = _build([_desc(K=4096)], 64)
    assert plan.max_prologue_k == 0 and plan.n_prologue == 0


def _mfma_bins(image, plan):
    """Per-bin window lists of a multi-column plan: [(product qs, window within it, K)] per bin,
    after checking the records, the map and the bounds against each other."""
    n, W, G = plan.n_records, plan.n_windows, plan.mfma_grid
    assert plan.mfma_columns == 1 and 1 <= G <= W
    assert plan.map_offset == n * 96
    assert plan.prologue_offset == (plan.map_offset + 4 * (W + G + 1) + 15) // 16 * 16
    recs = image[:plan.map_offset].view(np.int32).reshape(n, 24)
    ptrs = image[:plan.map_offset].view(np.int64).reshape(n, 12)
    words = image[plan.map_offset:plan.map_offset + 4 * (W + G + 1)].view(np.int32)
    wmap, bounds = words[:W], words[W:]
    # records in launch order, each a run of consecutive windows
    assert recs[0, 18] == 0 and (recs[1:, 18] == np.cumsum(recs[:-1, 19])).all() and recs[:, 19].sum() == W
    assert (wmap == np.repeat(np.arange(n), recs[:, 19])).all()
    assert bounds[0] == 0 and bounds[-1] == W and (np.diff(bounds) >= 0).all()
    windows = []
    for r in range(n):
        windows += [(int(ptrs[r, 0]), int(recs[r, 21]) + j, int(recs[r, 15])) for j in range(recs[r, 19])]
    return [windows[bounds[g]:bounds[g + 1]] for g in range(G)]


def test_group_build_multicolumn_packs_windows():
    """B = 5..8 groups on the multi-column route: the host packs the windows
    (64 rows each, cost K / 32) into one bin per workgroup.  Every window of
    every product is listed once; for eight Llama-3-8B-shaped layers the bins
    come out exactly equal (two down-projection windows and six of K = 4096,
    or thirteen of K = 4096: 1664 each), where contiguous cost shares of the
    caller's order leave up to 1792."""
    shapes = [(4096, 4096), (1024, 4096), (1024, 4096), (4096, 4096), (14336, 4096), (14336, 4096), (4096, 14336)]
    descs, products = [], {}
    for l in range(8):
        for i, (M, K) in enumerate(shapes):
            qs = 4096 * (1 + 7 * l + i)
            descs.append(_desc(M=M, K=K, qs=qs))
            products[qs] = (M, K)
    image, plan = _build(descs, 8)
    bins = _mfma_bins(image, plan)
    listed = sorted((qs, w) for b in bins for (qs, w, _) in b)
    assert listed == sorted((qs, w) for qs, (M, K) in products.items() for w in range((M + 63) // 64))
    for b in bins:
        for qs, w, K in b:
            assert products[qs][1] == K
    costs = [sum(K // 32 for (_, _, K) in b) for b in bins]
    total = sum(costs)
    if plan.mfma_grid == 512:
        assert max(costs) == min(costs) == total // 512 == 1664
    assert max(costs) <= -(-total // plan.mfma_grid) + 448
    # a product's windows keep their order within each record
    assert plan.n_records < 2 * plan.mfma_grid + len(descs)


@pytest.mark.parametrize("seed", range(6))
def test_group_build_multicolumn_random_groups(seed):
    """Random groups of Q4 or Q8_0 products: every window listed once, and no
    bin above the mean bin cost by more than one window of the costliest K."""
    rng = np.random.default_rng(seed)
    wf = q.WEIGHTS_Q8_0 if seed % 2 else 0
    kq = 128 if wf else 256
    descs, products = [], {}
    for i in range(int(rng.integers(1, 40))):
        M = int(rng.integers(1, 20000))
        K = kq * int(rng.integers(1024 // kq, 60))
        qs = 4096 * (i + 1)
        descs.append(_desc(M=M, K=K, qs=qs, flags=wf))
        products[qs] = (M, K)
    image, plan = _build(descs, int(rng.integers(5, 9)))
    bins = _mfma_bins(image, plan)
    listed = sorted((qs, w) for b in bins for (qs, w, _) in b)
    assert listed == sorted((qs, w) for qs, (M, K) in products.items() for w in range((M + 63) // 64))
    costs = [sum(K // 32 for (_, _, K) in b) for b in bins]
    kmax = max(K for (M, K) in products.values()) // 32
    assert max(costs) <= -(-sum(costs) // plan.mfma_grid) + kmax


@pytest.mark.parametrize("shapes,B", [([(1, 1024)], 8), ([(64, 1024)], 5), ([(65, 4096), (3, 1024)], 6),
                                      ([(130000, 1024)], 8), ([(640, 16384), (64, 1024)] * 3, 7)])
def test_group_build_multicolumn_edges(shapes, B):
    """Packing at the edges: one window (one workgroup), fewer windows than
    resident workgroups (one window each), ragged last windows, and a single
    product of many windows (equal bins)."""
    descs = [_desc(M=M, K=K, qs=4096 * (i + 1)) for i, (M, K) in enumerate(shapes)]
    image, plan = _build(descs, B)
    bins = _mfma_bins(image, plan)
    n_win = sum((M + 63) // 64 for M, _ in shapes)
    assert plan.n_windows == n_win and plan.mfma_grid == min(n_win, plan.mfma_grid)
    listed = sorted((qs, w) for b in bins for (qs, w, _) in b)
    assert listed == sorted((4096 * (i + 1), w) for i, (M, _) in enumerate(shapes) for w in range((M + 63) // 64))
    costs = [sum(K // 32 for (_, _, K) in b) for b in bins]
    if n_win <= plan.mfma_grid:
        # as many workgroups as windows: no bin above the costliest window
        assert max(costs) == max(K for _, K in shapes) // 32
    assert max(costs) <= -(-sum(costs) // plan.mfma_grid) + max(K for _, K in shapes) // 32


def test_group_build_multicolumn_many_distinct_k():
    """More distinct window costs than the packer searches (300 products, each
    its own K): the bins are filled greedily, every window still listed once."""
    descs = [_desc(M=64 + 64 * (i % 5), K=1024 + 256 * i, qs=4096 * (i + 1)) for i in range(300)]
    image, plan = _build(descs, 8)
    bins = _mfma_bins(image, plan)
    listed = sorted((qs, w) for b in bins for (qs, w, _) in b)
    assert listed == sorted((d.qs, w) for d in descs for w in range((d.M + 63) // 64))


def test_group_launch_rejects_foreign_plans():
    L = q.lib()
    plan = q.GroupPlan()
    assert L.mul_mat_q4q8_group(ctypes.c_void_p(256), ctypes.byref(plan), None) == q.Q4Q8_E_ARG
    _, good = _build([_desc()], 1)
    assert L.mul_mat_q4q8_group(None, ctypes.byref(good), None) == q.Q4Q8_E_ARG
    assert L.mul_mat_q4q8_group(ctypes.c_void_p(264), ctypes.byref(good), None) == q.Q4Q8_E_ALIGN
    for field, value in (("n_windows", 0), ("max_k", 40), ("table_bytes", 12), ("n_prologue", 5), ("B", 70000),
                         ("max_prologue_k", 64)):
        bad = q.GroupPlan.from_buffer_copy(good)
        setattr(bad, field, value)
        assert L.mul_mat_q4q8_group(ctypes.c_void_p(256), ctypes.byref(bad), None) == q.Q4Q8_E_ARG, field
    # the multi-column route's workgroup count must lie in [1, n_windows], and is 0 elsewhere
    _, mc = _build([_desc(M=4096, K=4096)], 8)
    for value in (0, mc.n_windows + 1):
        bad = q.GroupPlan.from_buffer_copy(mc)
        bad.mfma_grid = value
        assert L.mul_mat_q4q8_group(ctypes.c_void_p(256), ctypes.byref(bad), None) == q.Q4Q8_E_ARG, value
    bad = q.GroupPlan.from_buffer_copy(good)
    bad.mfma_grid = 1
    assert L.mul_mat_q4q8_group(ctypes.c_void_p(256), ctypes.byref(bad), None) == q.Q4Q8_E_ARG


def test_fused_single_validation():
    L = q.lib()
    p = ctypes.c_void_p(256)
    f = ctypes.c_float(1e-5)
    # g missing without Q8_NO_NORM; misaligned x; too large for the folded-in prologue
    assert L.mul_mat_q4q8_rmsnorm(p, p, 8, 64, p, None, f, 0, 1, p, None) == q.Q4Q8_E_ARG
    assert L.mul_mat_q4q8_rmsnorm(p, p, 8, 64, ctypes.c_void_p(260), p, f, 0, 1, p, None) == q.Q4Q8_E_ALIGN
    assert L.mul_mat_q4q8_rmsnorm(p, p, 8, 16384, p, p, f, 0, 4, p, None) == q.Q4Q8_E_UNSUPPORTED
    assert L.mul_mat_q4q8_rmsnorm(p, p, 8, 64, p, p, f, 0, 5, p, None) == q.Q4Q8_E_UNSUPPORTED  # B <= 4
    assert L.mul_mat_q4q8_rmsnorm(p, p, 8, 64, p, p, f, 2, 1, p, None) == q.Q4Q8_E_ARG


def test_q8_0_entry_points_validate():
    L = q.lib()
    # K not a multiple of 32, negative sizes
    assert L.q8_0_quantize(_v(256), 4, 48, _v(256), _v(256), None) == q.Q4Q8_E_ARG
    assert L.q8_0_quantize(_v(256), -1, 64, _v(256), _v(256), None) == q.Q4Q8_E_ARG
    assert L.mul_mat_q8_0_q8(_v(256), _v(256), 4, 33, _v(256), _v(256), 1, _v(256), None) == q.Q4Q8_E_ARG
    assert L.mul_mat_q8_0_q8(_v(256), _v(256), 4, 64, _v(256), _v(256), -2, _v(256), None) == q.Q4Q8_E_ARG
    # a grid past 2^31 workgroups is refused on the host
    assert L.q8_0_quantize(_v(256), 1 << 30, 1 << 14, _v(256), _v(256), None) == q.Q4Q8_E_ARG
    assert L.q4_quantize(_v(256), 1 << 30, 1 << 14, _v(256), _v(256), None) == q.Q4Q8_E_ARG
    assert "too large" in q.q4q8_last_error()
    # null pointers
    assert L.q8_0_quantize(None, 4, 64, _v(256), _v(256), None) == q.Q4Q8_E_ARG
    assert L.mul_mat_q8_0_q8(None, _v(256), 4, 64, _v(256), _v(256), 1, _v(256), None) == q.Q4Q8_E_ARG
    assert L.mul_mat_q8_0_q8_blocksums(_v(256), _v(256), 4, 64, _v(256), _v(256), 1, _v(256), None,
                                       None) == q.Q4Q8_E_ARG
    # misaligned weight codes (16-byte rule) and scales (2-byte rule)
    assert L.q8_0_quantize(_v(256), 4, 64, _v(264), _v(256), None) == q.Q4Q8_E_ALIGN
    assert L.q8_0_quantize(_v(256), 4, 64, _v(256), _v(257), None) == q.Q4Q8_E_ALIGN
    assert L.mul_mat_q8_0_q8(_v(264), _v(256), 4, 64, _v(256), _v(256), 1, _v(256), None) == q.Q4Q8_E_ALIGN
    assert L.mul_mat_q8_0_q8_blocksums(_v(256), _v(256), 4, 64, _v(256), _v(256), 1, _v(256), _v(258),
                                       None) == q.Q4Q8_E_ALIGN
    # empty products are no-ops
    assert L.mul_mat_q8_0_q8(None, None, 0, 64, None, None, 3, None, None) == q.Q4Q8_OK
    assert L.mul_mat_q8_0_q8_blocksums(None, None, 5, 64, None, None, 0, None, None, None) == q.Q4Q8_OK
    assert L.q8_0_quantize(None, 0, 64, None, None, None) == q.Q4Q8_OK


def test_q8_0_binding_checks_shapes():
    import torch
    qw = torch.zeros((4, 64), dtype=torch.int8)
    d = torch.zeros((4, 2), dtype=torch.int16)
    xq = torch.zeros((2, 96), dtype=torch.int8)
    xd = torch.zeros((2, 3), dtype=torch.float32)
    with pytest.raises(ValueError):
        q.mul_mat_q8_0_q8(qw, d, xq, xd)
    with pytest.raises((TypeError, ValueError)):
        q.mul_mat_q8_0_q8(qw.to(torch.uint8), d, xq[:, :64].contiguous(), xd[:, :2].contiguous())
