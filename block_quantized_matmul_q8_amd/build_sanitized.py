"""Build ``libq4q8_san.so``: the library with its host code (argument
validation, group plans, routing set-up, launch logic) compiled with
AddressSanitizer and UndefinedBehaviorSanitizer.

Only host code is instrumented: every sanitizer flag is given to hipcc as
``-Xarch_host`` followed by the flag, so the gfx950 device code is the same
as in ``libq4q8.so``.  The test suite loads this library on the CPU, in a
child process with the clang ASan runtime preloaded
(tests/test_sanitizers.py); it is never used on a GPU.
"""
from __future__ import annotations

import glob
import os
import tempfile
from concurrent.futures import ThreadPoolExecutor

from .build import COMMON, HERE, HIPCC, ROOT, _run, sources

SAN_LIB_PATH = os.path.join(HERE, "libq4q8_san.so")

# each host-only: -Xarch_host directly before every sanitizer option
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-shared-libasan"]


def asan_runtime() -> str:
    """Path of the clang ASan runtime that the instrumented host code needs."""
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise FileNotFoundError("libclang_rt.asan-x86_64.so not found under /opt/rocm/llvm")
    return hits[-1]


def build_sanitized() -> str:
    """Compile every source (the C ABI source with host sanitizers) and link
    ``libq4q8_san.so`` (always recompiles)."""
    srcs = sources()
    jobs = max(1, min(len(srcs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    inc = ["-I", os.path.join(ROOT, "include")]
    with tempfile.TemporaryDirectory(prefix="q4q8_san_") as tmpdir:
        objs = [os.path.join(tmpdir, os.path.basename(s) + ".o") for s in srcs]
        cmds = []
        for s, o in zip(srcs, objs):
            extra = ["-g", *HOST_SAN] if os.path.basename(s) == "api.hip" else []
            cmds.append([HIPCC, *COMMON, *extra, *inc, "-c", s, "-o", o])
        with ThreadPoolExecutor(max_workers=jobs) as pool:
            list(pool.map(_run, cmds))
        tmp = SAN_LIB_PATH + ".tmp%d" % os.getpid()
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs,
              "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
              "-Xarch_host", "-shared-libasan", "-o", tmp])
    os.replace(tmp, SAN_LIB_PATH)
    return SAN_LIB_PATH


if __name__ == "__main__":
    print(build_sanitized())
