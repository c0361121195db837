"""Build ``libq4q8.so`` (gfx950 only) in-tree with hipcc.

All HIP code is compiled without FMA contraction (the quantisation kernels
must reproduce single-rounded fp32 steps; the matmul kernels use explicit
fma builtins where they want fused operations) and with packed fp32 vector
ops disabled.  Each source compiles to its own object in parallel (device
code is not relocatable across sources: every kernel is launched from the
source that defines it), then the objects are linked into the library.
"""
from __future__ import annotations

import glob
import os
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB_PATH = os.path.join(HERE, "libq4q8.so")
ROOT = os.path.dirname(HERE)

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++20",
    "-fPIC",
    "-fvisibility=hidden",
    "-ffp-contract=off",
    "-fno-gpu-rdc",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-result",
]

# hipcc's host pass does not know the packed-fp32 feature; that warning is harmless.
_NOISE = "'-packed-fp32-ops' is not a recognized feature"


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _run(cmd: list[str]) -> str:
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if _NOISE not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + out)
    return out


def build(verbose: bool = False) -> str:
    """Compile every kernel source and link ``libq4q8.so`` (always recompiles)."""
    srcs = sources()
    jobs = max(1, min(len(srcs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with tempfile.TemporaryDirectory(prefix="q4q8_build_") as tmpdir:
        objs = [os.path.join(tmpdir, os.path.basename(s) + ".o") for s in srcs]
        cmds = [[HIPCC, *COMMON, "-I", os.path.join(ROOT, "include"), "-c", s, "-o", o]
                for s, o in zip(srcs, objs)]
        with ThreadPoolExecutor(max_workers=jobs) as pool:
            outs = list(pool.map(_run, cmds))
        tmp = LIB_PATH + ".tmp%d" % os.getpid()
        link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
        outs.append(_run(link))
    if verbose:
        for c in cmds:
            print(" ".join(c), flush=True)
        print(" ".join(link), flush=True)
        text = "\n".join(o for o in outs if o.strip())
        if text:
            print(text)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
