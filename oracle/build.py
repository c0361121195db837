"""Build the oracle shared library with gcc (host code only, no FMA contraction).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "q4q8_oracle.c")
LIB_PATH = os.path.join(HERE, "liboracle_q4q8.so")
SAN_LIB_PATH = os.path.join(HERE, "liboracle_q4q8_san.so")

CFLAGS = ["-O2", "-std=gnu11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
          "-Wall", "-Wextra", "-pthread"]


def build(verbose: bool = False) -> str:
    """Compile ``q4q8_oracle.c`` into ``liboracle_q4q8.so`` (always recompiles)."""
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


# AddressSanitizer + UndefinedBehaviorSanitizer build of the same source; the
# test suite loads it in a child process with gcc's libasan preloaded
SAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=undefined"]


def build_sanitized(verbose: bool = False) -> str:
    """Compile ``q4q8_oracle.c`` into ``liboracle_q4q8_san.so`` (always recompiles)."""
    tmp = SAN_LIB_PATH + ".tmp%d" % os.getpid()
    flags = [f for f in CFLAGS if f != "-O2"] + SAN_FLAGS
    cmd = ["gcc", *flags, SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, SAN_LIB_PATH)
    return SAN_LIB_PATH


def asan_runtime() -> str:
    """gcc's libasan, which the sanitizer build needs loaded first."""
    out = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True, check=True)
    return out.stdout.strip()


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_sanitized(verbose=True))
