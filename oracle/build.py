"""Build the oracle shared library with gcc (host code only, no FMA contraction).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "q4q8_oracle.c")
LIB_PATH = os.path.join(HERE, "liboracle_q4q8.so")

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


if __name__ == "__main__":
    print(build(verbose=True))
