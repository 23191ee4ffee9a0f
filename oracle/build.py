"""Builds the CPU oracle (test infrastructure only) with gcc.

The oracle is plain single-threaded C99 compiled for IEEE binary32 semantics:
SSE arithmetic, no contraction into fused multiply-adds, no fast-math.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "nvfp4_oracle.c")
LIB = os.path.join(HERE, "libnvfp4_oracle.so")

CFLAGS = ["-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-Wall", "-Wextra"]


def build(extra_flags=(), out=LIB):
    """Compile the oracle into a shared library; returns its path."""
    cmd = ["gcc", *CFLAGS, *extra_flags, "-shared", "-o", out, SRC, "-lm"]
    subprocess.run(cmd, check=True, cwd=HERE)
    return out


if __name__ == "__main__":
    print(build())
