"""Compile the HIP sources into the in-tree shared library (gfx950 only).

Flags that matter for exactness: -ffp-contract=off (no silent a*b+c fusion;
fused multiply-adds appear only where the source writes them), no fast-math
and no flush-to-zero (fp32 denormals are preserved), and packed-fp32 code
generation disabled.
"""
import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libnvfp4.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def build(out=LIB, extra=()):
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    cmd = [hipcc, *HIPCC_FLAGS, *extra, "-I", os.path.join(ROOT, "include"), *sources(), "-o", out]
    subprocess.run(cmd, check=True, cwd=HERE)
    return out


if __name__ == "__main__":
    print(build())
