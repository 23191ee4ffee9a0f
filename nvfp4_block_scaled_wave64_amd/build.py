"""Compile the HIP sources into the in-tree shared library (gfx950 only).

Flags that matter for exactness: -ffp-contract=off (no silent a*b+c fusion;
fused multiply-adds appear only where the source writes them), no fast-math
and no flush-to-zero (fp32 denormals are preserved), and packed-fp32 code
generation disabled.

Every translation unit launches only its own kernels, so the sources compile
to objects independently (in parallel) and one link makes the library.
"""
import glob
import hashlib
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libnvfp4.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def _hipcc():
    return os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")


CACHE = os.path.join(HERE, "_build")


def _key(src, flags):
    """Hash of a source, every header it may include, and the flags."""
    h = hashlib.sha256()
    h.update(repr(flags).encode())
    headers = sorted(glob.glob(os.path.join(HERE, "csrc", "*.h")) +
                     glob.glob(os.path.join(ROOT, "include", "*.h")))
    for f in [src, *headers]:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:24]


def build(out=LIB, extra=(), jobs=None, incremental=False):
    """Compile every csrc/*.hip and link them into `out`; returns its path.

    With incremental=True, objects whose source, headers and flags are
    unchanged are reused from _build/ (a developer convenience; the default
    always recompiles everything).
    """
    hipcc = _hipcc()
    srcs = sources()
    jobs = jobs or max(1, min(len(srcs), os.cpu_count() or 1, 16))
    with tempfile.TemporaryDirectory(prefix="nvfp4_build_") as tmp:
        def compile_one(src):
            flags = [*HIPCC_FLAGS, *extra]
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            cached = os.path.join(CACHE, os.path.basename(src) + "." + _key(src, flags) + ".o")
            if incremental and os.path.exists(cached):
                return cached
            cmd = [hipcc, *flags, "-I", os.path.join(ROOT, "include"), "-c", src, "-o", obj]
            subprocess.run(cmd, check=True, cwd=HERE)
            os.makedirs(CACHE, exist_ok=True)
            shutil.copyfile(obj, cached)
            return obj

        with ThreadPoolExecutor(max_workers=jobs) as ex:
            objs = list(ex.map(compile_one, srcs))
        tmp_out = out + ".tmp"
        subprocess.run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs,
                        "-o", tmp_out], check=True, cwd=HERE)
        os.replace(tmp_out, out)
    return out


if __name__ == "__main__":
    print(build(incremental="--incremental" in sys.argv[1:]))
