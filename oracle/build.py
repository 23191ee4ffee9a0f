"""Builds the CPU oracle (test infrastructure only) with gcc.

The oracle is plain single-threaded C99 compiled for IEEE binary32 semantics:
SSE arithmetic, no contraction into fused multiply-adds, no fast-math.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "nvfp4_oracle.c")
# The multi-threaded driver of the CPU baseline (calls the oracle's functions).
SRC_MT = os.path.join(HERE, "nvfp4_oracle_mt.c")
LIB = os.path.join(HERE, "libnvfp4_oracle.so")

CFLAGS = ["-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-Wall", "-Wextra"]
# AddressSanitizer + UndefinedBehaviorSanitizer build of the same source (CPU
# only), for running the oracle's pins under the sanitizers.  Loading it into
# Python needs libasan preloaded (see sanitizer_env()).
SAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=undefined"]


def build(extra_flags=(), out=LIB):
    """Compile the oracle into a shared library; returns its path."""
    cmd = ["gcc", *CFLAGS, *extra_flags, "-pthread", "-shared", "-o", out, SRC, SRC_MT, "-lm"]
    subprocess.run(cmd, check=True, cwd=HERE)
    return out


def build_sanitized(out):
    """Compile the oracle with ASan and UBSan into `out`; returns its path."""
    return build(SAN_FLAGS, out)


def sanitizer_env(lib_path):
    """Environment for a child Python that loads the sanitized oracle."""
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], check=True,
                          capture_output=True, text=True).stdout.strip()
    env = dict(os.environ)
    env["LD_PRELOAD"] = asan
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["NVFP4_ORACLE_LIB"] = lib_path
    return env


if __name__ == "__main__":
    print(build())
