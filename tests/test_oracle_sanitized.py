"""The oracle's pins, rerun against an AddressSanitizer + UndefinedBehavior-
Sanitizer build of the same C source (CPU only).

The oracle is plain C that indexes arrays by hand (blocks, transposes,
channel gathers, the GEMM's nibble and scale lookups); a stray index or an
overflowing shift would still leave most pins passing.  Here the oracle is
compiled with -fsanitize=address,undefined (halting on the first report),
loaded into a child Python with libasan preloaded, and every oracle pin file
runs against it.  Any sanitizer report fails the child and this test.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PIN_FILES = ["test_oracle_formats.py", "test_oracle_worked_facts.py", "test_oracle_tensor.py",
             "test_oracle_residual.py", "test_oracle_rmsnorm.py", "test_oracle_gemm.py"]


def test_oracle_pins_pass_under_asan_and_ubsan(tmp_path):
    sys.path.insert(0, ROOT)
    from oracle import build as ob

    lib = ob.build_sanitized(str(tmp_path / "liboracle_asan.so"))
    env = ob.sanitizer_env(lib)
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p", "no:cacheprovider", "-m",
           "not gpu and not slow", *[os.path.join(ROOT, "tests", f) for f in PIN_FILES]]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out, out[-2000:]


def test_sanitized_library_is_the_one_loaded(tmp_path):
    """The override really swaps the library (so the test above exercises
    the sanitized build, not the plain one)."""
    sys.path.insert(0, ROOT)
    from oracle import build as ob

    lib = ob.build_sanitized(str(tmp_path / "liboracle_asan.so"))
    env = ob.sanitizer_env(lib)
    code = ("import oracle, sys; oracle.lib(); "
            "maps = open('/proc/self/maps').read(); "
            f"sys.exit(0 if {lib!r} in maps else 3)")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
