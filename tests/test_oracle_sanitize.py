"""The oracle's C code under AddressSanitizer and UBSan (host code only):
the oracle is built with -fsanitize=address,undefined and every oracle pin
(forward, gradients, fusions) runs against that build in a child process with
the ASan runtime preloaded.  Any out-of-bounds access, use after free,
signed overflow or other undefined behaviour aborts the child."""
import os
import subprocess
import sys

import pytest

import oracle
from oracle import oracle as oracle_mod

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    r = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_pins_under_sanitizers(tmp_path):
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("gcc's ASan runtime is not installed")
    lib = oracle_mod.build(sanitize=True, out=str(tmp_path / "liboracle_asan.so"))
    env = dict(os.environ, LD_PRELOAD=rt, BDSSM_ORACLE_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1",
               OMP_NUM_THREADS="4")
    # the child really runs the sanitized build with the ASan runtime
    probe = subprocess.run([sys.executable, "-c", "import oracle; oracle.load(); "
                            "m = open('/proc/self/maps').read(); "
                            "print(int('libasan' in m), int('liboracle_asan' in m))"],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert probe.stdout.split() == ["1", "1"], probe.stdout + probe.stderr[-2000:]
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
           "tests/test_oracle.py", "tests/test_oracle_bwd.py", "tests/test_oracle_fused.py"]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out, out[-2000:]
