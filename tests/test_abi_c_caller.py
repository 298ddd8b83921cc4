"""The contract's C prototypes compile against include/bdssm.h unchanged:
tests/c/abi_caller.c assigns each of the five scan entry points and the
three helpers to a pointer of the contract's type (gcc -Werror), links
libbdssm.so and runs calls that the host checks reject (no GPU needed)."""
import os
import shutil
import subprocess

import pytest

import mamba_selective_scan_04_amd as m

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIP_INC = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("gcc") is None or not os.path.isdir(os.path.join(HIP_INC, "hip")),
                    reason="needs gcc and the HIP headers")
def test_contract_prototypes_compile_and_link(tmp_path):
    lib_dir = os.path.dirname(m.LIB_PATH)
    exe = str(tmp_path / "abi_caller")
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(ROOT, "include"), "-I", HIP_INC,
                    os.path.join(ROOT, "tests", "c", "abi_caller.c"), "-o", exe,
                    "-L", lib_dir, "-lbdssm", "-Wl,-rpath," + lib_dir],
                   check=True, capture_output=True, text=True)
    out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout
    got = dict(line.split(" ", 1) for line in out.strip().splitlines())
    assert int(got["version"]) == m.version()
    # the plain workspace query serves prefill, train_scan and full_scan
    n = int(got["workspace_65536"])
    for op in (m.OP_PREFILL, m.OP_TRAIN, m.OP_FULL):
        assert n >= m.workspace_bytes(8, 1536, 65536, op)
    assert n == max(m.workspace_bytes(8, 1536, 65536, op) for op in (m.OP_PREFILL, m.OP_TRAIN, m.OP_FULL))
    assert got["workspace_bad"] == "1"
    assert int(got["prefill_null"]) == -1
    assert int(got["prefill_shape"]) == -2
    assert int(got["block_step_null"]) == -1
    assert int(got["commit_shape"]) == -2
    assert int(got["train_scan_shape"]) == -2      # T % L != 0
    assert int(got["full_scan_empty"]) == 0
    assert got["status_ok"] == "ok"
