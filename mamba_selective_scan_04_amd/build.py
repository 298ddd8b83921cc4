"""Build step of the HIP library: compiles csrc/bdssm.hip for gfx950 into
libbdssm.so next to this file (in-tree, so it travels with the source tree).

    python -m mamba_selective_scan_04_amd.build
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "bdssm.hip")
DEPS = [SRC, os.path.join(HERE, "csrc", "bdssm_kernels.hpp"), os.path.join(HERE, "csrc", "bdssm_bwd_kernels.hpp"),
        os.path.join(ROOT, "include", "bdssm.h")]
LIB = os.path.join(HERE, "libbdssm.so")
ARCH = os.environ.get("BDSSM_ARCH", "gfx950")

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=" + ARCH, "-fPIC", "-shared",
    # keep the compiler from forming packed fp32 instructions (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    p = os.path.join(rocm, "bin", "hipcc")
    return p if os.path.exists(p) else "hipcc"


def up_to_date():
    return os.path.exists(LIB) and all(os.path.getmtime(LIB) >= os.path.getmtime(d) for d in DEPS)


def build(verbose=False):
    """Always compiles (the build check must exercise the compiler)."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc()] + HIPCC_FLAGS + ["-I", os.path.join(ROOT, "include"), "-o", tmp, SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the packed-fp32 feature and says so; drop that line
    out = "\n".join(l for l in r.stdout.splitlines() if "not a recognized feature" not in l)
    if r.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError("hipcc failed (%d):\n%s" % (r.returncode, out))
    if out.strip() and verbose:
        print(out)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    print("built", LIB)
    sys.exit(0)
