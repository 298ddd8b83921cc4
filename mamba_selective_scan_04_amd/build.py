"""Build step of the HIP library: compiles the sources under csrc/ for gfx950
and links libbdssm.so next to this file (in-tree, so it travels with the
source tree).

    python -m mamba_selective_scan_04_amd.build            # everything
    python -m mamba_selective_scan_04_amd.build --changed  # only objects older than their sources

The kernel launchers live in launch_*.hip; each is compiled twice, once per
stream type (-DBDSSM_TIN=float and -DBDSSM_TIN=uint16_t, the bf16 bits), so
that the template instantiations spread over parallel compiler processes.
bdssm.hip holds the C ABI and the launch plans.  Objects go to _build/.
libbdssm_probe.so (csrc/roof_probe.hip) holds the benchmark's
microbenchmarks; it is not part of the scan library.

The compiler's resource report of every kernel (registers, spills, scratch,
LDS, waves per SIMD) goes to _build/<object>.resources.tsv, one line per
kernel; tests/test_resources.py checks the hot kernels' lines (no spills,
the occupancy their design assumes).
"""
import concurrent.futures
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
HEADERS = [os.path.join(CSRC, h) for h in ("bdssm_kernels.hpp", "bdssm_bwd_kernels.hpp", "bdssm_launch.hpp")] + [
    os.path.join(ROOT, "include", "bdssm.h")]
LAUNCH_UNITS = ("launch_chunk", "launch_bidir", "launch_block", "launch_bwd", "launch_bwd_general")
STREAM_TYPES = (("f32", "float"), ("bf16", "uint16_t"))
LIB = os.path.join(HERE, "libbdssm.so")
PROBE_LIB = os.path.join(HERE, "libbdssm_probe.so")
PROBE_SRC = os.path.join(CSRC, "roof_probe.hip")
PROBE_OBJ = os.path.join(BUILD_DIR, "roof_probe.o")
ARCH = os.environ.get("BDSSM_ARCH", "gfx950")

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=" + ARCH, "-fPIC",
    # keep the compiler from forming packed fp32 instructions (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    # per-kernel register / LDS / occupancy report (collected by _resources)
    "-Rpass-analysis=kernel-resource-usage", "-fno-caret-diagnostics",
]


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    p = os.path.join(rocm, "bin", "hipcc")
    return p if os.path.exists(p) else "hipcc"


def units():
    """(source, object, extra flags) of every translation unit."""
    out = [(os.path.join(CSRC, "bdssm.hip"), os.path.join(BUILD_DIR, "bdssm.o"), [])]
    for u in LAUNCH_UNITS:
        for tag, ctype in STREAM_TYPES:
            out.append((os.path.join(CSRC, u + ".hip"), os.path.join(BUILD_DIR, "%s.%s.o" % (u, tag)),
                        ["-DBDSSM_TIN=" + ctype]))
    return out


def sources():
    return sorted({s for s, _, _ in units()}) + HEADERS + [PROBE_SRC]


def up_to_date():
    return os.path.exists(LIB) and all(os.path.getmtime(LIB) >= os.path.getmtime(d) for d in sources())


def _clean(out):
    # the host pass does not know the packed-fp32 feature and says so; drop
    # that line, and the resource remarks (kept in the .resources.tsv files)
    # with the include chains that introduce them
    keep, chain = [], []
    for l in out.splitlines():
        if l.startswith("In file included from"):
            chain.append(l)
            continue
        if "remark:" in l or "not a recognized feature" in l:
            chain = []
            continue
        keep += chain + [l]
        chain = []
    return "\n".join(keep + chain)


RESOURCE_FIELDS = (("VGPRs", "vgprs"), ("AGPRs", "agprs"), ("VGPRs Spill", "vgpr_spill"),
                   ("ScratchSize [bytes/lane]", "scratch"), ("Occupancy [waves/SIMD]", "waves"),
                   ("LDS Size [bytes/block]", "lds"))


def _resources(out):
    """The kernel-resource-usage remarks of one compiler run -> tsv text:
    kernel (mangled), then the RESOURCE_FIELDS values."""
    rows, cur = [], None
    for line in out.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = {"name": m.group(1)}
            rows.append(cur)
            continue
        m = re.search(r"remark:\s+([^:\[]+(?:\[[^\]]*\])?): (-?\d+)", line)
        if m and cur is not None:
            cur[m.group(1).strip()] = m.group(2)
    head = "kernel\t" + "\t".join(k for _, k in RESOURCE_FIELDS)
    return "\n".join([head] + ["\t".join([r["name"]] + [r.get(f, "") for f, _ in RESOURCE_FIELDS])
                               for r in rows if r["name"].startswith("_Z")]) + "\n"


def _compile(src, obj, extra):
    tmp = obj + ".tmp%d" % os.getpid()
    cmd = [hipcc()] + HIPCC_FLAGS + extra + ["-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c", "-o", tmp, src]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = _clean(r.stdout)
    if r.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError("hipcc failed (%d) on %s:\n%s\n%s" % (r.returncode, os.path.basename(obj), " ".join(cmd), out))
    with open(obj + ".resources.tsv", "w") as f:
        f.write(_resources(r.stdout))
    os.replace(tmp, obj)
    return out


def build(verbose=False, changed_only=False, jobs=None):
    """Compiles every translation unit (all of them unless changed_only, which
    skips objects newer than their source and every header) and links the
    library."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    todo = []
    for src, obj, extra in units() + [(PROBE_SRC, PROBE_OBJ, [])]:
        if changed_only and os.path.exists(obj):
            t = os.path.getmtime(obj)
            if all(os.path.getmtime(d) <= t for d in [src] + HEADERS):
                continue
        todo.append((src, obj, extra))
    jobs = jobs or min(len(todo) or 1, os.cpu_count() or 4, 12)
    if verbose:
        print("compiling %d of %d translation units with %d jobs" % (len(todo), len(units()) + 1, jobs),
              flush=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = {ex.submit(_compile, *t): t for t in todo}
        for fu in concurrent.futures.as_completed(futs):
            out = fu.result()
            if verbose:
                print("  built", os.path.basename(futs[fu][1]), flush=True)
                if out.strip():
                    print(out)
    _link(LIB, [o for _, o, _ in units()])
    _link(PROBE_LIB, [PROBE_OBJ])
    return LIB


def _link(lib, objs):
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError("link of %s failed (%d):\n%s" % (os.path.basename(lib), r.returncode, _clean(r.stdout)))
    os.replace(tmp, lib)


if __name__ == "__main__":
    build(verbose=True, changed_only="--changed" in sys.argv[1:])
    print("built", LIB)
    sys.exit(0)
