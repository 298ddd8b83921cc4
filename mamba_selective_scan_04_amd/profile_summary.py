"""Condense rocprofv3 CSV output into the short text summaries kept under
profiles/.

  python -m mamba_selective_scan_04_amd.profile_summary trace <kernel_trace.csv>
      per (kernel, grid) launch group: calls, average / min / max duration
  python -m mamba_selective_scan_04_amd.profile_summary valu <counter_collection.csv>
      per (kernel, grid): the clock the dies ran at and the VALU issue rate from
      GRBM_GUI_ACTIVE, SQ_INSTS_VALU, SQ_INSTS_VALU_TRANS_F32, SQ_ACTIVE_INST_VALU
  python -m mamba_selective_scan_04_amd.profile_summary pmc <FETCH counter_collection.csv> \
      <WRITE counter_collection.csv>
      per (kernel, grid): FETCH_SIZE and WRITE_SIZE per dispatch, raw (KiB) and
      scaled to bytes by what the same counter reads for a plain device copy of
      known size (the 1 GiB copyBuffer launches of bench.py --copy-calibration)

  python -m mamba_selective_scan_04_amd.profile_summary hash [family]
      the source hash of a kernel family (prefill, bidir, backward, train)
      or of every source

Only this library's kernels (bdssm_dev::) and the calibration copy are listed.
A summary starts with the source hash of the kernel family it measures, so
that a stale profile can be recognised: the hash covers the shared device
helpers, the family's kernels and their launch and plan code, and nothing
else, so that work on one family leaves the others' profiles valid.
"""
import collections
import csv
import hashlib
import os
import re
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
KERNEL_SOURCES = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                        if f.endswith((".hip", ".hpp")) and not f.startswith("roof_probe"))
COPY_BYTES = 1 << 30
# the definitions each profiled family depends on (kernels, launchers, plans)
_BIDIR = ("chunk_scan_body", "chunk_state_kernel", "carry_kernel", "carry_tree_kernel", "bidir_pair_kernel", "pair_scatter", "bidir_wave_kernel",
          "block_lane_kernel", "make_plan", "plan_long", "pair_long_capacity", "blocks_plan", "plan_for",
          "pair_path", "pair_long", "pair_bidir", "launch_chunk_state_k", "launch_chunk_state", "launch_carry",
          "launch_pair_k", "launch_pair_L", "launch_pair", "launch_bidir_k", "launch_bidir_L", "launch_bidir",
          "launch_block_lane", "block_lane_path", "run_bidirectional", "layout_ws")
_BACKWARD = ("bwd_pair_kernel", "bwd_wave_kernel", "adjoint_chunk_kernel", "adjoint_general_kernel",
             "group_state_kernel", "bwd_general_kernel", "carry_kernel", "carry_tree_kernel", "bc_reduce_kernel", "param_reduce_kernel",
             "fold16", "fold32", "make_plan", "blocks_plan", "plan_general", "bwd_plan", "bwd_blocks_plan",
             "bwd_use_wave", "bwd_general", "bwd_long", "bwd_channels", "bwd_block_channels",
             "bwd_block_capacity", "layout_bwd", "launch_bwd_L", "launch_bwd_n", "launch_bwd", "launch_bwd_long",
             "launch_bwd_reduce", "launch_adjoint_chunk_k", "launch_adjoint_chunk", "launch_adjoint_general",
             "launch_bwd_general")
FAMILIES = {
    "prefill": ("chunk_scan_body", "chunk_state_kernel", "carry_kernel", "carry_tree_kernel", "make_plan", "plan_for", "launch_chunk_state_k",
                "launch_chunk_state", "launch_carry", "run_state_only", "layout_ws"),
    "bidir": _BIDIR,
    "backward": _BACKWARD,
    # the training step: the forward passes, the backward and the baseline's sweeps
    "train": tuple(dict.fromkeys(_BIDIR + _BACKWARD + ("sweep_output_kernel", "chunk_both_kernel", "launch_chunk_both",
                                                        "run_full"))),
}


def _definitions(text, name):
    """The text of every definition of `name` in a source: from its template
    line (if any) to the first closing brace in column 0."""
    lines = text.split("\n")
    out = []
    i = 0
    while i < len(lines):
        l = lines[i]
        if l[:1] not in ("", " ", "/", "#", "}") and re.search(r"\b%s\(" % re.escape(name), l):
            j = i
            while j < len(lines) and not lines[j].rstrip().endswith(("{", ";")):
                j += 1
            if j < len(lines) and lines[j].rstrip().endswith("{"):
                k0 = i - 1 if i > 0 and lines[i - 1].startswith("template") else i
                k = j
                while k < len(lines) and lines[k] != "}":
                    k += 1
                out.append("\n".join(lines[k0:k + 1]))
                i = k
        i += 1
    return out


def source_hash(family=None):
    """Hash of every kernel and launch source (family None), or of one
    family's definitions plus the shared device helpers (the kernel header up
    to its first kernel)."""
    h = hashlib.sha256()
    if family is None:
        for p in KERNEL_SOURCES:
            with open(p, "rb") as f:
                h.update(f.read())
        return h.hexdigest()[:16]
    texts = [open(p).read() for p in KERNEL_SOURCES]
    kern = open(os.path.join(CSRC, "bdssm_kernels.hpp")).read()
    h.update(kern[:kern.index("__global__")].encode())
    for name in FAMILIES[family]:
        found = [d for t in texts for d in _definitions(t, name)]
        if not found:
            raise KeyError("no definition of %s in the sources" % name)
        for d in found:
            h.update(d.encode())
    return h.hexdigest()[:16]


def hash_line(family):
    if family is None:
        return "kernel source hash: %s" % source_hash()
    return "kernel source hash (%s): %s" % (family, source_hash(family))


def short(name):
    n = name.split("(")[0]
    return n.replace("void ", "").replace("bdssm_dev::", "").replace("unsigned short", "bf16")


def keep(name):
    return "bdssm_dev::" in name or "copyBuffer" in name


def trace(path, family=None):
    groups = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        if not keep(r["Kernel_Name"]):
            continue
        grid = (int(r["Grid_Size_X"]), int(r["Grid_Size_Y"]), int(r["Grid_Size_Z"]))
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        groups[(short(r["Kernel_Name"]), grid)].append(dur)
    out = [hash_line(family), "",
           "| kernel | grid (threads x,y,z) | calls | avg us | min us | max us |",
           "|---|---|---:|---:|---:|---:|"]
    for (k, g), v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        out.append("| %s | %s | %d | %.2f | %.2f | %.2f |" % (k, "x".join(map(str, g)), len(v),
                                                           sum(v) / len(v), min(v), max(v)))
    return "\n".join(out)


def _counters(path):
    groups = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        if not keep(r["Kernel_Name"]):
            continue
        groups[(short(r["Kernel_Name"]), int(r["Grid_Size"]))].append(float(r["Counter_Value"]))
    return groups


def pmc(fetch_path, write_path, family=None):
    f = _counters(fetch_path)
    w = _counters(write_path)
    # the calibration copies are the copyBuffer launch group that writes the most
    copies = [key for key in w if "copyBuffer" in key[0]]
    if not copies:
        raise SystemExit("no calibration copy in the counter files (run bench.py --copy-calibration)")
    ckey = max(copies, key=lambda k: sum(w[k]) / len(w[k]))
    cf, cw = f.get(ckey, []), w[ckey]
    if not cf or not cw:
        raise SystemExit("no calibration copy in the counter files (run bench.py --copy-calibration)")
    sf = COPY_BYTES / (sum(cf) / len(cf) * 1024)
    sw = COPY_BYTES / (sum(cw) / len(cw) * 1024)
    out = [hash_line(family), "",
           "calibration: a 1 GiB device copy reads FETCH_SIZE %.0f KiB and WRITE_SIZE %.0f KiB per "
           "dispatch, so bytes = FETCH_SIZE x 1024 x %.4f and WRITE_SIZE x 1024 x %.4f"
           % (sum(cf) / len(cf), sum(cw) / len(cw), sf, sw), "",
           "| kernel | grid (threads) | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | read bytes | write bytes |",
           "|---|---:|---:|---:|---:|---:|---:|"]
    for key in sorted(set(f) | set(w), key=lambda k: -sum(f.get(k, [0]))):
        if "copyBuffer" in key[0]:
            continue
        fv, wv = f.get(key, []), w.get(key, [])
        fa = sum(fv) / len(fv) if fv else float("nan")
        wa = sum(wv) / len(wv) if wv else float("nan")
        out.append("| %s | %d | %d | %.1f | %.1f | %.4g | %.4g |" % (
            key[0], key[1], max(len(fv), len(wv)), fa, wa, fa * 1024 * sf, wa * 1024 * sw))
    return "\n".join(out)


N_XCC = 8             # MI355X: GRBM_GUI_ACTIVE is summed over its 8 accelerator dies
N_CU = 256
VALU_LANES = 1024 * 16   # 256 CUs x 4 SIMDs x 16 lanes: lane issue slots per clock
NOMINAL_GHZ = 2.4


def valu(path, family=None):
    """Per kernel launch group: duration, the clock the dies ran at
    (GRBM_GUI_ACTIVE / N_XCC / duration), VALU instructions issued (a v_exp
    counts twice, as it occupies the SIMD for twice the cycles), the lane issue
    slots per second that makes, and that rate against the nominal 2.4 GHz peak
    and against the peak at the measured clock; VALUBusy as rocprofv3 defines it."""
    rows = collections.defaultdict(dict)
    for r in csv.DictReader(open(path)):
        if not keep(r["Kernel_Name"]):
            continue
        key = (int(r["Dispatch_Id"]), short(r["Kernel_Name"]), int(r["Grid_Size"]),
               (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        rows[key][r["Counter_Name"]] = float(r["Counter_Value"])
    groups = collections.defaultdict(list)
    for (disp, name, grid, us), c in rows.items():
        groups[(name, grid)].append((us, c))
    out = [hash_line(family), "",
           "| kernel | grid (threads) | dispatches | avg us | clock GHz | VALU instr (v_exp x2) | "
           "lane slots / s | of 2.4 GHz peak | of peak at measured clock | VALUBusy % |",
           "|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|"]
    for (name, grid), v in sorted(groups.items(), key=lambda kv: -sum(u for u, _ in kv[1])):
        if "copyBuffer" in name:
            continue
        us = sum(u for u, _ in v) / len(v)
        get = lambda k: sum(c.get(k, 0.0) for _, c in v) / len(v)
        cyc = get("GRBM_GUI_ACTIVE") / N_XCC
        ghz = cyc / (us * 1e3) if us > 0 else float("nan")
        instr = get("SQ_INSTS_VALU") + get("SQ_INSTS_VALU_TRANS_F32")
        rate = instr * 64 / (us * 1e-6) if us > 0 else float("nan")
        peak = VALU_LANES * NOMINAL_GHZ * 1e9
        peak_clk = VALU_LANES * ghz * 1e9
        busy = 100 * get("SQ_ACTIVE_INST_VALU") / N_CU / cyc if cyc > 0 else float("nan")
        out.append("| %s | %d | %d | %.2f | %.3f | %.4g | %.4g | %.3f | %.3f | %.1f |" % (
            name, grid, len(v), us, ghz, instr, rate, rate / peak, rate / peak_clk, busy))
    return "\n".join(out)


def main(argv):
    fam = None
    if "--family" in argv:
        i = argv.index("--family")
        fam = argv[i + 1]
        argv = argv[:i] + argv[i + 2:]
    if len(argv) >= 2 and argv[0] == "trace":
        print(trace(argv[1], fam))
    elif len(argv) >= 3 and argv[0] == "pmc":
        print(pmc(argv[1], argv[2], fam))
    elif len(argv) >= 2 and argv[0] == "valu":
        print(valu(argv[1], fam))
    elif len(argv) >= 1 and argv[0] == "hash":
        print(source_hash(argv[1] if len(argv) > 1 else None))
    else:
        print(__doc__)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
