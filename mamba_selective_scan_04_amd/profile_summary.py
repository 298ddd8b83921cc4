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

Only this library's kernels (bdssm_dev::) and the calibration copy are listed.
The summary starts with the source hash of the kernels so a stale profile can
be recognised.
"""
import collections
import csv
import hashlib
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
# every kernel and launch source: a change to any of them marks a summary stale
KERNEL_SOURCES = sorted(os.path.join(HERE, "csrc", f) for f in os.listdir(os.path.join(HERE, "csrc"))
                        if f.endswith((".hip", ".hpp")))
COPY_BYTES = 1 << 30


def source_hash():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def short(name):
    n = name.split("(")[0]
    return n.replace("void ", "").replace("bdssm_dev::", "").replace("unsigned short", "bf16")


def keep(name):
    return "bdssm_dev::" in name or "copyBuffer" in name


def trace(path):
    groups = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        if not keep(r["Kernel_Name"]):
            continue
        grid = (int(r["Grid_Size_X"]), int(r["Grid_Size_Y"]), int(r["Grid_Size_Z"]))
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        groups[(short(r["Kernel_Name"]), grid)].append(dur)
    out = ["kernel source hash: %s" % source_hash(), "",
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


def pmc(fetch_path, write_path):
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
    out = ["kernel source hash: %s" % source_hash(), "",
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


def valu(path):
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
    out = ["kernel source hash: %s" % source_hash(), "",
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
    if len(argv) >= 2 and argv[0] == "trace":
        print(trace(argv[1]))
    elif len(argv) >= 3 and argv[0] == "pmc":
        print(pmc(argv[1], argv[2]))
    elif len(argv) >= 2 and argv[0] == "valu":
        print(valu(argv[1]))
    elif len(argv) >= 1 and argv[0] == "hash":
        print(source_hash())
    else:
        print(__doc__)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
