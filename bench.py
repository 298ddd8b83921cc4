#!/usr/bin/env python3
"""Benchmark of the block-restricted bidirectional selective scan on one MI355X.

Default run (`python bench.py`): the headline workload infer_65k_b8, then every
other workload of the scan at its full size under "configs".

One headline step = one pass of the inference hot path over one batch of
synthetic, device-resident input (65,536-token context, batch 8, d_inner 1536):
    prefill of the clean context (forward scan, cache written)
    then, for each of n_blocks blocks: 16 denoising block steps (forward from
    the cache + in-block reverse + output) and one commit (cache advanced).
The prefill is launched eagerly; each block's 16 block steps + commit are
replayed from a captured HIP graph (one graph per block: the launches are
identical every step, so capture removes only host launch overhead).

Printed: one JSON line on stdout (progress goes to stderr).
  value        whole-step algorithmic HBM throughput (GB/s): bytes every call
               in the step must move (inputs read once, outputs written once,
               states read or written once) / measured step time
  roofline     the dominant launch (the prefill: chunk-local forward scan +
               its carry), timed with HIP events on its stream.  It is bound
               by the fp32 VALU: "achieved" / "peak" count VALU issue slots
               (mul / FMA one, v_exp_f32 two) against 256 CUs x 4 SIMDs x 16
               lanes x 2.4 GHz; beside it the graded HBM fraction (frac_hbm),
               the fraction of the published fp32 peak (frac_fp32_published,
               FMA = 2 flop, exp = 1), and the probed rates of this chip
  max_rel_err  the timed step's outputs (prefill state, last block step's y,
               committed state) against the fp64 oracle on sampled channels
  cpu_baseline the fp64 CPU oracle timed on a bounded sample of the same step
  configs      the other workloads (65K b1, 262K b1 / b4 / b16, the 87M and
               350M training shapes), each with its times, algorithmic GB/s,
               HBM and issue-slot fractions, errors against the oracle and an
               oracle time extrapolated from sampled channels
  roof_probe   the probed FMA, exp2 and scan-mix issue rates and the HBM read
               bandwidth of this chip (libbdssm_probe.so)

Training workloads (--workload train_87m | train_350m) time the all-block
training scan, the two-stream form, the backward passes and the full-sequence
scan instead.  --crossover sweeps the context length from 8K to 64K tokens;
--model-loop runs the scan inside a random-weight stand-in Mamba stack
(context only); --roof-probe prints the microbenchmarks alone.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--no-configs] [--crossover] [--model-loop] [--roof-probe]
"""
import argparse
import ctypes
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# fp32 VALU issue slots per second: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz
VALU_SLOTS_PER_S = 256 * 4 * 16 * 2.4e9
# MI355X's published fp32 vector peak (packed FMA: 2 flop x 2 lanes per slot)
FP32_PUBLISHED_FLOPS = 157.3e12
EXP_SLOTS = 2            # v_exp_f32 issues at half rate on gfx950 (probe_exp)
# dt = softplus(dt_raw + bias) per (token, channel): bias add, |v| scale, exp2
# (2), 1 + w, log2 (2), ln 2 scale, u - 1, rcp (2), two muls, compare, select,
# max, add
SOFTPLUS_SLOTS = 17
NS = 16
STATE_TOL = 1e-4
CONFIG_WORKLOADS = ("infer_65k_b1", "infer_65k_b8", "infer_262k_b1", "infer_262k_b4", "infer_262k_b16",
                    "train_87m", "train_350m")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------ algorithmic cost

def bytes_prefill(batch, T, D, e, h_init=False):
    return batch * T * D * 2 * e + batch * T * NS * e + 4 * D * NS + 4 * batch * D * NS * (2 if h_init else 1)


def bytes_block_step(batch, L, D, e):
    return batch * L * D * 3 * e + batch * L * NS * 2 * e + 4 * D * NS + 4 * D + 4 * batch * D * NS


def bytes_commit(batch, L, D, e):
    return batch * L * D * 2 * e + batch * L * NS * e + 4 * D * NS + 2 * 4 * batch * D * NS


def bytes_full(batch, T, D, e, ns=NS):
    return batch * T * D * 3 * e + batch * T * ns * 2 * e + 4 * D * ns + 4 * D


def bytes_backward(batch, T, D, e, L, ns=NS, blocks=False):
    """x, dt, dy, B, C in; dx, ddt, dB, dC out; the block states read (and,
    two-stream form, their gradients written); A, Dskip in, dA, dDskip out."""
    nb = batch * (T // L + 1) * D * ns * 4
    return (batch * T * D * 5 * e + batch * T * ns * 4 * e + 2 * (4 * D * ns + 4 * D)
            + nb * (2 if blocks else 1))


def slots_forward(batch, T, D):
    """exp2 (2 slots) + dt*A' mul + (dt*x)*B mul + state FMA per (b,t,d,n),
    plus the dt*x multiply per (b,t,d)."""
    return batch * T * D * (NS * (EXP_SLOTS + 3) + 1)


def flops_forward(batch, T, D):
    """The same operations counted as flops: exp2 1, mul 1, FMA 2 -> 5 per
    (b,t,d,n) plus the dt*x multiply."""
    return batch * T * D * (NS * 5 + 1)


def slots_backward(batch, T, D, ns=NS):
    """Algorithmic issue slots of the backward pass per (b,t,d,n): one exp2 (2)
    and dt*A' (1); the forward state (u, FMA), the reverse state (FMA), the
    forward adjoint (FMA, mul), the reverse adjoint (FMA, mul); du (add), da
    (FMA, mul), the dt / x / A sums (FMA, mul, FMA, FMA), dB (mul), dC (FMA,
    add, mul): 22; plus 4 per (b,t,d) for the dt and x gradients."""
    return batch * T * D * (ns * 22 + 4)


def slots_bidirectional(batch, T, D, ns=NS):
    """forward + in-block reverse + output: exp2 + 2 mul + 4 FMA per
    (b,t,d,n), plus dt*x and the Dskip*x FMA per (b,t,d)."""
    return batch * T * D * (ns * (EXP_SLOTS + 6) + 2)


def committed_traffic(workload, batch, D):
    """HBM bytes per prefill (chunk scan + carry) from the committed counter
    summary for this workload, or None if there is none or the kernels have
    changed since it was taken (source hash mismatch)."""
    from mamba_selective_scan_04_amd import profile_summary
    path = os.path.join(ROOT, "profiles", "prefill_%s_hbm_traffic.md" % workload.replace("infer_", ""))
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    if profile_summary.hash_line("prefill") not in txt:
        return None
    chunk, carry = None, None
    carry_grid = (batch * D * NS + 255) // 256 * 256
    for line in txt.splitlines():
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) != 7:
            continue
        try:
            grid, rd, wr = int(cells[1]), float(cells[5]), float(cells[6])
        except ValueError:
            continue
        if re.fullmatch(r"chunk_state_kernel<\w+, false, false(, 0)?(, 16)?>", cells[0]):
            if chunk is None or grid > chunk[0]:
                chunk = (grid, rd + wr)
        if cells[0] == "carry_kernel<false>" and grid == carry_grid:
            carry = rd + wr
    if chunk is None or carry is None:
        return None
    return chunk[1] + carry


def committed_clock(workload):
    """Clock and issue figures of the prefill's chunk scan from the committed VALU
    counter summary for this workload, or None if there is none or the kernels
    have changed since it was taken. Every figure comes from that one counter
    run: its clock, VALUBusy, kernel average and issue fraction at its clock."""
    from mamba_selective_scan_04_amd import profile_summary
    path = os.path.join(ROOT, "profiles", "prefill_%s_valu_counters.md" % workload.replace("infer_", ""))
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    if profile_summary.hash_line("prefill") not in txt:
        return None
    best = None
    for line in txt.splitlines():
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) != 10 or not re.fullmatch(r"chunk_state_kernel<\w+, false, false, 0, 16>", cells[0]):
            continue
        try:
            grid, us, ghz, frac, busy = (int(cells[1]), float(cells[3]), float(cells[4]), float(cells[8]),
                                         float(cells[9]))
        except ValueError:
            continue
        if best is None or grid > best[0]:
            best = (grid, {"clock_GHz": ghz, "valu_busy_pct": busy, "kernel_us": us,
                           "slot_frac_at_its_clock": frac})
    return None if best is None else best[1]


# ------------------------------------------------------------ microbenchmarks

class Probe:
    """libbdssm_probe.so: launch-rate and issue-rate microbenchmarks."""

    def __init__(self, torch):
        path = os.path.join(ROOT, "mamba_selective_scan_04_amd", "libbdssm_probe.so")
        if not os.path.exists(path):
            raise ImportError("libbdssm_probe.so not built: run `python -m mamba_selective_scan_04_amd.build`")
        self.lib = ctypes.CDLL(path)
        P, I = ctypes.c_void_p, ctypes.c_int
        self.lib.probe_fma.argtypes = [P, I, I, P]
        self.lib.probe_exp.argtypes = [P, I, I, P]
        self.lib.probe_mix.argtypes = [P, P, P, I, I, P]
        self.lib.probe_read.argtypes = [P, ctypes.c_int64, P, I, P]
        self.lib.probe_empty.argtypes = [I, I, I, I, P]
        self.torch = torch

    def stream(self):
        return ctypes.c_void_p(self.torch.cuda.current_stream().cuda_stream)

    def empty(self, gx, gy, gz, block):
        rc = self.lib.probe_empty(gx, gy, gz, block, self.stream())
        if rc != 0:
            raise RuntimeError("probe_empty failed (%d)" % rc)


def time_calls(torch, fn, reps):
    """Average ms per call of fn over reps calls, HIP events on the current stream."""
    st = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fn()
    torch.cuda.synchronize()
    a.record(st)
    for _ in range(reps):
        fn()
    b.record(st)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def run_probes(torch, probe):
    """Issue rates (FMA, exp2, the forward scan's op mix) and HBM read and
    copy bandwidth, each the best of a few launches."""
    dev = "cuda:0"
    lib = probe.lib
    grid = 256 * 4 * 8            # 8 waves per SIMD (256-lane workgroups: 4 waves each) x 2
    out = torch.zeros(grid * 256, device=dev)
    iters = 4096

    def best(fn, reps=3):
        return min(time_calls(torch, fn, 1) for _ in range(reps))

    ms = best(lambda: lib.probe_fma(ctypes.c_void_p(out.data_ptr()), grid, iters, probe.stream()))
    fma_rate = grid * 256 * iters * 8 / (ms * 1e-3)
    ms = best(lambda: lib.probe_exp(ctypes.c_void_p(out.data_ptr()), grid, iters, probe.stream()))
    exp_rate = grid * 256 * iters * 8 / (ms * 1e-3)
    A = -(torch.arange(1, 17, device=dev, dtype=torch.float32)) * 1.4426950408889634
    Bv = torch.randn(16, device=dev)
    mgrid = 256 * 4 * 8           # one-wave workgroups: 8 waves per SIMD, as chunk_state_kernel
    mix_iters = 2048
    ms = best(lambda: lib.probe_mix(ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(A.data_ptr()),
                                    ctypes.c_void_p(Bv.data_ptr()), mgrid, mix_iters, probe.stream()))
    mix_elems = mgrid * 64 * mix_iters * 16 / (ms * 1e-3)
    src = torch.empty(1 << 30, dtype=torch.float32, device=dev).fill_(1.0)   # 4 GiB
    ms = best(lambda: lib.probe_read(ctypes.c_void_p(src.data_ptr()), src.numel() // 4,
                                     ctypes.c_void_p(out.data_ptr()), grid, probe.stream()))
    read_GBs = src.numel() * 4 / (ms * 1e-3) / 1e9
    dst = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    srcc = src[: 1 << 28]
    ms = best(lambda: dst.copy_(srcc))
    copy_GBs = 2 * dst.numel() * 4 / (ms * 1e-3) / 1e9
    del src, dst, srcc, out
    torch.cuda.empty_cache()
    return {
        "fma_T_per_s": fma_rate / 1e12,
        "fma_frac_of_slot_peak": fma_rate / VALU_SLOTS_PER_S,
        "exp2_T_per_s": exp_rate / 1e12,
        "exp2_slots": fma_rate / exp_rate,
        "scan_mix_T_elements_per_s": mix_elems / 1e12,
        "scan_mix_slot_frac": mix_elems * (NS * (EXP_SLOTS + 3) + 1) / NS / VALU_SLOTS_PER_S,
        "hbm_read_GBs": read_GBs,
        "hbm_copy_GBs": copy_GBs,
        "note": "fma / exp2: 8 independent chains per lane, 8192 workgroups of 256 lanes; scan mix: "
                "per (token, state) dt*A' mul, exp2, (dt*x)*B mul, state FMA, 16 states per lane, "
                "8192 one-wave workgroups; read: 4 GiB float4 sum; copy: 1 GiB device copy (read + "
                "write counted); best of 3 launches each",
    }


# ------------------------------------------------------------ the oracle leg
#
# The errors of the timed runs against the fp64 oracle and the oracle's own
# time (the CPU baseline).  The oracle recomputes sampled channels' rows from
# the same device-resident inputs (rows are independent, so a subset of
# channels is an exact sub-problem of the prefill, the block steps, the
# commits and the per-channel gradients); channel-summed gradients (dB, dC)
# are recomputed over every channel of batch row 0.

def err_metrics(got, ref, bar):
    """max |g - r| / max(|r|, floor) with the floor at rms(r) (the parity
    tests' metric) and at 0.01 rms(r), and the normwise max |g - r| / max |r|."""
    import numpy as np
    g = np.asarray(got, np.float64)
    r = np.asarray(ref, np.float64)
    rms = float(np.sqrt(np.mean(r * r))) + 1e-300
    d = np.abs(g - r)
    return {"rel_rms_floor": float(np.max(d / np.maximum(np.abs(r), rms))),
            "rel_0.01rms_floor": float(np.max(d / np.maximum(np.abs(r), 0.01 * rms))),
            "normwise": float(np.max(d) / max(float(np.max(np.abs(r))), 1e-300)),
            "bar": bar}


def sample_channels(D, k, seed):
    import numpy as np
    g = np.random.default_rng(seed)
    ch = np.sort(g.choice(D, size=min(k, D), replace=False))
    ch[0] = 0
    ch[-1] = D - 1
    return ch


def n_sample_channels(batch, threads):
    """Channels to sample: at least 8, and enough rows for every oracle thread."""
    return max(8, -(-threads // batch))


def worst_of(errs):
    return max(v["rel_rms_floor"] for v in errs.values())


def oracle_leg_inference(torch, synth, x, dt, Bm, Cm, A, Dskip, steps_in, commit_in, L, h_pf, y_last, h_fin,
                         ytol, step_bytes, seed):
    """Errors of one step's outputs (prefill state, the last block step's y,
    the final committed state) against the oracle on sampled channels, and the
    oracle's time for the whole step on those channels, extrapolated to all."""
    import oracle
    oracle.load()
    batch, ctx, D = x.shape
    threads = oracle.num_threads()
    ch = sample_channels(D, n_sample_channels(batch, threads), seed)
    idx = torch.as_tensor(ch, device=x.device)
    to = synth.to_oracle
    g = lambda t: to(t.index_select(2, idx))
    xo, dto, Bo, Co = g(x), g(dt), to(Bm), to(Cm)
    Ao, Do = to(A.index_select(0, idx)), to(Dskip.index_select(0, idx))
    so = [(g(s[0]), g(s[1]), to(s[2]), to(s[3])) for s in steps_in]
    co = [(g(c[0]), g(c[1]), to(c[2]), to(c[3])) for c in commit_in]
    t0 = time.perf_counter()
    ho, _ = oracle.prefill(xo, dto, Bo, Co, Ao, Do, L)
    h = ho
    yo = None
    for k in range(len(co)):
        for s in so:
            yo = oracle.block_step(h, *s, Ao, Do)
        h, _ = oracle.commit(h, *co[k], Ao, Do)
    spent = time.perf_counter() - t0
    to_np = lambda t: t.detach().float().cpu().numpy()
    errs = {
        "prefill_state": err_metrics(to_np(h_pf.index_select(1, idx)), ho, STATE_TOL),
        "block_step_y": err_metrics(to_np(y_last.index_select(2, idx)), yo, ytol),
        "commit_state": err_metrics(to_np(h_fin.index_select(1, idx)), h, STATE_TOL),
    }
    full_s = spent * D / len(ch)
    cpu = {"value": step_bytes / full_s / 1e9, "unit": "GB/s", "cores": min(threads, batch * len(ch)),
           "kind": "oracle", "extrapolated": True, "seconds_sample": spent, "seconds_step_extrapolated": full_s,
           "sample": "%d of %d channels, every batch row (%d rows): prefill, %d x (%d block steps + commit); "
                     "time scaled by channel count" % (len(ch), D, batch * len(ch), len(co), len(so))}
    return errs, cpu


def oracle_leg_training(torch, synth, x, dt, Bm, Cm, A, Dskip, L, dy, y_c, bnd, y_n, gn, gc, ytol, step_bytes,
                        seed):
    """The all-block training step's outputs against the oracle: clean y and
    block states, noisy y (from the oracle's own block states), the noisy and
    clean gradients per channel on sampled channels, dB and dC on batch row 0
    over every channel; and the oracle's time for the step on the sampled
    channels, extrapolated to all."""
    import oracle
    oracle.load()
    batch, T, D = x.shape
    threads = oracle.num_threads()
    ch = sample_channels(D, n_sample_channels(batch, threads), seed)
    idx = torch.as_tensor(ch, device=x.device)
    to = synth.to_oracle
    to_np = lambda t: t.detach().float().cpu().numpy()
    g = lambda t: to(t.index_select(2, idx))
    args = (g(x), g(dt), to(Bm), to(Cm), to(A.index_select(0, idx)), to(Dskip.index_select(0, idx)))
    dyo = to_np(dy.index_select(2, idx)).astype("float64")
    t0 = time.perf_counter()
    r = oracle.scan(*args, L, want_y=True, want_bounds=True)
    yn = oracle.train_blocks(*args, L, r["bounds"])
    rn = oracle.scan_bwd(*args, L, dyo, h0_blocks=r["bounds"])
    rc = oracle.scan_bwd(*args, L, dyo, dbounds=rn["dh0_blocks"])
    spent = time.perf_counter() - t0
    errs = {"clean_y": err_metrics(to_np(y_c.index_select(2, idx)), r["y"], ytol),
            "clean_bounds": err_metrics(to_np(bnd.index_select(2, idx)), r["bounds"], STATE_TOL),
            "noisy_y": err_metrics(to_np(y_n.index_select(2, idx)), yn, ytol)}
    for tag, gg, rr, hk, hr in (("noisy", gn, rn, "dh0_blocks", "dh0_blocks"), ("clean", gc, rc, "dh_init", "dh0")):
        for k in ("dx", "ddt"):
            errs["%s_%s" % (tag, k)] = err_metrics(to_np(gg[k].index_select(2, idx)), rr[k], ytol)
        errs["%s_dA" % tag] = err_metrics(to_np(gg["dA"].index_select(0, idx)), rr["dA"], STATE_TOL)
        errs["%s_dDskip" % tag] = err_metrics(to_np(gg["dDskip"].index_select(0, idx)), rr["dDskip"], STATE_TOL)
        hs = gg[hk].index_select(gg[hk].dim() - 2, idx)
        errs["%s_%s" % (tag, hr)] = err_metrics(to_np(hs), rr[hr], STATE_TOL)
    # dB, dC sum over every channel: batch row 0, all channels
    a0 = (to(x[:1]), to(dt[:1]), to(Bm[:1]), to(Cm[:1]), to(A), to(Dskip))
    dy0 = to_np(dy[:1]).astype("float64")
    r0 = oracle.scan(*a0, L, want_y=False, want_bounds=True)
    rn0 = oracle.scan_bwd(*a0, L, dy0, h0_blocks=r0["bounds"])
    rc0 = oracle.scan_bwd(*a0, L, dy0, dbounds=rn0["dh0_blocks"])
    for tag, gg, rr in (("noisy", gn, rn0), ("clean", gc, rc0)):
        for k in ("dB", "dC"):
            errs["%s_%s_row0" % (tag, k)] = err_metrics(to_np(gg[k][:1]), rr[k], ytol)
    full_s = spent * D / len(ch)
    cpu = {"value": step_bytes / full_s / 1e9, "unit": "GB/s", "cores": min(threads, batch * len(ch)),
           "kind": "oracle", "extrapolated": True, "seconds_sample": spent, "seconds_step_extrapolated": full_s,
           "sample": "%d of %d channels, every batch row (%d rows): the all-block step (clean scan with "
                     "block states, noisy two-stream scan, both backward passes); time scaled by channel "
                     "count" % (len(ch), D, batch * len(ch))}
    return errs, cpu


def cpu_baseline(x, dt, Bm, Cm, A, Dskip, steps_in, commit_in, L, target_s, e):
    """Time the oracle (as it stands) on batch rows 0..k-1 of the step:
    prefill of the whole context, the block steps and the commits, all
    channels.  k grows until about target_s seconds of wall time."""
    import oracle
    from mamba_selective_scan_04_amd import synth

    oracle.load()
    batch, ctx, D = x.shape
    to = synth.to_oracle
    Ah, Dh = to(A), to(Dskip)
    spent = 0.0
    rows = 0
    sample_bytes = 0
    for b in range(batch):
        xb, dtb, Bb, Cb = (to(t[b:b + 1]) for t in (x, dt, Bm, Cm))
        sb = [tuple(to(t[b:b + 1]) for t in s) for s in steps_in]
        cb = [tuple(to(t[b:b + 1]) for t in c) for c in commit_in]
        t0 = time.perf_counter()
        hcache, _ = oracle.prefill(xb, dtb, Bb, Cb, Ah, Dh, L)
        for k in range(len(cb)):
            for s in sb:
                oracle.block_step(hcache, *s, Ah, Dh)
            hcache, _ = oracle.commit(hcache, *cb[k], Ah, Dh)
        spent += time.perf_counter() - t0
        rows += 1
        sample_bytes += (bytes_prefill(1, ctx, D, e)
                         + len(cb) * (len(sb) * bytes_block_step(1, L, D, e) + bytes_commit(1, L, D, e)))
        log("[bench] cpu oracle: batch row %d done, %.1f s so far" % (b, spent))
        if spent >= target_s:
            break
    return {"value": sample_bytes / spent / 1e9, "unit": "GB/s", "cores": min(oracle.num_threads(), D),
            "kind": "oracle", "extrapolated": False,
            "sample": "batch rows 0..%d of %d (all %d channels): prefill of %d tokens + the "
                      "block steps and commits; %.1f s wall" % (rows - 1, batch, D, ctx, spent),
            "seconds": spent}


# ------------------------------------------------------------ inference

def run_inference(name, opts, m, synth, torch, probe, steps, warmup, cpu_rows_baseline=False):
    """One inference workload: prefill + n_blocks x (16 block steps + commit),
    timed as whole steps and call by call; the full-sequence baseline over the
    context; the last step's outputs against the oracle.  -> dict."""
    wl = dict(synth.WORKLOADS[name])
    batch, D, ctx, L = wl["batch"], wl["d_inner"], wl["ctx"], wl["block"]
    S, nblk, sid = wl["steps"], wl["n_blocks"], wl["sid"]
    dtype = synth.TORCH_DTYPE[wl["dtype"]]
    e = 2 if dtype == torch.bfloat16 else 4
    dev = "cuda:0"
    st = torch.cuda.current_stream()
    fused, rev_ops = bool(getattr(opts, "fused", False)), bool(getattr(opts, "reverse_operands", False))

    log("[bench] workload %s: batch %d, d_inner %d, ctx %d, block %d, %d steps x %d blocks"
        % (name, batch, D, ctx, L, S, nblk))
    t_gen = time.time()
    x, dt, Bm, Cm = synth.stream(batch, ctx, D, NS, sid, 0, dtype, dev)
    A, Dskip = synth.params(D, NS, sid, "default", dev)
    steps_in = [synth.step_inputs(batch, L, D, NS, sid, j, dtype, dev) for j in range(S)]
    commit_in = [synth.commit_inputs(batch, L, D, NS, sid, k, dtype, dev) for k in range(nblk)]
    fz_pf, fz_bs = {}, {}
    if fused:
        # raw step sizes in place of dt, a per-channel bias, and the gates
        raw = lambda shape, seed: synth.normal(shape, seed, dev, dtype, mean=-1.0, std=0.5)
        dt = raw((batch, ctx, D), 1000 * sid + 70)
        steps_in = [(sx, raw((batch, L, D), 1000 * sid + 71 + j), sb, sc) for j, (sx, _, sb, sc) in enumerate(steps_in)]
        commit_in = [(cx, raw((batch, L, D), 1000 * sid + 91 + k), cb, cc) for k, (cx, _, cb, cc) in enumerate(commit_in)]
        bias = synth.normal((D,), 1000 * sid + 72, dev, torch.float32, std=0.3)
        fz_pf = dict(dt_bias=bias, dt_softplus=True)
        fz_bs = dict(fz_pf, z=synth.normal((batch, L, D), 1000 * sid + 73, dev, dtype))
    if rev_ops:
        fz_bs = dict(fz_bs, rev=reverse_operands(synth, batch, L, D, sid, dtype, dev, torch))
    h = torch.empty(batch, D, NS, dtype=torch.float32, device=dev)
    y_blk = torch.empty(batch, L, D, dtype=dtype, device=dev)
    ws = torch.empty(max(1, m.workspace_bytes(batch, D, ctx, m.OP_PREFILL, L, NS, dtype)),
                     dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    log("[bench] inputs generated on device in %.1f s" % (time.time() - t_gen))

    def prefill():
        m.prefill(x, dt, Bm, Cm, A, Dskip, L, h_cache=h, ws=ws, **fz_pf)

    def block(k):
        for j in range(S):
            m.block_step(h, *steps_in[j], A, Dskip, y=y_blk, **fz_bs)
        m.commit(h, *commit_in[k], A, Dskip, **fz_pf)

    launch = "eager"
    graphs = None
    if not getattr(opts, "eager", False):
        try:
            prefill()
            torch.cuda.synchronize()
            graphs = []
            for k in range(nblk):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    block(k)
                graphs.append(g)
            torch.cuda.synchronize()
            launch = "graph"
        except Exception as exc:       # capture unsupported: fall back to eager launches
            log("[bench] graph capture failed (%s); launching eagerly" % exc)
            graphs = None

    def run_block(k):
        if graphs is not None:
            graphs[k].replay()
        else:
            block(k)

    def step(ev=None):
        if ev is not None:
            ev[0].record(st)
        prefill()
        if ev is not None:
            ev[1].record(st)
        for k in range(nblk):
            run_block(k)
        if ev is not None:
            ev[2].record(st)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pf_ms = sum(ev[0].elapsed_time(ev[1]) for ev in evs) / steps
    blk_ms = sum(ev[1].elapsed_time(ev[2]) for ev in evs) / steps
    ms_per_step = wall * 1e3 / steps
    log("[bench] %s: timed %d steps: %.3f ms/step (prefill %.3f ms, blocks %.3f ms)"
        % (name, steps, ms_per_step, pf_ms, blk_ms))

    # the outputs of one more step, for the oracle: prefill state, the last
    # block step's y, the committed state
    prefill()
    h_pf = h.clone()
    for k in range(nblk):
        run_block(k)
    torch.cuda.synchronize()
    y_last, h_fin = y_blk.clone(), h.clone()

    # ---- per-call breakdown of the block phase (events around R replays)
    R = 50
    bs_x = [steps_in[0][i] for i in range(4)]
    hs = h.clone()
    g_bs = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_bs):
        for _ in range(R):
            m.block_step(hs, *bs_x, A, Dskip, y=y_blk, **fz_bs)
    g_cm = torch.cuda.CUDAGraph()
    hc = h.clone()
    with torch.cuda.graph(g_cm):
        for _ in range(R):
            m.commit(hc, *commit_in[0], A, Dskip, **fz_pf)
    bs_ms = time_calls(torch, g_bs.replay, 4) / R
    cm_ms = time_calls(torch, g_cm.replay, 4) / R
    bs_eager_ms = time_calls(torch, lambda: m.block_step(hs, *bs_x, A, Dskip, y=y_blk, **fz_bs), 200)
    bound = m.bind_block_step(hs, *bs_x, A, Dskip, y_blk, **fz_bs)
    bs_bound_ms = time_calls(torch, bound, 200)
    del g_bs, g_cm, bound
    # the launch floor: an empty kernel on the block step's grid (one
    # 256-lane workgroup per 64 channels and batch row), R launches in a graph
    # and eagerly
    gx = (D + 63) // 64
    g_fl = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_fl):
        for _ in range(R):
            probe.empty(gx, 1, batch, 256)
    floor_ms = time_calls(torch, g_fl.replay, 4) / R
    floor_eager_ms = time_calls(torch, lambda: probe.empty(gx, 1, batch, 256), 200)
    del g_fl

    # ---- cold block step: graphs of K x (512 MB scrub write, block step) and
    # of K x (scrub write) alone; the difference per call is the block step
    # with the cache, its inputs and A evicted from the 256 MB last-level
    # cache (the best of 5 replays of each)
    K = 20
    scrub = torch.empty(128 << 20, dtype=torch.float32, device=dev)
    g_cold = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_cold):
        for i in range(K):
            scrub.fill_(float(i))
            m.block_step(hs, *bs_x, A, Dskip, y=y_blk, **fz_bs)
    g_scrub = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_scrub):
        for i in range(K):
            scrub.fill_(float(i))

    def best_replay_ms(g, reps=5):
        return min(time_calls(torch, g.replay, 1) for _ in range(reps))

    bs_cold_ms = (best_replay_ms(g_cold) - best_replay_ms(g_scrub)) / K
    del g_cold, g_scrub, scrub

    # the fused path also reads the bias (4 D bytes per call) and the block
    # steps' gates (one element per (token, channel))
    fz_bytes_bs = (batch * L * D * e + 4 * D) if fused else 0
    if rev_ops:   # dt_r per (token, channel), B_r and C_r per token, A_r
        fz_bytes_bs += batch * L * D * e + 2 * batch * L * NS * e + 4 * D * NS
    fz_bytes_pf = 4 * D if fused else 0
    pf_bytes = bytes_prefill(batch, ctx, D, e) + fz_bytes_pf
    bs_bytes = bytes_block_step(batch, L, D, e) + fz_bytes_bs
    cm_bytes = bytes_commit(batch, L, D, e) + fz_bytes_pf
    step_bytes = pf_bytes + nblk * (S * bs_bytes + cm_bytes)
    pf_slots = slots_forward(batch, ctx, D) + (batch * ctx * D * SOFTPLUS_SLOTS if fused else 0)
    gen_tok = batch * L * nblk
    gen_ms = nblk * (S * bs_ms + cm_ms)
    res = {
        "workload": name, "batch": batch, "d_inner": D, "d_state": NS, "ctx": ctx, "block": L,
        "denoising_steps": S, "n_blocks": nblk, "launch": launch, "steps": steps, "warmup": warmup,
        "step": {"ms": ms_per_step, "bytes": step_bytes, "GBs": step_bytes / (ms_per_step * 1e-3) / 1e9,
                 "hbm_frac": step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
                 "prefill_ms_events": pf_ms, "blocks_ms_events": blk_ms},
        "prefill": {"ms": pf_ms, "tokens_per_s": batch * ctx / (pf_ms * 1e-3), "bytes": pf_bytes,
                    "GBs": pf_bytes / (pf_ms * 1e-3) / 1e9,
                    "hbm_frac": pf_bytes / (pf_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                    "slot_frac": pf_slots / (pf_ms * 1e-3) / VALU_SLOTS_PER_S,
                    "flop_frac_fp32_published": flops_forward(batch, ctx, D) / (pf_ms * 1e-3) / FP32_PUBLISHED_FLOPS},
        "block_step": {"us_graph": bs_ms * 1e3, "us_eager": bs_eager_ms * 1e3, "us_eager_bound": bs_bound_ms * 1e3,
                       "us_graph_cold": bs_cold_ms * 1e3, "bytes": bs_bytes,
                       "GBs": bs_bytes / (bs_ms * 1e-3) / 1e9,
                       "hbm_frac": bs_bytes / (bs_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                       "GBs_cold": bs_bytes / (bs_cold_ms * 1e-3) / 1e9,
                       "us_floor_empty_kernel_graph": floor_ms * 1e3,
                       "us_floor_empty_kernel_eager": floor_eager_ms * 1e3,
                       "us_over_floor": (bs_ms - floor_ms) * 1e3,
                       "note": "us_graph: 50 calls in one graph, back to back; us_eager: the plain binding "
                               "call; us_eager_bound: a BoundCall (checked and marshalled once); "
                               "us_graph_cold: graph of 20 x (512 MB scrub write + call) minus graph of 20 "
                               "scrub writes, per call; floor: an empty kernel on the block step's grid "
                               "(ceil(D/64) x batch workgroups of 256 lanes), 50 in a graph / eager"},
        "commit": {"us_graph": cm_ms * 1e3, "bytes": cm_bytes, "GBs": cm_bytes / (cm_ms * 1e-3) / 1e9},
        "generation_tokens_per_s": gen_tok / (gen_ms * 1e-3),
    }

    # ---- contrast: the full-sequence bidirectional baseline over the context
    if not getattr(opts, "no_baseline_scan", False) and not fused and not rev_ops:
        del ws
        yf = torch.empty_like(x)
        wsf = torch.empty(max(1, m.workspace_bytes(batch, D, ctx, m.OP_FULL, 1, NS, dtype)),
                          dtype=torch.uint8, device=dev)
        f_ms = time_calls(torch, lambda: m.full_scan(x, dt, Bm, Cm, A, Dskip, y=yf, ws=wsf), 3)
        base_gen = batch * L / (S * f_ms * 1e-3)
        fb = bytes_full(batch, ctx, D, e)
        res["baseline_full_scan"] = {
            "ms": f_ms, "T": ctx, "GBs": fb / (f_ms * 1e-3) / 1e9,
            "slot_frac": slots_bidirectional(batch, ctx, D) / (f_ms * 1e-3) / VALU_SLOTS_PER_S,
            "generation_tokens_per_s": base_gen,
            "speedup_block_restricted": res["generation_tokens_per_s"] / base_gen,
            "note": "one rescan of the whole context in both directions per denoising step (T = context)"}
        del yf, wsf
        log("[bench] %s: baseline full scan over %d tokens: %.3f ms" % (name, ctx, f_ms))
    else:
        del ws

    # ---- the oracle leg: errors of the last step's outputs, CPU baseline
    if not getattr(opts, "no_cpu_baseline", False) and not fused and not rev_ops:
        errs, cpu_s = oracle_leg_inference(torch, synth, x, dt, Bm, Cm, A, Dskip, steps_in, commit_in, L, h_pf,
                                           y_last, h_fin, 2e-2 if e == 2 else 1e-4, step_bytes, 17)
        res["max_rel_err"] = errs
        res["worst_rel_err"] = worst_of(errs)
        res["cpu_baseline_sampled"] = cpu_s
        log("[bench] %s: oracle check: worst rel err %.2e" % (name, res["worst_rel_err"]))
        if cpu_rows_baseline:
            res["cpu_baseline"] = cpu_baseline(x, dt, Bm, Cm, A, Dskip, steps_in, commit_in, L,
                                               getattr(opts, "cpu_seconds", 10.0), e)
    del x, dt, Bm, Cm, steps_in, commit_in, h, y_blk, hs, hc, h_pf, y_last, h_fin
    torch.cuda.empty_cache()
    return res


# ------------------------------------------------------------ training

def run_training(name, opts, m, synth, torch, steps, warmup, check=True):
    """One training workload: the all-block scan (train_scan), the two-stream
    form, both backward passes, the whole all-block step, and the
    full-sequence scan; the step's outputs against the oracle.  -> dict."""
    wl = synth.WORKLOADS[name]
    batch, D, T, L, sid = wl["batch"], wl["d_inner"], wl["seq"], wl["block"], wl["sid"]
    L = getattr(opts, "block_len", 0) or L
    ns = getattr(opts, "d_state", 0) or NS
    fused, rev_ops = bool(getattr(opts, "fused", False)), bool(getattr(opts, "reverse_operands", False))
    if T % L != 0:
        raise SystemExit("block length %d does not divide the sequence length %d" % (L, T))
    dtype = synth.TORCH_DTYPE[wl["dtype"]]
    e = 2 if dtype == torch.bfloat16 else 4
    dev = "cuda:0"
    st = torch.cuda.current_stream()
    log("[bench] workload %s: batch %d, d_inner %d, d_state %d, T %d, block %d" % (name, batch, D, ns, T, L))
    x, dt, Bm, Cm = synth.stream(batch, T, D, ns, sid, 0, dtype, dev)
    A, Dskip = synth.params(D, ns, sid, "default", dev)
    y = torch.empty_like(x)
    fz = {}
    if fused:
        dt = synth.normal((batch, T, D), 1000 * sid + 70, dev, dtype, mean=-1.0, std=0.5)
        fz = dict(dt_bias=synth.normal((D,), 1000 * sid + 72, dev, torch.float32, std=0.3),
                  dt_softplus=True, z=synth.normal((batch, T, D), 1000 * sid + 73, dev, dtype))
    if rev_ops:
        fz = dict(fz, rev=reverse_operands(synth, batch, T, D, sid, dtype, dev, torch, ns))
    ws = torch.empty(max(1, m.workspace_bytes(batch, D, T, m.OP_TRAIN, L, ns, dtype)),
                     dtype=torch.uint8, device=dev)
    wsf = torch.empty(max(1, m.workspace_bytes(batch, D, T, m.OP_FULL, 1, ns, dtype)),
                      dtype=torch.uint8, device=dev)

    def timed(fn):
        return time_calls(torch, fn, steps)

    for _ in range(warmup):
        m.train_scan(x, dt, Bm, Cm, A, Dskip, L, y=y, ws=ws, **fz)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        evs[i][0].record(st)
        m.train_scan(x, dt, Bm, Cm, A, Dskip, L, y=y, ws=ws, **fz)
        evs[i][1].record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = sum(a.elapsed_time(b) for a, b in evs) / steps
    ms_per_step = wall * 1e3 / steps
    full_ms = timed(lambda: m.full_scan(x, dt, Bm, Cm, A, Dskip, y=y, ws=wsf, **fz))
    bnd = torch.empty(batch, T // L + 1, D, ns, dtype=torch.float32, device=dev)
    m.train_scan(x, dt, Bm, Cm, A, Dskip, L, y=y, h_bounds=bnd, ws=ws, **fz)
    blocks_ms = timed(lambda: m.train_scan_blocks(x, dt, Bm, Cm, A, Dskip, L, bnd, y=y, **fz))

    def two():
        m.train_scan(x, dt, Bm, Cm, A, Dskip, L, y=y, h_bounds=bnd, ws=ws, **fz)
        m.train_scan_blocks(x, dt, Bm, Cm, A, Dskip, L, bnd, y=y, **fz)

    two_ms = timed(two)
    dy = synth.normal((batch, T, D), 1000 * sid + 8, dev, dtype)
    wsb = torch.empty(max(1, m.workspace_bytes(batch, D, T, m.OP_TRAIN_BWD_REV if rev_ops else m.OP_TRAIN_BWD,
                                               L, ns, dtype)), dtype=torch.uint8, device=dev)
    wsbb = torch.empty(max(1, m.workspace_bytes(batch, D, T, m.OP_BLOCKS_BWD_REV if rev_ops else m.OP_BLOCKS_BWD,
                                                L, ns, dtype)), dtype=torch.uint8, device=dev)
    m.train_scan(x, dt, Bm, Cm, A, Dskip, L, y=y, h_bounds=bnd, ws=ws, **fz)
    bwd_ms = timed(lambda: m.train_scan_bwd(x, dt, Bm, Cm, A, Dskip, L, bnd, dy, ws=wsb, **fz))
    bbwd_ms = timed(lambda: m.train_scan_blocks_bwd(x, dt, Bm, Cm, A, Dskip, L, bnd, dy, want_dh0_blocks=True,
                                                    ws=wsbb, **fz))
    y_c, y_n = torch.empty_like(x), torch.empty_like(x)
    out = {}

    def all_block_step():
        m.train_scan(x, dt, Bm, Cm, A, Dskip, L, y=y_c, h_bounds=bnd, ws=ws, **fz)
        m.train_scan_blocks(x, dt, Bm, Cm, A, Dskip, L, bnd, y=y_n, **fz)
        gn = m.train_scan_blocks_bwd(x, dt, Bm, Cm, A, Dskip, L, bnd, dy, want_dh0_blocks=True, ws=wsbb, **fz)
        gc = m.train_scan_bwd(x, dt, Bm, Cm, A, Dskip, L, bnd, dy, d_bounds=gn["dh0_blocks"], want_dh_init=True,
                              ws=wsb, **fz)
        out["gn"], out["gc"] = gn, gc

    step_ms = timed(all_block_step)
    log("[bench] %s: train_scan %.3f ms, all-block step %.3f ms" % (name, ev_ms, step_ms))
    all_block_step()
    torch.cuda.synchronize()
    nbytes = bytes_full(batch, T, D, e, ns)
    slots = slots_bidirectional(batch, T, D, ns)
    bslots = slots_backward(batch, T, D, ns)
    bb = bytes_backward(batch, T, D, e, L, ns)
    bbb = bytes_backward(batch, T, D, e, L, ns, blocks=True)
    step_bytes = 2 * nbytes + bb + bbb
    step_slots = 2 * slots + 2 * bslots
    frac = lambda n, ms: n / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS
    sfrac = lambda n, ms: n / (ms * 1e-3) / VALU_SLOTS_PER_S
    res = {
        "workload": name, "batch": batch, "d_inner": D, "d_state": ns, "seq": T, "block": L,
        "fused": fused, "reverse_operands": rev_ops, "steps": steps, "warmup": warmup,
        "train_scan": {"ms": ev_ms, "ms_wall": ms_per_step, "tokens_per_s": batch * T / (ev_ms * 1e-3),
                       "bytes": nbytes, "GBs": nbytes / (ev_ms * 1e-3) / 1e9, "hbm_frac": frac(nbytes, ev_ms),
                       "slot_frac": sfrac(slots, ev_ms)},
        "train_scan_blocks": {"ms": blocks_ms, "tokens_per_s": batch * T / (blocks_ms * 1e-3),
                              "GBs": nbytes / (blocks_ms * 1e-3) / 1e9, "hbm_frac": frac(nbytes, blocks_ms),
                              "slot_frac": sfrac(slots, blocks_ms)},
        "train_scan_bwd": {"ms": bwd_ms, "bytes": bb, "GBs": bb / (bwd_ms * 1e-3) / 1e9,
                           "hbm_frac": frac(bb, bwd_ms), "slot_frac": sfrac(bslots, bwd_ms)},
        "train_scan_blocks_bwd": {"ms": bbwd_ms, "bytes": bbb, "GBs": bbb / (bbwd_ms * 1e-3) / 1e9,
                                  "hbm_frac": frac(bbb, bbwd_ms), "slot_frac": sfrac(bslots, bbwd_ms)},
        "all_block_step": {"ms": step_ms, "tokens_per_s": batch * T / (step_ms * 1e-3), "bytes": step_bytes,
                           "GBs": step_bytes / (step_ms * 1e-3) / 1e9, "hbm_frac": frac(step_bytes, step_ms),
                           "slot_frac": sfrac(step_slots, step_ms),
                           "note": "clean train_scan with block states, noisy train_scan_blocks, noisy "
                                   "backward, clean backward fed the noisy block-start gradients"},
        "full_scan": {"ms": full_ms, "tokens_per_s": batch * T / (full_ms * 1e-3),
                      "slot_frac": sfrac(slots, full_ms), "train_scan_over_full_scan_time": ev_ms / full_ms},
        "two_stream": {"ms": two_ms, "over_full_scan_time": two_ms / full_ms,
                       "note": "clean train_scan with h_bounds + noisy train_scan_blocks, against one "
                               "full-sequence scan of the noisy stream"},
    }
    if check and not fused and not rev_ops:
        errs, cpu_s = oracle_leg_training(torch, synth, x, dt, Bm, Cm, A, Dskip, L, dy, y_c, bnd, y_n,
                                          out["gn"], out["gc"], 2e-2 if e == 2 else 1e-4, step_bytes, 23)
        res["max_rel_err"] = errs
        res["worst_rel_err"] = worst_of(errs)
        res["cpu_baseline_sampled"] = cpu_s
        log("[bench] %s: oracle check: worst rel err %.2e" % (name, res["worst_rel_err"]))
    del x, dt, Bm, Cm, y, ws, wsf, wsb, wsbb, bnd, dy, y_c, y_n, out
    torch.cuda.empty_cache()
    return res


def config_summary(r):
    """The compact per-workload record of the configs object."""
    if "seq" in r:
        keys = ("train_scan", "train_scan_blocks", "train_scan_bwd", "train_scan_blocks_bwd", "all_block_step",
                "full_scan")
        out = {k: r[k] for k in ("workload", "batch", "d_inner", "d_state", "seq", "block")}
        for k in keys:
            out[k] = r[k]
    else:
        out = {k: r[k] for k in ("workload", "batch", "d_inner", "d_state", "ctx", "block", "denoising_steps",
                                 "n_blocks", "launch")}
        for k in ("step", "prefill", "block_step", "commit", "generation_tokens_per_s", "baseline_full_scan"):
            if k in r:
                out[k] = r[k]
    for k in ("worst_rel_err", "max_rel_err", "cpu_baseline_sampled"):
        if k in r:
            out[k] = r[k]
    return out


# ------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="infer_65k_b8")
    ap.add_argument("--no-configs", action="store_true", help="headline workload only (no configs object)")
    ap.add_argument("--config-steps", type=int, default=10, help="timed steps per config")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-baseline-scan", action="store_true")
    ap.add_argument("--eager", action="store_true", help="launch block steps eagerly (no graph)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (scale for HBM byte counters)")
    ap.add_argument("--fused", action="store_true",
                    help="use the Mamba-1 fusions: the dt stream holds the raw step size, "
                         "dt = softplus(dt_raw + bias) inside the scan, block-step outputs gated by silu(z)")
    ap.add_argument("--reverse-operands", action="store_true",
                    help="give the in-block reverse scan its own dt, B, C and A (block steps, "
                         "training forms and the baseline)")
    ap.add_argument("--block-len", type=int, default=0,
                    help="training workloads: block length other than the workload's (1..256)")
    ap.add_argument("--d-state", type=int, default=0,
                    help="training workloads: state count other than 16 (4, 8 or 32)")
    ap.add_argument("--crossover", action="store_true",
                    help="sweep the context length (8K..64K, batch 8, d_inner 1536) and report "
                         "block-restricted against full-sequence generation rates")
    ap.add_argument("--model-loop", action="store_true",
                    help="stand-in multi-layer denoising loop (random-weight Mamba stack around "
                         "the fused scan, no attention): cached block-restricted step against the "
                         "full-sequence rescan, at 8K and 64K context")
    ap.add_argument("--layers", type=int, default=24, help="--model-loop: layers of the stack")
    ap.add_argument("--roof-probe", action="store_true", help="print the microbenchmarks alone")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        return 2

    import torch
    import mamba_selective_scan_04_amd as m
    from mamba_selective_scan_04_amd import synth

    m.load()   # fails loudly if the HIP library is missing
    torch.cuda.set_device(0)
    probe = Probe(torch)
    if args.roof_probe:
        r = run_probes(torch, probe)
        print(json.dumps({"metric": "microbenchmarks of the chip's issue rates and HBM bandwidth",
                          "roof_probe": r}), flush=True)
        return 0
    if args.crossover:
        return crossover_main(args, m, synth, torch)
    if args.model_loop:
        return model_loop_main(args, m, synth, torch)
    wl = dict(synth.WORKLOADS[args.workload])
    if args.copy_calibration:
        # a plain copy of known size: 1 GiB read + 1 GiB written per launch
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda:0").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log("[bench] copy calibration: 3 x 1 GiB device copies")
    if "seq" in wl:
        r = run_training(args.workload, args, m, synth, torch, args.steps, args.warmup)
        print(json.dumps(train_line(args, r, torch)), flush=True)
        return 0
    if args.block_len or args.d_state:
        print("--block-len / --d-state apply to the training workloads", file=sys.stderr)
        return 2

    head = run_inference(args.workload, args, m, synth, torch, probe, args.steps, args.warmup,
                         cpu_rows_baseline=True)
    default_run = (args.workload == "infer_65k_b8" and not args.fused and not args.reverse_operands
                   and not args.eager)
    probes = run_probes(torch, probe)
    log("[bench] roof probe: FMA %.1f T/s, exp2 %.1f T/s, read %.0f GB/s"
        % (probes["fma_T_per_s"], probes["exp2_T_per_s"], probes["hbm_read_GBs"]))
    configs = None
    if default_run and not args.no_configs:
        configs = {}
        for name in CONFIG_WORKLOADS:
            if name == args.workload:
                configs[name] = config_summary(head)
                continue
            if "seq" in synth.WORKLOADS[name]:
                r = run_training(name, argparse.Namespace(), m, synth, torch, args.config_steps, 2)
            else:
                r = run_inference(name, argparse.Namespace(), m, synth, torch, probe, args.config_steps, 2)
            configs[name] = config_summary(r)
    print(json.dumps(inference_line(args, head, probes, configs)), flush=True)
    return 0


def inference_line(args, r, probes, configs):
    pf, fused = r["prefill"], bool(args.fused)
    e_ms = pf["ms"]
    pf_slots = pf["slot_frac"] * VALU_SLOTS_PER_S * (e_ms * 1e-3)
    roofline = {
        "kernel": "prefill: chunk_state_kernel (chunk-local forward scan) + carry_kernel, one launch sequence "
                  "timed with HIP events on its stream",
        "bound": "alu",
        "achieved": pf["slot_frac"] * VALU_SLOTS_PER_S / 1e12,
        "peak": VALU_SLOTS_PER_S / 1e12,
        "unit": "T fp32 VALU issue slots/s",
        "op": "fp32 VALU issue slot (mul/FMA 1, v_exp_f32 %d); per (token, channel): "
              "16 x (exp2 + 2 mul + FMA) + 1 mul%s" % (
                  EXP_SLOTS, " + %d for dt = softplus(dt_raw + bias)" % SOFTPLUS_SLOTS if fused else ""),
        "frac": pf["slot_frac"],
        "traffic": None if fused else committed_traffic(args.workload, r["batch"], r["d_inner"]),
        "frac_hbm": pf["hbm_frac"],
        "hbm_achieved_GBs": pf["GBs"],
        "hbm_peak_GBs": HBM_PEAK_GBS,
        "frac_fp32_published": pf["flop_frac_fp32_published"],
        "fp32_published_TFLOPs": FP32_PUBLISHED_FLOPS / 1e12,
        "flop_note": "flops per (token, channel): 16 x (exp2 1 + 2 mul + FMA 2) + 1 = 81; the published "
                     "157.3 TFLOP/s counts packed FMA (two fp32 lanes per slot), which this build does not "
                     "issue",
        "launch_ms": e_ms,
        "frac_of_probed_fma_rate": pf_slots / (e_ms * 1e-3) / (probes["fma_T_per_s"] * 1e12),
        "frac_of_probed_scan_mix": pf["tokens_per_s"] * r["d_inner"] * NS / (probes["scan_mix_T_elements_per_s"] * 1e12),
        "frac_hbm_of_probed_read": pf["GBs"] / probes["hbm_read_GBs"],
    }
    clk = None if fused else committed_clock(args.workload)
    if clk is not None:
        roofline["counter_run"] = dict(clk, note=(
            "the chunk scan alone, from the committed VALU counter pass (a profiled run, own clock); "
            "slot_frac_at_its_clock above 1 means the SIMDs overlapped part of each v_exp_f32's second "
            "issue cycle with other waves' VALU work, so the 2-slot exp model is a conservative roof"))
    line = {
        "metric": "block-step scan GB/s & % HBM peak at 65K/262K ctx; prefill tokens/s",
        "value": r["step"]["GBs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["step"]["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": r["batch"], "d_inner": r["d_inner"], "d_state": NS,
                   "ctx": r["ctx"], "block": r["block"], "denoising_steps": r["denoising_steps"],
                   "n_blocks": r["n_blocks"], "launch": r["launch"], "fused": fused,
                   "reverse_operands": bool(args.reverse_operands)},
        "hbm_frac_step": r["step"]["hbm_frac"],
        "hbm_copy_GBs": probes["hbm_copy_GBs"],
        "hbm_frac_step_of_copy": r["step"]["GBs"] / probes["hbm_copy_GBs"],
        "prefill_tokens_per_s": pf["tokens_per_s"],
        "block_step_GBs": r["block_step"]["GBs"],
        "calls": {k: r[k] for k in ("prefill", "block_step", "commit", "generation_tokens_per_s")},
        "baseline_full_scan": r.get("baseline_full_scan"),
        "roofline": roofline,
        "max_rel_err": r.get("max_rel_err"),
        "worst_rel_err": r.get("worst_rel_err"),
        "cpu_baseline": r.get("cpu_baseline"),
        "cpu_baseline_sampled": r.get("cpu_baseline_sampled"),
        "roof_probe": probes,
        "configs": configs,
    }
    return line


def train_line(args, r, torch):
    """The JSON line of a training workload (--workload train_*)."""
    ts = r["train_scan"]
    line = {
        "metric": "all-block training scan GB/s (forward over T + reverse per block)",
        "value": ts["bytes"] / (ts["ms_wall"] * 1e-3) / 1e9, "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ts["ms_wall"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": args.workload, "batch": r["batch"], "d_inner": r["d_inner"],
                   "d_state": r["d_state"], "seq": r["seq"], "block": r["block"], "fused": r["fused"],
                   "reverse_operands": r["reverse_operands"]},
    }
    for k in ("train_scan", "train_scan_blocks", "train_scan_bwd", "train_scan_blocks_bwd", "all_block_step",
              "full_scan", "two_stream", "worst_rel_err", "max_rel_err", "cpu_baseline_sampled"):
        if k in r:
            line[k] = r[k]
    return line


def reverse_operands(synth, batch, T, D, sid, dtype, dev, torch, ns=NS):
    """Seeded operands of the reverse direction: dt_r, B_r, C_r, A_r."""
    return dict(dt=synth.positive_step((batch, T, D), 1000 * sid + 80, dev, dtype),
                B=synth.normal((batch, T, ns), 1000 * sid + 81, dev, dtype),
                C=synth.normal((batch, T, ns), 1000 * sid + 82, dev, dtype),
                A=synth.a_matrix(D, ns, "default", device=dev))


def crossover_main(args, m, synth, torch):
    """Context-length sweep at batch 8, d_inner 1536: per context, the cost of
    generating one 16-token block (16 denoising block steps + the commit, from
    the cache) against the full-sequence scheme, which rescans context + block
    in both directions at each of the 16 steps.  Also reported: the prefill,
    and the break-even number of generated blocks after which the prefill has
    paid for itself against rescanning (the kernel-level crossover)."""
    batch, D, L, S, sid = 8, 1536, 16, 16, 6
    dtype = torch.bfloat16
    e = 2
    dev = "cuda:0"
    torch.cuda.set_device(0)
    st = torch.cuda.current_stream()
    A, Dskip = synth.params(D, NS, sid, "default", dev)
    steps_in = [synth.step_inputs(batch, L, D, NS, sid, j, dtype, dev) for j in range(S)]
    commit_in = synth.commit_inputs(batch, L, D, NS, sid, 0, dtype, dev)
    y_blk = torch.empty(batch, L, D, dtype=dtype, device=dev)

    def time_calls(fn, reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fn()
        torch.cuda.synchronize()
        a.record(st)
        for _ in range(reps):
            fn()
        b.record(st)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    rows = []
    for ctx in (8192, 16384, 32768, 65536):
        log("[bench] crossover: ctx %d" % ctx)
        Tf = ctx + L
        x, dt, Bm, Cm = synth.stream(batch, Tf, D, NS, sid, 0, dtype, dev)
        h = torch.empty(batch, D, NS, dtype=torch.float32, device=dev)
        ws = torch.empty(max(1, m.workspace_bytes(batch, D, Tf, m.OP_FULL, 1, NS, dtype)),
                         dtype=torch.uint8, device=dev)
        xc, dtc, Bc, Cc = x[:, :ctx], dt[:, :ctx], Bm[:, :ctx], Cm[:, :ctx]
        xc, dtc, Bc, Cc = xc.contiguous(), dtc.contiguous(), Bc.contiguous(), Cc.contiguous()
        pf_ms = time_calls(lambda: m.prefill(xc, dtc, Bc, Cc, A, Dskip, L, h_cache=h, ws=ws), 10)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for j in range(S):
                m.block_step(h, *steps_in[j], A, Dskip, y=y_blk)
            m.commit(h, *commit_in, A, Dskip)
        blk_ms = time_calls(g.replay, 20)
        yf = torch.empty_like(x)
        f_ms = time_calls(lambda: m.full_scan(x, dt, Bm, Cm, A, Dskip, y=yf, ws=ws), 5)
        full_blk_ms = S * f_ms
        rows.append({
            "ctx": ctx, "prefill_ms": pf_ms, "block_restricted_block_ms": blk_ms,
            "full_sequence_block_ms": full_blk_ms,
            "generation_tokens_per_s": batch * L / (blk_ms * 1e-3),
            "full_sequence_generation_tokens_per_s": batch * L / (full_blk_ms * 1e-3),
            "ratio": full_blk_ms / blk_ms,
            "break_even_blocks": pf_ms / max(full_blk_ms - blk_ms, 1e-9),
        })
        del x, dt, Bm, Cm, xc, dtc, Bc, Cc, yf, ws, g
        torch.cuda.empty_cache()
    r8 = rows[0]
    line = {
        "metric": "kernel-level generation tokens/s, block-restricted vs full-sequence, by context",
        "value": r8["generation_tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": len(rows), "warmup": 1, "ms_per_step": r8["block_restricted_block_ms"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "crossover sweep, contexts 8192..65536", "batch": batch,
                   "d_inner": D, "d_state": NS, "block": L, "denoising_steps": S},
        "rows": rows,
    }
    print(json.dumps(line), flush=True)
    return 0


def model_loop_main(args, m, synth, torch):
    """A stand-in for the model around the scan: a stack of random-weight
    Mamba-1 mixer layers (RMSNorm, in-projection to x and the gate z,
    x-projection to the low-rank dt and B, C, dt-projection, the fused scan
    with dt = softplus(dt_raw + bias) and the silu(z) gate, out-projection,
    residual), batch 8, d_model 768, d_inner 1536, 16 states, dt rank 48.  The
    projections are plain torch GEMMs; there are no attention layers and no
    short convolution.  Per denoising step of one 16-token block it times
      cached: the block's 16 tokens through every layer, each layer's scan a
              block_step from that layer's cache (plus, per block, the commit
              pass of the clean tokens, reported apart);
      full:   context + block through every layer, each scan a full_scan (the
              full-sequence scheme rescans everything every step).
    The ratio is a model-level analog for a Mamba-only stack; the pages'
    figures include attention layers and are quoted only as context."""
    batch, dm, D, R, L, S = 8, 768, 1536, 48, 16, 16
    nl = args.layers
    dtype = torch.bfloat16
    dev = "cuda:0"
    torch.cuda.set_device(0)
    st = torch.cuda.current_stream()
    g = torch.Generator(device=dev)
    g.manual_seed(4242)

    def w(shape, fan_in):
        return (torch.randn(shape, generator=g, device=dev, dtype=torch.float32) / math.sqrt(fan_in)).to(dtype)

    layers = []
    for i in range(nl):
        A, Dskip = synth.params(D, NS, 900 + i, "default", dev)
        layers.append(dict(norm=torch.ones(dm, device=dev, dtype=dtype), w_x=w((dm, D), dm),
                           w_z=w((dm, D), dm), w_p=w((D, R + 2 * NS), D), w_dt=w((R, D), R),
                           dt_bias=torch.full((D,), math.log(math.expm1(0.05)), device=dev),
                           A=A, Dskip=Dskip, w_out=w((D, dm), D)))

    def mixer_inputs(lay, X):
        """[batch, T, d_model] -> the scan's x, dt_raw, B, C, z ([batch, T, .])"""
        b, T = X.shape[0], X.shape[1]
        h = X.view(-1, dm)
        h = (h.float() * torch.rsqrt(h.float().pow(2).mean(-1, keepdim=True) + 1e-5)).to(dtype) * lay["norm"]
        x = torch.mm(h, lay["w_x"])
        z = torch.mm(h, lay["w_z"])
        p = torch.mm(x, lay["w_p"])
        dt = torch.mm(p[:, :R], lay["w_dt"])
        Bm = p[:, R:R + NS].contiguous()
        Cm = p[:, R + NS:].contiguous()
        return (x.view(b, T, D), dt.view(b, T, D), Bm.view(b, T, NS), Cm.view(b, T, NS), z.view(b, T, D))

    def layer_out(lay, X, y):
        return X + torch.mm(y.view(-1, D), lay["w_out"]).view(X.shape)

    def cached_step(X, caches):
        for lay, h in zip(layers, caches):
            x, dt, Bm, Cm, z = mixer_inputs(lay, X)
            y = m.block_step(h, x, dt, Bm, Cm, lay["A"], lay["Dskip"], dt_bias=lay["dt_bias"],
                             dt_softplus=True, z=z)
            X = layer_out(lay, X, y)
        return X

    def commit_pass(X, caches):
        for lay, h in zip(layers, caches):
            x, dt, Bm, Cm, z = mixer_inputs(lay, X)
            _, y = m.commit(h, x, dt, Bm, Cm, lay["A"], lay["Dskip"], want_y=True,
                            dt_bias=lay["dt_bias"], dt_softplus=True, z=z)
            X = layer_out(lay, X, y)
        return X

    def full_step(X, ws):
        for lay in layers:
            x, dt, Bm, Cm, z = mixer_inputs(lay, X)
            y = m.full_scan(x, dt, Bm, Cm, lay["A"], lay["Dskip"], ws=ws, dt_bias=lay["dt_bias"],
                            dt_softplus=True, z=z)
            X = layer_out(lay, X, y)
        return X

    def prefill_pass(X, caches, ws):
        for lay, h in zip(layers, caches):
            x, dt, Bm, Cm, z = mixer_inputs(lay, X)
            _, y = m.prefill(x, dt, Bm, Cm, lay["A"], lay["Dskip"], L, h_cache=h, want_y=True, ws=ws,
                             dt_bias=lay["dt_bias"], dt_softplus=True, z=z)
            X = layer_out(lay, X, y)
        return X

    def time_calls(fn, reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fn()
        torch.cuda.synchronize()
        a.record(st)
        for _ in range(reps):
            fn()
        b.record(st)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    rows = []
    for ctx in (8192, 65536):
        log("[bench] model loop: ctx %d, %d layers" % (ctx, nl))
        Tf = ctx + L
        Xc = torch.randn(batch, ctx, dm, generator=g, device=dev, dtype=torch.float32).to(dtype)
        Xb = torch.randn(batch, L, dm, generator=g, device=dev, dtype=torch.float32).to(dtype)
        Xf = torch.randn(batch, Tf, dm, generator=g, device=dev, dtype=torch.float32).to(dtype)
        caches = [torch.zeros(batch, D, NS, dtype=torch.float32, device=dev) for _ in range(nl)]
        wsp = torch.empty(max(1, m.workspace_bytes(batch, D, ctx, m.OP_PREFILL, L, NS, dtype)),
                          dtype=torch.uint8, device=dev)
        wsf = torch.empty(max(1, m.workspace_bytes(batch, D, Tf, m.OP_FULL, 1, NS, dtype)),
                          dtype=torch.uint8, device=dev)
        pf_ms = time_calls(lambda: prefill_pass(Xc, caches, wsp), 1)
        step_ms = time_calls(lambda: cached_step(Xb, caches), 20)
        # the cached step replayed from a HIP graph (the launches are the same
        # every step); kept only if every replay, with eager work between
        # them, reproduces the eager result bit for bit
        ref = cached_step(Xb, caches).clone()
        gr = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(st)
        with torch.cuda.stream(side):
            cached_step(Xb, caches)
        st.wait_stream(side)
        with torch.cuda.graph(gr):
            out_g = cached_step(Xb, caches)
        graph_ok = True
        for _ in range(3):
            gr.replay()
            torch.cuda.synchronize()
            graph_ok = graph_ok and torch.equal(out_g, ref)
            cached_step(Xb, caches)
            torch.cuda.synchronize()
        step_graph_ms = time_calls(gr.replay, 50) if graph_ok else None
        del gr, out_g
        ccaches = [c.clone() for c in caches]
        commit_ms = time_calls(lambda: commit_pass(Xb, ccaches), 5)
        full_ms = time_calls(lambda: full_step(Xf, wsf), 2)
        # the scans alone, for the share of the step they take
        scan_in = mixer_inputs(layers[0], Xb)
        scan_ms = nl * time_calls(lambda: m.block_step(caches[0], *scan_in[:4], layers[0]["A"], layers[0]["Dskip"],
                                                       dt_bias=layers[0]["dt_bias"], dt_softplus=True,
                                                       z=scan_in[4]), 50)
        full_in = mixer_inputs(layers[0], Xf)
        full_scan_ms = nl * time_calls(lambda: m.full_scan(*full_in[:4], layers[0]["A"], layers[0]["Dskip"], ws=wsf,
                                                           dt_bias=layers[0]["dt_bias"], dt_softplus=True,
                                                           z=full_in[4]), 2)
        blk_ms = S * step_ms + commit_ms
        blk_g_ms = None if step_graph_ms is None else S * step_graph_ms + commit_ms
        rows.append({"ctx": ctx, "layers": nl, "prefill_ms": pf_ms,
                     "cached_step_ms": step_ms, "cached_step_graph_ms": step_graph_ms,
                     "graph_replays_match_eager": graph_ok, "commit_pass_ms": commit_ms,
                     "cached_block_ms": blk_ms, "cached_block_graph_ms": blk_g_ms,
                     "full_step_ms": full_ms, "full_block_ms": S * full_ms,
                     "step_ratio": full_ms / step_ms, "block_ratio": S * full_ms / blk_ms,
                     "block_ratio_graph": None if blk_g_ms is None else S * full_ms / blk_g_ms,
                     "scan_share_cached": scan_ms / step_ms,
                     "scan_share_cached_graph": None if step_graph_ms is None else scan_ms / step_graph_ms,
                     "scan_share_full": full_scan_ms / full_ms,
                     "generation_tokens_per_s": batch * L / (blk_ms * 1e-3),
                     "full_generation_tokens_per_s": batch * L / (S * full_ms * 1e-3)})
        del Xc, Xf, caches, ccaches, wsp, wsf, full_in
        torch.cuda.empty_cache()
    r = rows[-1]
    line = {
        "metric": "stand-in model loop: denoising-step time, cached block-restricted vs full-sequence rescan",
        "value": r["block_ratio"], "unit": "x (full-sequence time / block-restricted time per block)",
        "n_gpus": 1, "steps": S, "warmup": 1, "ms_per_step": r["cached_step_ms"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (random weights)",
        "config": {"workload": "random-weight Mamba-1 stack, no attention, eager launches "
                               "(cached step also from a HIP graph)",
                   "batch": batch, "d_model": dm, "d_inner": D, "d_state": NS, "dt_rank": R,
                   "layers": nl, "block": L, "denoising_steps": S},
        "rows": rows,
    }
    print(json.dumps(line), flush=True)
    return 0



if __name__ == "__main__":
    sys.exit(main())
