#!/usr/bin/env python3
"""Benchmark of the block-restricted bidirectional selective scan on one MI355X.

One step = one pass of the inference hot path over one batch of synthetic,
device-resident input of the chosen workload:
    prefill of the clean context (forward scan, cache written)
    then, for each of n_blocks blocks: 16 denoising block steps (forward from
    the cache + in-block reverse + output) and one commit (cache advanced).
The prefill is launched eagerly; each block's 16 block steps + commit are
replayed from a captured HIP graph (one graph per block: the launches are
identical every step, so capture removes only host launch overhead).

Printed: one JSON line on stdout (progress goes to stderr).
  value   whole-step algorithmic HBM throughput (GB/s): bytes every call in the
          step must move (inputs read once, outputs written once, states read
          or written once) / measured step time
  roofline  for the dominant kernel (the prefill's chunk-local forward scan +
          its carry), which is VALU-bound: achieved fp32 VALU issue slots per
          second against the chip's slot rate (256 CUs x 4 SIMDs x 16 lanes x
          2.4 GHz; v_exp_f32 takes two slots), plus the HBM view
  cpu_baseline  the fp64 CPU oracle timed on a bounded sample of the same step
Also measured outside the timed region: the full-sequence bidirectional
baseline (reverse over the whole sequence, rescanned every denoising step).

Training workloads (train_87m, train_350m) time the all-block training scan,
the two-stream form and the full-sequence scan instead.  --crossover sweeps the
context length from 8K to 64K tokens and prints generation rates of the
block-restricted and the full-sequence schemes; --model-loop runs the scan
inside a random-weight stand-in Mamba stack (context only).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--crossover]
"""
import argparse
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
EXP_SLOTS = 2            # v_exp_f32 issues at half rate on gfx950
# dt = softplus(dt_raw + bias) per (token, channel): bias add, |v| scale, exp2
# (2), 1 + w, log2 (2), ln 2 scale, u - 1, rcp (2), two muls, compare, select,
# max, add
SOFTPLUS_SLOTS = 17
NS = 16


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------ algorithmic cost

def bytes_prefill(batch, T, D, e, h_init=False):
    return batch * T * D * 2 * e + batch * T * NS * e + 4 * D * NS + 4 * batch * D * NS * (2 if h_init else 1)


def bytes_block_step(batch, L, D, e):
    return batch * L * D * 3 * e + batch * L * NS * 2 * e + 4 * D * NS + 4 * D + 4 * batch * D * NS


def bytes_commit(batch, L, D, e):
    return batch * L * D * 2 * e + batch * L * NS * e + 4 * D * NS + 2 * 4 * batch * D * NS


def bytes_full(batch, T, D, e):
    return batch * T * D * 3 * e + batch * T * NS * 2 * e + 4 * D * NS + 4 * D


def committed_traffic(workload, batch, D):
    """HBM bytes per prefill (chunk scan + carry) from the committed counter
    summary for this workload, or None if there is none or the kernels have
    changed since it was taken (source hash mismatch)."""
    from mamba_selective_scan_04_amd import profile_summary
    path = os.path.join(ROOT, "profiles", "prefill_%s_hbm_traffic.md" % workload.replace("infer_", ""))
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    if "kernel source hash: %s" % profile_summary.source_hash() not in txt:
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
    """(clock GHz, VALUBusy %) of the prefill's chunk scan from the committed
    VALU counter summary for this workload, or None if there is none or the
    kernels have changed since it was taken."""
    from mamba_selective_scan_04_amd import profile_summary
    path = os.path.join(ROOT, "profiles", "prefill_%s_valu_counters.md" % workload.replace("infer_", ""))
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    if "kernel source hash: %s" % profile_summary.source_hash() not in txt:
        return None
    best = None
    for line in txt.splitlines():
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) != 10 or not re.fullmatch(r"chunk_state_kernel<\w+, false, false, 0, 16>", cells[0]):
            continue
        try:
            grid, ghz, busy = int(cells[1]), float(cells[4]), float(cells[9])
        except ValueError:
            continue
        if best is None or grid > best[0]:
            best = (grid, ghz, busy)
    return None if best is None else best[1:]


def slots_forward(batch, T, D):
    """exp2 (2 slots) + dt*A' mul + (dt*x)*B mul + state FMA per (b,t,d,n),
    plus the dt*x multiply per (b,t,d)."""
    return batch * T * D * (NS * (EXP_SLOTS + 3) + 1)


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


# ------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="infer_65k_b8")
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
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        return 2

    import torch
    import mamba_selective_scan_04_amd as m
    from mamba_selective_scan_04_amd import synth

    m.load()   # fails loudly if the HIP library is missing
    if args.crossover:
        return crossover_main(args, m, synth, torch)
    if args.model_loop:
        return model_loop_main(args, m, synth, torch)
    wl = dict(synth.WORKLOADS[args.workload])
    if "seq" in wl:
        return train_main(args, wl, m, synth, torch)
    if args.block_len or args.d_state:
        print("--block-len / --d-state apply to the training workloads", file=sys.stderr)
        return 2
    batch, D, ctx, L = wl["batch"], wl["d_inner"], wl["ctx"], wl["block"]
    S, nblk, sid = wl["steps"], wl["n_blocks"], wl["sid"]
    dtype = synth.TORCH_DTYPE[wl["dtype"]]
    e = 2 if dtype == torch.bfloat16 else 4
    dev = "cuda:0"
    torch.cuda.set_device(0)
    st = torch.cuda.current_stream()

    log("[bench] workload %s: batch %d, d_inner %d, ctx %d, block %d, %d steps x %d blocks"
        % (args.workload, batch, D, ctx, L, S, nblk))
    t_gen = time.time()
    x, dt, Bm, Cm = synth.stream(batch, ctx, D, NS, sid, 0, dtype, dev)
    A, Dskip = synth.params(D, NS, sid, "default", dev)
    steps_in = [synth.step_inputs(batch, L, D, NS, sid, j, dtype, dev) for j in range(S)]
    commit_in = [synth.commit_inputs(batch, L, D, NS, sid, k, dtype, dev) for k in range(nblk)]
    fz_pf, fz_bs = {}, {}
    if args.fused:
        # raw step sizes in place of dt, a per-channel bias, and the gates
        raw = lambda shape, seed: synth.normal(shape, seed, dev, dtype, mean=-1.0, std=0.5)
        dt = raw((batch, ctx, D), 1000 * sid + 70)
        steps_in = [(sx, raw((batch, L, D), 1000 * sid + 71 + j), sb, sc) for j, (sx, _, sb, sc) in enumerate(steps_in)]
        commit_in = [(cx, raw((batch, L, D), 1000 * sid + 91 + k), cb, cc) for k, (cx, _, cb, cc) in enumerate(commit_in)]
        bias = synth.normal((D,), 1000 * sid + 72, dev, torch.float32, std=0.3)
        fz_pf = dict(dt_bias=bias, dt_softplus=True)
        fz_bs = dict(fz_pf, z=synth.normal((batch, L, D), 1000 * sid + 73, dev, dtype))
    if args.reverse_operands:
        fz_bs = dict(fz_bs, rev=reverse_operands(synth, batch, L, D, sid, dtype, dev, torch))
    h = torch.empty(batch, D, NS, dtype=torch.float32, device=dev)
    y_blk = torch.empty(batch, L, D, dtype=dtype, device=dev)
    ws = torch.empty(max(1, m.workspace_bytes(batch, D, ctx, m.OP_PREFILL, L, NS, dtype)),
                     dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    log("[bench] inputs generated on device in %.1f s" % (time.time() - t_gen))
    if args.copy_calibration:
        # a plain copy of known size: 1 GiB read + 1 GiB written per launch
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log("[bench] copy calibration: 3 x 1 GiB device copies")

    def prefill():
        m.prefill(x, dt, Bm, Cm, A, Dskip, L, h_cache=h, ws=ws, **fz_pf)

    def block(k):
        for j in range(S):
            m.block_step(h, *steps_in[j], A, Dskip, y=y_blk, **fz_bs)
        m.commit(h, *commit_in[k], A, Dskip, **fz_pf)

    launch = "eager"
    graphs = None
    if not args.eager:
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

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log("[bench] warmup done (%d steps, %s block launches)" % (args.warmup, launch))

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pf_ms = sum(ev[0].elapsed_time(ev[1]) for ev in evs) / args.steps
    blk_ms = sum(ev[1].elapsed_time(ev[2]) for ev in evs) / args.steps
    ms_per_step = wall * 1e3 / args.steps
    log("[bench] timed %d steps: %.3f ms/step (prefill %.3f ms, blocks %.3f ms)"
        % (args.steps, ms_per_step, pf_ms, blk_ms))

    # ---- per-call breakdown of the block phase (events around R replays)
    R = 50
    bs_x = [steps_in[0][i] for i in range(4)]
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
    g_bs = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_bs):
        for _ in range(R):
            m.block_step(h, *bs_x, A, Dskip, y=y_blk, **fz_bs)
    g_cm = torch.cuda.CUDAGraph()
    hc = h.clone()
    with torch.cuda.graph(g_cm):
        for _ in range(R):
            m.commit(hc, *commit_in[0], A, Dskip, **fz_pf)
    bs_ms = time_calls(g_bs.replay, 4) / R
    cm_ms = time_calls(g_cm.replay, 4) / R
    bs_eager_ms = time_calls(lambda: m.block_step(h, *bs_x, A, Dskip, y=y_blk, **fz_bs), 200)

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
            m.block_step(h, *bs_x, A, Dskip, y=y_blk, **fz_bs)
    g_scrub = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_scrub):
        for i in range(K):
            scrub.fill_(float(i))

    def best_replay_ms(g, reps=5):
        best = None
        for _ in range(reps):
            v = time_calls(g.replay, 1)
            best = v if best is None else min(best, v)
        return best

    bs_cold_ms = (best_replay_ms(g_cold) - best_replay_ms(g_scrub)) / K
    del g_cold, g_scrub, scrub

    # ---- the practical HBM roof in the same run: a 1 GiB device copy
    csrc = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
    cdst = torch.empty_like(csrc)
    copy_ms = time_calls(lambda: cdst.copy_(csrc), 5)
    copy_GBs = 2 * csrc.numel() * 4 / (copy_ms * 1e-3) / 1e9
    del csrc, cdst

    # the fused path also reads the bias (4 D bytes per call) and the block
    # steps' gates (one element per (token, channel))
    fz_bytes_bs = (batch * L * D * e + 4 * D) if args.fused else 0
    if args.reverse_operands:   # dt_r per (token, channel), B_r and C_r per token, A_r
        fz_bytes_bs += batch * L * D * e + 2 * batch * L * NS * e + 4 * D * NS
    fz_bytes_pf = 4 * D if args.fused else 0
    step_bytes = (bytes_prefill(batch, ctx, D, e) + fz_bytes_pf
                  + nblk * (S * (bytes_block_step(batch, L, D, e) + fz_bytes_bs)
                            + bytes_commit(batch, L, D, e) + fz_bytes_pf))
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    pf_bytes = bytes_prefill(batch, ctx, D, e) + fz_bytes_pf
    pf_slots = slots_forward(batch, ctx, D) + (batch * ctx * D * SOFTPLUS_SLOTS if args.fused else 0)
    achieved_slots = pf_slots / (pf_ms * 1e-3)
    roofline = {
        "kernel": "prefill: chunk_state_kernel (chunk-local forward scan) + carry_kernel",
        "bound": "alu",
        "achieved": achieved_slots / 1e12,
        "peak": VALU_SLOTS_PER_S / 1e12,
        "unit": "TFLOP/s",
        "op": "fp32 VALU issue slot (mul/FMA 1, v_exp_f32 %d); per (token, channel): "
              "16 x (exp2 + 2 mul + FMA) + 1 mul%s" % (
                  EXP_SLOTS, " + %d for dt = softplus(dt_raw + bias)" % SOFTPLUS_SLOTS if args.fused else ""),
        "frac": achieved_slots / VALU_SLOTS_PER_S,
        "traffic": None if args.fused else committed_traffic(args.workload, batch, D),
        "hbm_achieved_GBs": pf_bytes / (pf_ms * 1e-3) / 1e9,
        "hbm_frac": pf_bytes / (pf_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "launch_ms": pf_ms,
        "hbm_frac_of_copy": pf_bytes / (pf_ms * 1e-3) / 1e9 / copy_GBs,
    }
    clk = None if args.fused else committed_clock(args.workload)
    if clk is not None:
        # the clock the dies sustained under this kernel (rocprofv3 counters,
        # committed summary): the peak at that clock, and VALUBusy
        roofline["clock_GHz_measured"] = clk[0]
        roofline["frac_at_measured_clock"] = achieved_slots / (VALU_SLOTS_PER_S * clk[0] / 2.4)
        roofline["valu_busy_pct"] = clk[1]

    gen_tok = batch * L * nblk
    gen_ms = nblk * (S * bs_ms + cm_ms)
    calls = {
        "prefill": {"ms": pf_ms, "tokens_per_s": batch * ctx / (pf_ms * 1e-3),
                    "GBs": pf_bytes / (pf_ms * 1e-3) / 1e9, "bytes": pf_bytes},
        "block_step": {"us_graph": bs_ms * 1e3, "us_eager": bs_eager_ms * 1e3,
                       "GBs": (bytes_block_step(batch, L, D, e) + fz_bytes_bs) / (bs_ms * 1e-3) / 1e9,
                       "bytes": bytes_block_step(batch, L, D, e) + fz_bytes_bs,
                       "us_graph_cold": bs_cold_ms * 1e3,
                       "GBs_cold": (bytes_block_step(batch, L, D, e) + fz_bytes_bs) / (bs_cold_ms * 1e-3) / 1e9,
                       "note": "us_graph: 50 calls in one graph, back to back; us_graph_cold: "
                               "graph of 20 x (512 MB scrub write + call) minus graph of 20 scrub "
                               "writes, per call"},
        "commit": {"us_graph": cm_ms * 1e3,
                   "GBs": bytes_commit(batch, L, D, e) / (cm_ms * 1e-3) / 1e9,
                   "bytes": bytes_commit(batch, L, D, e)},
        "generation_tokens_per_s": gen_tok / (gen_ms * 1e-3),
    }

    # ---- contrast: full-sequence bidirectional baseline, rescanned every step
    baseline = None
    if not args.no_baseline_scan and not args.fused and not args.reverse_operands:
        Tf = ctx + L
        del ws
        xf, dtf, Bf, Cf = synth.stream(batch, Tf, D, NS, sid, 200, dtype, dev)
        yf = torch.empty_like(xf)
        wsf = torch.empty(max(1, m.workspace_bytes(batch, D, Tf, m.OP_FULL, 1, NS, dtype)),
                          dtype=torch.uint8, device=dev)
        f_ms = time_calls(lambda: m.full_scan(xf, dtf, Bf, Cf, A, Dskip, y=yf, ws=wsf), 3)
        base_gen = batch * L / (S * f_ms * 1e-3)
        baseline = {"full_scan_ms": f_ms, "T": Tf,
                    "GBs": bytes_full(batch, Tf, D, e) / (f_ms * 1e-3) / 1e9,
                    "generation_tokens_per_s": base_gen,
                    "speedup_block_restricted": calls["generation_tokens_per_s"] / base_gen}
        del xf, dtf, Bf, Cf, yf, wsf
        log("[bench] baseline full scan over %d tokens: %.3f ms" % (Tf, f_ms))

    # ---- CPU baseline: the fp64 oracle on a bounded sample of the same step
    cpu = None
    if not args.no_cpu_baseline and not args.fused and not args.reverse_operands:
        cpu = cpu_baseline(x, dt, Bm, Cm, A, Dskip, steps_in, commit_in, L, args.cpu_seconds, e)

    line = {
        "metric": "block-step scan GB/s & % HBM peak at 65K/262K ctx; prefill tokens/s",
        "value": value,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if dtype == torch.bfloat16 else "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": batch, "d_inner": D, "d_state": NS,
                   "ctx": ctx, "block": L, "denoising_steps": S, "n_blocks": nblk,
                   "launch": launch, "fused": bool(args.fused),
                   "reverse_operands": bool(args.reverse_operands)},
        "hbm_frac_step": value / HBM_PEAK_GBS,
        "hbm_copy_GBs": copy_GBs,
        "hbm_frac_step_of_copy": value / copy_GBs,
        "prefill_tokens_per_s": calls["prefill"]["tokens_per_s"],
        "block_step_GBs": calls["block_step"]["GBs"],
        "calls": calls,
        "baseline_full_scan": baseline,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


def train_main(args, wl, m, synth, torch):
    """Training workloads: one step = one all-block training scan (continuous
    forward + reverse segmented per block) over the batch.  The full-sequence
    bidirectional scan over the same tokens is timed beside it."""
    batch, D, T, L, sid = wl["batch"], wl["d_inner"], wl["seq"], wl["block"], wl["sid"]
    L = args.block_len or L
    ns = args.d_state or NS
    if T % L != 0:
        raise SystemExit("block length %d does not divide the sequence length %d" % (L, T))
    dtype = synth.TORCH_DTYPE[wl["dtype"]]
    e = 2 if dtype == torch.bfloat16 else 4
    dev = "cuda:0"
    torch.cuda.set_device(0)
    st = torch.cuda.current_stream()
    log("[bench] workload %s: batch %d, d_inner %d, d_state %d, T %d, block %d"
        % (args.workload, batch, D, ns, T, L))
    x, dt, Bm, Cm = synth.stream(batch, T, D, ns, sid, 0, dtype, dev)
    A, Dskip = synth.params(D, ns, sid, "default", dev)
    y = torch.empty_like(x)
    fz = {}
    if args.fused:
        dt = synth.normal((batch, T, D), 1000 * sid + 70, dev, dtype, mean=-1.0, std=0.5)
        fz = dict(dt_bias=synth.normal((D,), 1000 * sid + 72, dev, torch.float32, std=0.3),
                  dt_softplus=True, z=synth.normal((batch, T, D), 1000 * sid + 73, dev, dtype))
    if args.reverse_operands:
        fz = dict(fz, rev=reverse_operands(synth, batch, T, D, sid, dtype, dev, torch, ns))
    ws = torch.empty(max(1, m.workspace_bytes(batch, D, T, m.OP_TRAIN, L, ns, dtype)),
                     dtype=torch.uint8, device=dev)
    wsf = torch.empty(max(1, m.workspace_bytes(batch, D, T, m.OP_FULL, 1, ns, dtype)),
                      dtype=torch.uint8, device=dev)

    def step():
        m.train_scan(x, dt, Bm, Cm, A, Dskip, L, y=y, ws=ws, **fz)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        evs[i][0].record(st)
        step()
        evs[i][1].record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = sum(a.elapsed_time(b) for a, b in evs) / args.steps
    ms_per_step = wall * 1e3 / args.steps
    nbytes = bytes_full(batch, T, D, e)
    slots = slots_bidirectional(batch, T, D, ns)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    m.full_scan(x, dt, Bm, Cm, A, Dskip, y=y, ws=wsf, **fz)
    a.record(st)
    for _ in range(args.steps):
        m.full_scan(x, dt, Bm, Cm, A, Dskip, y=y, ws=wsf, **fz)
    b.record(st)
    torch.cuda.synchronize()
    full_ms = a.elapsed_time(b) / args.steps
    # two-stream form: the noisy stream scanned from the clean stream's bounds
    bnd = torch.empty(batch, T // L + 1, D, ns, dtype=torch.float32, device=dev)
    m.train_scan(x, dt, Bm, Cm, A, Dskip, L, y=y, h_bounds=bnd, ws=ws, **fz)
    a.record(st)
    for _ in range(args.steps):
        m.train_scan_blocks(x, dt, Bm, Cm, A, Dskip, L, bnd, y=y, **fz)
    b.record(st)
    torch.cuda.synchronize()
    blocks_ms = a.elapsed_time(b) / args.steps
    # the all-block objective's two streams: the clean stream with its block
    # bounds, then the noisy stream scanned block by block from those bounds
    a.record(st)
    for _ in range(args.steps):
        m.train_scan(x, dt, Bm, Cm, A, Dskip, L, y=y, h_bounds=bnd, ws=ws, **fz)
        m.train_scan_blocks(x, dt, Bm, Cm, A, Dskip, L, bnd, y=y, **fz)
    b.record(st)
    torch.cuda.synchronize()
    two_ms = a.elapsed_time(b) / args.steps
    # backward passes: continuous form (from the saved block states) and the
    # two-stream form; then one whole all-block training step, forward and
    # backward over both streams
    dy = synth.normal((batch, T, D), 1000 * sid + 8, dev, dtype)
    sep = args.reverse_operands
    wsb = torch.empty(max(1, m.workspace_bytes(batch, D, T, m.OP_TRAIN_BWD_REV if sep else m.OP_TRAIN_BWD,
                                               L, ns, dtype)), dtype=torch.uint8, device=dev)
    wsbb = torch.empty(max(1, m.workspace_bytes(batch, D, T, m.OP_BLOCKS_BWD_REV if sep else m.OP_BLOCKS_BWD,
                                                L, ns, dtype)), dtype=torch.uint8, device=dev)
    m.train_scan(x, dt, Bm, Cm, A, Dskip, L, y=y, h_bounds=bnd, ws=ws, **fz)
    m.train_scan_bwd(x, dt, Bm, Cm, A, Dskip, L, bnd, dy, ws=wsb, **fz)
    torch.cuda.synchronize()
    a.record(st)
    for _ in range(args.steps):
        m.train_scan_bwd(x, dt, Bm, Cm, A, Dskip, L, bnd, dy, ws=wsb, **fz)
    b.record(st)
    torch.cuda.synchronize()
    bwd_ms = a.elapsed_time(b) / args.steps
    a.record(st)
    for _ in range(args.steps):
        m.train_scan_blocks_bwd(x, dt, Bm, Cm, A, Dskip, L, bnd, dy, want_dh0_blocks=True, ws=wsbb,
                                **fz)
    b.record(st)
    torch.cuda.synchronize()
    bbwd_ms = a.elapsed_time(b) / args.steps

    def all_block_step():
        m.train_scan(x, dt, Bm, Cm, A, Dskip, L, y=y, h_bounds=bnd, ws=ws, **fz)
        m.train_scan_blocks(x, dt, Bm, Cm, A, Dskip, L, bnd, y=y, **fz)
        gn = m.train_scan_blocks_bwd(x, dt, Bm, Cm, A, Dskip, L, bnd, dy, want_dh0_blocks=True,
                                     ws=wsbb, **fz)
        m.train_scan_bwd(x, dt, Bm, Cm, A, Dskip, L, bnd, dy, d_bounds=gn["dh0_blocks"], ws=wsb,
                         **fz)

    all_block_step()
    torch.cuda.synchronize()
    a.record(st)
    for _ in range(args.steps):
        all_block_step()
    b.record(st)
    torch.cuda.synchronize()
    step_ms = a.elapsed_time(b) / args.steps
    line = train_line(args, batch, D, T, L, dtype, nbytes, slots, ms_per_step, ev_ms, blocks_ms,
                      full_ms, two_ms, bwd_ms, bbwd_ms, step_ms, torch, ns)
    print(json.dumps(line), flush=True)
    return 0


def reverse_operands(synth, batch, T, D, sid, dtype, dev, torch, ns=NS):
    """Seeded operands of the reverse direction: dt_r, B_r, C_r, A_r."""
    return dict(dt=synth.positive_step((batch, T, D), 1000 * sid + 80, dev, dtype),
                B=synth.normal((batch, T, ns), 1000 * sid + 81, dev, dtype),
                C=synth.normal((batch, T, ns), 1000 * sid + 82, dev, dtype),
                A=synth.a_matrix(D, ns, "default", device=dev))


def train_line(args, batch, D, T, L, dtype, nbytes, slots, ms_per_step, ev_ms, blocks_ms, full_ms,
               two_ms, bwd_ms, bbwd_ms, step_ms, torch, ns=NS):
    """The JSON line of a training workload (bwd_ms / bbwd_ms / step_ms are
    None when the backward was not run)."""
    bslots = slots_backward(batch, T, D, ns)
    line = {
        "metric": "all-block training scan GB/s (forward over T + reverse per block)",
        "value": nbytes / (ms_per_step * 1e-3) / 1e9, "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if dtype == torch.bfloat16 else "f32", "data": "synthetic",
        "config": {"workload": args.workload, "batch": batch, "d_inner": D, "d_state": ns,
                   "seq": T, "block": L, "fused": bool(args.fused),
                   "reverse_operands": bool(args.reverse_operands)},
        "train_scan": {"ms": ev_ms, "tokens_per_s": batch * T / (ev_ms * 1e-3),
                       "GBs": nbytes / (ev_ms * 1e-3) / 1e9,
                       "valu_slot_frac": slots / (ev_ms * 1e-3) / VALU_SLOTS_PER_S,
                       "hbm_frac": nbytes / (ev_ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "train_scan_blocks": {"ms": blocks_ms, "tokens_per_s": batch * T / (blocks_ms * 1e-3),
                              "valu_slot_frac": slots / (blocks_ms * 1e-3) / VALU_SLOTS_PER_S},
        "full_scan": {"ms": full_ms, "tokens_per_s": batch * T / (full_ms * 1e-3),
                      "train_scan_over_full_scan_time": ev_ms / full_ms},
        "two_stream": {"ms": two_ms, "over_full_scan_time": two_ms / full_ms,
                       "note": "clean train_scan with h_bounds + noisy train_scan_blocks, "
                               "against one full-sequence scan of the noisy stream"},
        "backward": None if bwd_ms is None else {"train_scan_bwd_ms": bwd_ms,
                     "train_scan_bwd_valu_slot_frac": bslots / (bwd_ms * 1e-3) / VALU_SLOTS_PER_S,
                     "train_scan_blocks_bwd_ms": bbwd_ms,
                     "train_scan_blocks_bwd_valu_slot_frac": bslots / (bbwd_ms * 1e-3) / VALU_SLOTS_PER_S,
                     "bwd_over_fwd_time": bwd_ms / ev_ms},
        "all_block_training_step": None if step_ms is None else {
            "ms": step_ms, "tokens_per_s": batch * T / (step_ms * 1e-3),
            "note": "forward and backward of both streams: clean train_scan (block states), "
                    "noisy train_scan_blocks, noisy backward, clean backward fed the noisy "
                    "block-start gradients"},
    }
    return line


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
    return {"value": sample_bytes / spent / 1e9, "unit": "GB/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": "batch rows 0..%d of %d (all %d channels): prefill of %d tokens + the "
                      "block steps and commits; %.1f s wall" % (rows - 1, batch, D, ctx, spent),
            "seconds": spent}


if __name__ == "__main__":
    sys.exit(main())
