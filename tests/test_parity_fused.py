"""GPU parity of the optional Mamba-1 fusions (dt = softplus(dt_raw + bias),
dt = dt_raw + bias, y * silu(z)) on every forward entry point, against the
fp64 oracle with the same fusions, on seeded inputs with forced multi-chunk
plans (so the fused chunk kernels, the carry and the fused output passes all
run), ragged channel counts and a wide range of softplus arguments.
"""
import numpy as np
import pytest
import torch

import mamba_selective_scan_04_amd as m
import oracle
from mamba_selective_scan_04_amd import synth
from parity_util import Case, N, STATE_TOL, TOL, rel_err, to_np, worst

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request, dev):
    print("\n[parity-fused] %s" % request.node.name, flush=True)
    yield


def fused_case(batch, T, D, dtype, sid, mode, raw_range=None):
    """Case whose dt stream holds the raw step size for the given mode."""
    c = Case(batch, T, D, dtype, sid=sid, a_kind="random")
    if raw_range is not None:
        lo, hi = raw_range
        raw = torch.linspace(lo, hi, batch * T * D).reshape(batch, T, D)
        raw = raw[:, :, torch.randperm(D, generator=torch.Generator().manual_seed(sid))]
    elif mode == "bias":
        # without softplus the caller keeps dt positive: raw around 1, small bias
        raw = synth.normal((batch, T, D), 1000 * sid + 60, "cpu", torch.float32, mean=1.0, std=0.1)
    else:
        raw = synth.normal((batch, T, D), 1000 * sid + 60, "cpu", torch.float32, mean=-1.0, std=0.5)
    c.dev["dt"] = raw.to(dtype).to("cuda").contiguous()
    bias = None
    if mode in ("softplus_bias", "bias"):
        std = 0.05 if mode == "bias" else 0.3
        bias = synth.normal((D,), 1000 * sid + 61, "cpu", torch.float32, std=std).to("cuda")
    z = synth.normal((batch, T, D), 1000 * sid + 62, "cpu", torch.float32, std=2.0).to(dtype).to("cuda")
    kw = dict(dt_bias=bias, dt_softplus=mode != "bias", z=z)
    return c, kw


def oracle_kw(kw, t0=None, t1=None):
    z = kw["z"]
    if t0 is not None:
        z = z[:, t0:t1]
    return dict(dt_bias=None if kw["dt_bias"] is None else to_np(kw["dt_bias"]),
                dt_softplus=kw["dt_softplus"], z=synth.to_oracle(z))


def sub(kw, t0, t1):
    out = dict(kw)
    out["z"] = kw["z"][:, t0:t1].clone(memory_format=torch.contiguous_format)
    return out


MODES = ["softplus_bias", "softplus", "bias"]


# the bidirectional pass on bidir_pair_kernel (two states per lane, the
# default) and on bidir_wave_kernel (four states per lane)
BIDIR = ["pair", "wave"]


@pytest.mark.parametrize("bidir", BIDIR)
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("mode", MODES)
def test_fused_training_and_baseline_forms(dev, dtype, mode, bidir, monkeypatch):
    monkeypatch.setenv("BDSSM_CHUNK", "64")
    monkeypatch.setenv("BDSSM_BIDIR_KERNEL", bidir)
    batch, T, D, L = 2, 512, 130, 16
    c, kw = fused_case(batch, T, D, dtype, 51, mode)
    y, bnd = m.train_scan(*c.args(), L, want_bounds=True, **kw)
    h0b = synth.normal((batch, T // L + 1, D, N), 5163, "cuda")
    yb = m.train_scan_blocks(*c.args(), L, h0b, **kw)
    yfull = m.full_scan(*c.args(), **kw)
    torch.cuda.synchronize()
    oa = c.oracle_args()
    ok = oracle_kw(kw)
    yo, bo = oracle.train_scan(*oa, L, want_bounds=True, **ok)
    ybo = oracle.train_blocks(*oa, L, to_np(h0b), **ok)
    yfo = oracle.full_scan(*oa, **ok)
    tol = TOL[dtype]
    assert rel_err(to_np(y), yo) < tol, worst(to_np(y), yo)
    assert rel_err(to_np(bnd), bo) < STATE_TOL, worst(to_np(bnd), bo)
    assert rel_err(to_np(yb), ybo) < tol, worst(to_np(yb), ybo)
    assert rel_err(to_np(yfull), yfo) < tol, worst(to_np(yfull), yfo)


@pytest.mark.parametrize("bidir", BIDIR)
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("mode", MODES)
def test_fused_inference_cycle(dev, dtype, mode, bidir, monkeypatch):
    """prefill (state only and with y), block step, commit (with and without y)."""
    monkeypatch.setenv("BDSSM_CHUNK", "64")
    monkeypatch.setenv("BDSSM_BIDIR_KERNEL", bidir)
    batch, D, L, P = 2, 200, 16, 480
    T = P + 2 * L
    c, kw = fused_case(batch, T, D, dtype, 52, mode)
    seg = c.segment(0, P)
    h, yp = m.prefill(*seg, L, want_y=True, **sub(kw, 0, P))
    h2, _ = m.prefill(*seg, L, **sub(kw, 0, P))
    blk = c.segment(P, P + L)
    ys = m.block_step(h, *blk, **sub(kw, P, P + L))
    hc = h.clone()
    _, yc = m.commit(hc, *blk, want_y=True, **sub(kw, P, P + L))
    blk2 = c.segment(P + L, T)
    hc2 = hc.clone()
    m.commit(hc2, *blk2, **sub(kw, P + L, T))
    torch.cuda.synchronize()
    tol = TOL[dtype]
    oa = c.oracle_args(0, P)
    ho, ypo = oracle.prefill(*oa, L, want_y=True, **oracle_kw(kw, 0, P))
    assert rel_err(to_np(h), ho) < STATE_TOL, worst(to_np(h), ho)
    assert rel_err(to_np(h2), ho) < STATE_TOL
    assert rel_err(to_np(yp), ypo) < tol, worst(to_np(yp), ypo)
    ob = c.oracle_args(P, P + L)
    yso = oracle.block_step(ho, *ob, **oracle_kw(kw, P, P + L))
    assert rel_err(to_np(ys), yso) < tol, worst(to_np(ys), yso)
    hco, yco = oracle.commit(ho, *ob, want_y=True, **oracle_kw(kw, P, P + L))
    assert rel_err(to_np(yc), yco) < tol
    assert rel_err(to_np(hc), hco) < STATE_TOL
    hco2, _ = oracle.commit(hco, *c.oracle_args(P + L, T), **oracle_kw(kw, P + L, T))
    assert rel_err(to_np(hc2), hco2) < STATE_TOL


def test_softplus_over_a_wide_range(dev, monkeypatch):
    """Raw step sizes from -20 to 8: softplus runs from ~2e-9 (nearly no
    step) to ~8; fp32 streams so the transform itself is what is checked."""
    monkeypatch.setenv("BDSSM_CHUNK", "64")
    batch, T, D, L = 1, 256, 64, 16
    c, kw = fused_case(batch, T, D, torch.float32, 53, "softplus", raw_range=(-20.0, 8.0))
    kw["z"] = None
    y, bnd = m.train_scan(*c.args(), L, want_bounds=True, **kw)
    h, _ = m.prefill(*c.args(), L, **kw)
    torch.cuda.synchronize()
    ok = dict(dt_softplus=True)
    yo, bo = oracle.train_scan(*c.oracle_args(), L, want_bounds=True, **ok)
    ho, _ = oracle.prefill(*c.oracle_args(), L, **ok)
    assert rel_err(to_np(y), yo) < TOL[torch.float32], worst(to_np(y), yo)
    assert rel_err(to_np(bnd), bo) < STATE_TOL, worst(to_np(bnd), bo)
    assert rel_err(to_np(h), ho) < STATE_TOL


def test_no_fusion_arguments_is_bitwise_unfused(dev):
    """dt_bias = None, dt_softplus = False, z = None takes the unfused path."""
    c = Case(2, 256, 96, torch.bfloat16, sid=54)
    y1, _ = m.train_scan(*c.args(), 16)
    y2, _ = m.train_scan(*c.args(), 16, dt_bias=None, dt_softplus=False, z=None)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


# ---- separate reverse-direction operands

def rev_case(c, batch, T, D, dtype, sid, with_bias):
    dt_r = synth.positive_step((batch, T, D), 1000 * sid + 80, "cpu", dtype)
    B_r = synth.normal((batch, T, N), 1000 * sid + 81, "cpu", dtype)
    C_r = synth.normal((batch, T, N), 1000 * sid + 82, "cpu", dtype)
    A_r = synth.a_matrix(D, N, "random", seed=1000 * sid + 83)
    rev = {k: v.to("cuda").contiguous() for k, v in dict(dt=dt_r, B=B_r, C=C_r, A=A_r).items()}
    if with_bias:
        rev["dt_bias"] = synth.normal((D,), 1000 * sid + 84, "cuda", torch.float32, std=0.05)
    return rev


def rev_oracle(rev, t0=None, t1=None):
    sl = (lambda t: t) if t0 is None else (lambda t: t[:, t0:t1])
    out = dict(dt=synth.to_oracle(sl(rev["dt"])), B=synth.to_oracle(sl(rev["B"])),
               C=synth.to_oracle(sl(rev["C"])), A=synth.to_oracle(rev["A"]))
    if "dt_bias" in rev:
        out["dt_bias"] = to_np(rev["dt_bias"])
    return out


def rev_sub(rev, t0, t1):
    out = dict(rev)
    for k in ("dt", "B", "C"):
        out[k] = rev[k][:, t0:t1].clone(memory_format=torch.contiguous_format)
    return out


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("fused", [False, True])
def test_reverse_operands_training_and_baseline(dev, dtype, fused, monkeypatch):
    monkeypatch.setenv("BDSSM_CHUNK", "64")
    batch, T, D, L = 2, 512, 130, 16
    c = Case(batch, T, D, dtype, sid=55, a_kind="random")
    rev = rev_case(c, batch, T, D, dtype, 55, with_bias=fused)
    kw = dict(rev=rev)
    ok = dict(rev=rev_oracle(rev))
    if fused:
        # both dt streams go through softplus with their own bias (positive
        # inputs: the steps stay positive), and the output is gated
        z = synth.normal((batch, T, D), 5590, "cuda", dtype)
        bias = synth.normal((D,), 5591, "cuda", torch.float32, std=0.3)
        kw.update(dt_bias=bias, dt_softplus=True, z=z)
        ok.update(dt_bias=to_np(bias), dt_softplus=True, z=synth.to_oracle(z))
    y, bnd = m.train_scan(*c.args(), L, want_bounds=True, **kw)
    h0b = synth.normal((batch, T // L + 1, D, N), 5592, "cuda")
    yb = m.train_scan_blocks(*c.args(), L, h0b, **kw)
    yfull = m.full_scan(*c.args(), **kw)
    torch.cuda.synchronize()
    oa = c.oracle_args()
    yo, bo = oracle.train_scan(*oa, L, want_bounds=True, **ok)
    ybo = oracle.train_blocks(*oa, L, to_np(h0b), **ok)
    yfo = oracle.full_scan(*oa, **ok)
    tol = TOL[dtype]
    assert rel_err(to_np(y), yo) < tol, worst(to_np(y), yo)
    assert rel_err(to_np(bnd), bo) < STATE_TOL
    assert rel_err(to_np(yb), ybo) < tol, worst(to_np(yb), ybo)
    assert rel_err(to_np(yfull), yfo) < tol, worst(to_np(yfull), yfo)


@pytest.mark.parametrize("L", [4, 16])
def test_reverse_operands_inference_cycle(dev, L, monkeypatch):
    monkeypatch.setenv("BDSSM_CHUNK", "64")
    batch, D, P = 2, 96, 256
    T = P + L
    dtype = torch.bfloat16
    c = Case(batch, T, D, dtype, sid=56, a_kind="random")
    rev = rev_case(c, batch, T, D, dtype, 56, with_bias=False)
    h, yp = m.prefill(*c.segment(0, P), L, want_y=True, rev=rev_sub(rev, 0, P))
    ys = m.block_step(h, *c.segment(P, T), rev=rev_sub(rev, P, T))
    hc = h.clone()
    _, yc = m.commit(hc, *c.segment(P, T), want_y=True, rev=rev_sub(rev, P, T))
    torch.cuda.synchronize()
    ho, ypo = oracle.prefill(*c.oracle_args(0, P), L, want_y=True, rev=rev_oracle(rev, 0, P))
    assert rel_err(to_np(h), ho) < STATE_TOL
    assert rel_err(to_np(yp), ypo) < TOL[dtype], worst(to_np(yp), ypo)
    yso = oracle.block_step(ho, *c.oracle_args(P, T), rev=rev_oracle(rev, P, T))
    assert rel_err(to_np(ys), yso) < TOL[dtype], worst(to_np(ys), yso)
    hco, yco = oracle.commit(ho, *c.oracle_args(P, T), want_y=True, rev=rev_oracle(rev, P, T))
    assert rel_err(to_np(yc), yco) < TOL[dtype]
    assert rel_err(to_np(hc), hco) < STATE_TOL
