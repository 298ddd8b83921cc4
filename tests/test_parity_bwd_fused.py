"""GPU parity of the backward entry points with the forward's fusions in
place (the step size softplus(dt + bias) or dt + bias, and the silu(z) output
gate) against the fp64 oracle's gradients, element by element: ddt is then
the gradient of the raw dt stream, and the backward also returns d_dt_bias
and dz.  Both training forms, every supported block length, forced
multi-chunk plans (the adjoint carry sees the fused step sizes and the
gate), ragged channel counts and a ragged last 16-token group.

The oracle receives the same input values as the GPU (read back from the
device tensors); dy, d_bounds, the two-stream block starts, the bias and the
gate are seeded inputs.
"""
import pytest
import torch

import mamba_selective_scan_04_amd as m
import oracle
from mamba_selective_scan_04_amd import synth
from parity_util import Case, N, STATE_TOL, TOL, rel_err, to_np, worst

pytestmark = pytest.mark.gpu

GRADS = ("dx", "ddt", "dB", "dC")
PARAM_GRADS = ("dA", "dDskip")

# name -> (softplus, bias, gate)
MODES = {"softplus_bias_gate": (True, True, True), "softplus_gate": (True, False, True),
         "softplus_bias": (True, True, False), "bias_gate": (False, True, True),
         "gate_only": (False, False, True), "bias_only": (False, True, False)}


@pytest.fixture(autouse=True)
def _announce(request, dev):
    print("\n[parity-bwd-fused] %s" % request.node.name, flush=True)
    yield


def seeded(shape, seed, dtype=torch.float32, std=1.0):
    return synth.normal(shape, seed, "cpu", dtype, std=std).to("cuda").contiguous()


def check(got, ref, names, tol, label=""):
    for k in names:
        g = to_np(got[k])
        assert g.shape == ref[k].shape, (label, k, g.shape, ref[k].shape)
        e = rel_err(g, ref[k])
        assert e < tol, (label, k, e, worst(g, ref[k]))


def fused_case(batch, T, D, dtype, sid, mode):
    """Seeded inputs for one fusion mode -> (Case, GPU kwargs, oracle kwargs).
    With softplus the dt stream is the raw pre-activation (either sign);
    without it the bias is small and positive so the step stays positive."""
    softplus, with_bias, with_gate = MODES[mode]
    c = Case(batch, T, D, dtype, sid=sid, a_kind="random")
    if softplus:
        c.dev["dt"] = synth.normal((batch, T, D), 1000 * sid + 11, "cpu", torch.float32, mean=-1.0,
                                   std=0.8).to(dtype).to("cuda").contiguous()
    kw, ok = {}, {}
    if softplus:
        kw["dt_softplus"] = ok["dt_softplus"] = True
    if with_bias:
        bias = seeded((D,), 1000 * sid + 12, std=0.3 if softplus else 0.02)
        if not softplus:
            bias = bias.abs()
        kw["dt_bias"], ok["dt_bias"] = bias, to_np(bias)
    if with_gate:
        z = seeded((batch, T, D), 1000 * sid + 13, dtype, std=1.5)
        kw["z"], ok["z"] = z, synth.to_oracle(z)
    return c, kw, ok


def fused_names(mode):
    _, with_bias, with_gate = MODES[mode]
    return (("d_dt_bias",) if with_bias else ()), (("dz",) if with_gate else ())


def run_both_forms(c, L, mode, kw, ok, dy, db, h0b, label):
    """Continuous form (with d_bounds, dh_init) and two-stream form, GPU vs
    oracle, for one case."""
    mode_bias, mode_gate = fused_names(mode)
    tol = TOL[c.dtype]
    _, bnd = m.train_scan(*c.args(), L, want_bounds=True, **kw)
    g = m.train_scan_bwd(*c.args(), L, bnd, dy, d_bounds=db, want_dh_init=True, **kw)
    gb = m.train_scan_blocks_bwd(*c.args(), L, h0b, dy, want_dh0_blocks=True, **kw)
    torch.cuda.synchronize()
    oa = c.oracle_args()
    r = oracle.scan_bwd(*oa, L, to_np(dy), dbounds=to_np(db), **ok)
    r["dh_init"] = r.pop("dh0")
    rb = oracle.scan_bwd(*oa, L, to_np(dy), h0_blocks=to_np(h0b), **ok)
    check(g, r, GRADS + mode_gate, tol, label)
    check(g, r, PARAM_GRADS + ("dh_init",) + mode_bias, STATE_TOL, label)
    check(gb, rb, GRADS + mode_gate, tol, label + " blocks")
    check(gb, rb, PARAM_GRADS + ("dh0_blocks",) + mode_bias, STATE_TOL, label + " blocks")
    for k in mode_bias + mode_gate:
        assert k in g and k in gb, k


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("mode", list(MODES))
def test_fused_bwd_modes(dev, mode, dtype, monkeypatch):
    """Every fusion mode, both dtypes, L = 16, several coarse chunks."""
    monkeypatch.setenv("BDSSM_CHUNK", "64")
    monkeypatch.setenv("BDSSM_COARSE_CHUNKS", "3")
    batch, T, D, L = 2, 448, 100, 16
    c, kw, ok = fused_case(batch, T, D, dtype, 51, mode)
    dy = seeded((batch, T, D), 5101, dtype)
    db = seeded((batch, T // L + 1, D, N), 5102)
    h0b = seeded((batch, T // L + 1, D, N), 5103)
    run_both_forms(c, L, mode, kw, ok, dy, db, h0b, mode)


@pytest.mark.parametrize("L", [1, 2, 4, 8])
def test_fused_bwd_block_lengths(dev, L, monkeypatch):
    """Softplus, bias and gate at the short block lengths, with a ragged last
    16-token group."""
    monkeypatch.setenv("BDSSM_CHUNK", "64")
    monkeypatch.setenv("BDSSM_COARSE_CHUNKS", "3")
    batch, T, D = 2, 456, 70
    c, kw, ok = fused_case(batch, T, D, torch.bfloat16, 52, "softplus_bias_gate")
    dy = seeded((batch, T, D), 5201 + L, torch.bfloat16)
    db = seeded((batch, T // L + 1, D, N), 5210 + L)
    h0b = seeded((batch, T // L + 1, D, N), 5220 + L)
    run_both_forms(c, L, "softplus_bias_gate", kw, ok, dy, db, h0b, "L=%d" % L)


@pytest.mark.parametrize("D", [1, 33, 200])
def test_fused_bwd_ragged_channels(dev, D):
    batch, T, L = 2, 96, 16
    c, kw, ok = fused_case(batch, T, D, torch.float32, 53, "softplus_bias_gate")
    dy = seeded((batch, T, D), 5301)
    db = seeded((batch, T // L + 1, D, N), 5302)
    h0b = seeded((batch, T // L + 1, D, N), 5303)
    run_both_forms(c, L, "softplus_bias_gate", kw, ok, dy, db, h0b, "D=%d" % D)


def test_fused_bwd_is_deterministic(dev, monkeypatch):
    monkeypatch.setenv("BDSSM_CHUNK", "64")
    monkeypatch.setenv("BDSSM_COARSE_CHUNKS", "4")
    batch, T, D, L = 2, 512, 130, 16
    c, kw, _ = fused_case(batch, T, D, torch.bfloat16, 54, "softplus_bias_gate")
    dy = seeded((batch, T, D), 5401, torch.bfloat16)
    _, bnd = m.train_scan(*c.args(), L, want_bounds=True, **kw)
    g1 = m.train_scan_bwd(*c.args(), L, bnd, dy, want_dh_init=True, **kw)
    g2 = m.train_scan_bwd(*c.args(), L, bnd, dy, want_dh_init=True, **kw)
    torch.cuda.synchronize()
    assert set(g1) == set(g2)
    for k in g1:
        assert torch.equal(g1[k], g2[k]), k


def test_fused_bwd_empty_sequence(dev):
    batch, D, L = 2, 64, 16
    c, kw, _ = fused_case(batch, 0, D, torch.float32, 55, "softplus_bias_gate")
    bnd = seeded((batch, 1, D, N), 5501)
    db = seeded((batch, 1, D, N), 5502)
    dy = torch.empty(batch, 0, D, device="cuda")
    g = m.train_scan_bwd(*c.args(), L, bnd, dy, d_bounds=db, want_dh_init=True, **kw)
    torch.cuda.synchronize()
    assert torch.count_nonzero(g["d_dt_bias"]) == 0
    assert g["dz"].shape == (batch, 0, D)
    assert torch.equal(g["dh_init"], db[:, 0])

