"""GPU parity of state counts other than 16 (d_state 4, 8 and 32: the
one-lane-per-channel kernels instantiated per state count) on every forward
entry point and the baseline, against the fp64 oracle, element by element:
block lengths inside and outside {1, 2, 4, 8, 16}, forced multi-chunk plans,
ragged channel counts, the two-stream form, the fusions and separate reverse
operands.  The backward of these state counts is covered by
test_parity_bwd_general.py.
"""
import pytest
import torch

import mamba_selective_scan_04_amd as m
import oracle
from mamba_selective_scan_04_amd import synth
from parity_util import Case, STATE_TOL, TOL, rel_err, to_np, worst

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request, dev):
    print("\n[parity-dstate] %s" % request.node.name, flush=True)
    yield


def close(got, ref, tol, what):
    g = to_np(got)
    assert g.shape == ref.shape, (what, g.shape, ref.shape)
    e = rel_err(g, ref)
    assert e < tol, (what, e, worst(g, ref))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("n", [4, 8, 32])
@pytest.mark.parametrize("L", [16, 4, 24])
def test_training_and_baseline(dev, dtype, n, L, monkeypatch):
    monkeypatch.setenv("BDSSM_CHUNK", "64")
    batch, T, D = 2, 384, 130
    c = Case(batch, T, D, dtype, sid=71, a_kind="random", n=n)
    y, bnd = m.train_scan(*c.args(), L, want_bounds=True)
    h0b = synth.normal((batch, T // L + 1, D, n), 7101, "cuda")
    yb = m.train_scan_blocks(*c.args(), L, h0b)
    yf = m.full_scan(*c.args())
    torch.cuda.synchronize()
    oa = c.oracle_args()
    yo, bo = oracle.train_scan(*oa, L, want_bounds=True)
    close(y, yo, TOL[dtype], "train_scan y")
    close(bnd, bo, STATE_TOL, "h_bounds")
    close(yb, oracle.train_blocks(*oa, L, to_np(h0b)), TOL[dtype], "two-stream y")
    close(yf, oracle.full_scan(*oa), TOL[dtype], "full_scan y")


@pytest.mark.parametrize("n", [4, 8, 32])
@pytest.mark.parametrize("L", [16, 12])
def test_inference_cycle(dev, n, L, monkeypatch):
    monkeypatch.setenv("BDSSM_CHUNK", "64")
    batch, D, P = 2, 96, 240
    T = P + 2 * L
    dtype = torch.bfloat16
    c = Case(batch, T, D, dtype, sid=72, a_kind="random", n=n)
    h, yp = m.prefill(*c.segment(0, P), L, want_y=True)
    h2, _ = m.prefill(*c.segment(0, P), L)
    ys = m.block_step(h, *c.segment(P, P + L))
    hc = h.clone()
    _, yc = m.commit(hc, *c.segment(P, P + L), want_y=True)
    hc2 = hc.clone()
    m.commit(hc2, *c.segment(P + L, T))
    torch.cuda.synchronize()
    tol = TOL[dtype]
    ho, ypo = oracle.prefill(*c.oracle_args(0, P), L, want_y=True)
    close(h, ho, STATE_TOL, "prefill state")
    close(h2, ho, STATE_TOL, "prefill state (state only)")
    close(yp, ypo, tol, "prefill y")
    close(ys, oracle.block_step(ho, *c.oracle_args(P, P + L)), tol, "block_step y")
    hco, yco = oracle.commit(ho, *c.oracle_args(P, P + L), want_y=True)
    close(yc, yco, tol, "commit y")
    close(hc, hco, STATE_TOL, "commit state")
    hco2, _ = oracle.commit(hco, *c.oracle_args(P + L, T))
    close(hc2, hco2, STATE_TOL, "commit state (no y)")


@pytest.mark.parametrize("D", [1, 65])
def test_ragged_channels_long_memory(dev, D):
    batch, T, L, n = 2, 256, 16, 8
    c = Case(batch, T, D, torch.float32, sid=73, a_kind="long", n=n)
    h0 = synth.normal((batch, D, n), 7301, "cuda")
    y, bnd = m.train_scan(*c.args(), L, h_init=h0, want_bounds=True)
    torch.cuda.synchronize()
    yo, bo = oracle.train_scan(*c.oracle_args(), L, h_init=to_np(h0), want_bounds=True)
    close(y, yo, TOL[torch.float32], "y")
    close(bnd, bo, STATE_TOL, "h_bounds")


def test_fusions_and_reverse_operands(dev, monkeypatch):
    """n = 8: softplus(dt_raw + bias), gate, separate reverse operands."""
    monkeypatch.setenv("BDSSM_CHUNK", "64")
    batch, T, D, L, n = 2, 320, 80, 16, 8
    dtype = torch.bfloat16
    c = Case(batch, T, D, dtype, sid=74, a_kind="random", n=n)
    c.dev["dt"] = synth.normal((batch, T, D), 7401, "cpu", torch.float32, mean=-1.0,
                               std=0.5).to(dtype).to("cuda").contiguous()
    bias = synth.normal((D,), 7402, "cuda", torch.float32, std=0.3)
    z = synth.normal((batch, T, D), 7403, "cuda", dtype, std=2.0)
    rev = dict(dt=synth.normal((batch, T, D), 7404, "cuda", dtype, mean=-1.0, std=0.5),
               B=synth.normal((batch, T, n), 7405, "cuda", dtype),
               C=synth.normal((batch, T, n), 7406, "cuda", dtype),
               A=synth.a_matrix(D, n, "random", seed=7407).to("cuda"),
               dt_bias=synth.normal((D,), 7408, "cuda", torch.float32, std=0.3))
    kw = dict(dt_bias=bias, dt_softplus=True, z=z, rev=rev)
    ro = dict(dt=synth.to_oracle(rev["dt"]), B=synth.to_oracle(rev["B"]), C=synth.to_oracle(rev["C"]),
              A=synth.to_oracle(rev["A"]), dt_bias=to_np(rev["dt_bias"]))
    ok = dict(dt_bias=to_np(bias), dt_softplus=True, z=synth.to_oracle(z), rev=ro)
    y, bnd = m.train_scan(*c.args(), L, want_bounds=True, **kw)
    yf = m.full_scan(*c.args(), **kw)
    torch.cuda.synchronize()
    oa = c.oracle_args()
    yo, bo = oracle.train_scan(*oa, L, want_bounds=True, **ok)
    close(y, yo, TOL[dtype], "train_scan y")
    close(bnd, bo, STATE_TOL, "h_bounds")
    close(yf, oracle.full_scan(*oa, **ok), TOL[dtype], "full_scan y")

