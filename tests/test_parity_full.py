"""GPU parity of the full-sequence bidirectional baseline (bdssm_full_scan)
in both forms of its chunk aggregates: one forward pass that forms the
forward and the reverse aggregate of every chunk together (the default with
shared operands; the reverse aggregate as the sum of each token's injection
times the product of the decays before it in the chunk) and one pass per
direction (BDSSM_FULL_AGG=separate).  Forced chunk lengths give many chunks
and a ragged last chunk; state counts 4 to 32, both stream dtypes, the
step-size fusions and long-memory A (decay products near 1 across whole
chunks) are covered, against the oracle and between the two forms.
"""
import pytest
import torch

import mamba_selective_scan_04_amd as m
import oracle
from mamba_selective_scan_04_amd import synth
from parity_util import Case, TOL, rel_err, to_np, worst

pytestmark = pytest.mark.gpu

FORMS = ["both", "separate"]


@pytest.fixture(autouse=True)
def _announce(request, dev):
    print("\n[parity-full] %s" % request.node.name, flush=True)
    yield


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("T,D,n,dtype,a_kind,chunk", [
    (1000, 70, 16, torch.float32, "long", "48"),      # 21 chunks, the last one 40 tokens
    (1024, 130, 16, torch.bfloat16, "random", "64"),
    (520, 37, 4, torch.float32, "default", "32"),
    (520, 65, 8, torch.bfloat16, "random", "160"),
    (400, 40, 32, torch.float32, "random", "80"),
    (48, 64, 16, torch.float32, "default", "100000"),  # one chunk: no aggregates
])
def test_full_scan_aggregate_forms(dev, form, T, D, n, dtype, a_kind, chunk, monkeypatch):
    monkeypatch.setenv("BDSSM_CHUNK", chunk)
    monkeypatch.setenv("BDSSM_FULL_AGG", form)
    c = Case(2, T, D, dtype, sid=95, a_kind=a_kind, n=n)
    y = m.full_scan(*c.args())
    torch.cuda.synchronize()
    ref = oracle.full_scan(*c.oracle_args())
    g = to_np(y)
    assert rel_err(g, ref) < TOL[dtype], worst(g, ref)


@pytest.mark.parametrize("mode", ["softplus_bias", "bias"])
def test_full_scan_fused_step_size(dev, mode, monkeypatch):
    """dt = softplus(dt_raw + bias) (or dt_raw + bias) formed inside both
    aggregate forms and the sweeps, the output gated by silu(z)."""
    monkeypatch.setenv("BDSSM_CHUNK", "64")
    batch, T, D = 2, 704, 100
    c = Case(batch, T, D, torch.float32, sid=96, a_kind="random")
    mean, std = (1.0, 0.1) if mode == "bias" else (-1.0, 0.5)
    c.dev["dt"] = synth.normal((batch, T, D), 9601, "cpu", torch.float32, mean=mean, std=std).to("cuda")
    bias = synth.normal((D,), 9602, "cpu", torch.float32, std=0.1).to("cuda")
    z = synth.normal((batch, T, D), 9603, "cpu", torch.float32).to("cuda")
    kw = dict(dt_bias=bias, dt_softplus=(mode == "softplus_bias"), z=z)
    out = {}
    for form in FORMS:
        monkeypatch.setenv("BDSSM_FULL_AGG", form)
        out[form] = to_np(m.full_scan(*c.args(), **kw))
    torch.cuda.synchronize()
    ref = oracle.full_scan(*c.oracle_args(), dt_bias=to_np(bias), dt_softplus=kw["dt_softplus"],
                           z=synth.to_oracle(z))
    for form in FORMS:
        assert rel_err(out[form], ref) < TOL[torch.float32], (form, worst(out[form], ref))
    assert rel_err(out["both"], out["separate"]) < 1e-5


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("a_kind", ["zero", "steep"])
def test_full_scan_decay_extremes(dev, form, a_kind, monkeypatch):
    """A = 0 (every decay exactly 1: the decay product stays 1 and the
    reverse aggregate is the plain sum of the chunk's injections) and a
    steep A (-1000 (n + 1): decays underflow to zero within a token, so the
    running product does too)."""
    monkeypatch.setenv("BDSSM_CHUNK", "48")
    monkeypatch.setenv("BDSSM_FULL_AGG", form)
    c = Case(2, 960, 72, torch.float32, sid=97, a_kind="zero" if a_kind == "zero" else "default")
    if a_kind == "steep":
        c.dev["A"] = (c.dev["A"] * 1000.0).contiguous()
    y = m.full_scan(*c.args())
    torch.cuda.synchronize()
    ref = oracle.full_scan(*c.oracle_args())
    g = to_np(y)
    assert rel_err(g, ref) < TOL[torch.float32], worst(g, ref)
