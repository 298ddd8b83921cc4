"""GPU parity of the backward with separate reverse-direction operands
(dt_r with its own bias, B_r, C_r, A_r) against the fp64 oracle's gradients,
element by element: both training forms, with and without the step-size and
gate fusions, several state counts and block lengths (including 16 and 16,
which this case also runs on the general kernel), forced multi-chunk plans.
Every gradient term splits by direction: ddt, dB, dC, dA for the forward
operands, ddt_rev, dB_rev, dC_rev, dA_rev (and d_dt_bias_rev) for the reverse.
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
    print("\n[parity-bwd-rev] %s" % request.node.name, flush=True)
    yield


def seeded(shape, seed, dtype=torch.float32, std=1.0, mean=0.0):
    return synth.normal(shape, seed, "cpu", dtype, mean=mean, std=std).to("cuda").contiguous()


def check(got, ref, names, tol, label=""):
    for k in names:
        g = to_np(got[k])
        assert g.shape == ref[k].shape, (label, k, g.shape, ref[k].shape)
        e = rel_err(g, ref[k])
        assert e < tol, (label, k, e, worst(g, ref[k]))


CASES = [  # (N, L, T, D, dtype, fused)
    (16, 16, 256, 70, torch.bfloat16, True),
    (16, 16, 192, 130, torch.float32, False),
    (8, 24, 480, 50, torch.bfloat16, True),
    (32, 48, 480, 33, torch.float32, True),
    (4, 5, 200, 100, torch.bfloat16, False),
]


@pytest.mark.parametrize("N,L,T,D,dtype,fused", CASES)
def test_backward_with_separate_reverse_operands(dev, N, L, T, D, dtype, fused, monkeypatch):
    monkeypatch.setenv("BDSSM_CHUNK", "64")
    batch = 2
    sid = 110 + CASES.index((N, L, T, D, dtype, fused))
    c = Case(batch, T, D, dtype, sid=sid, a_kind="random", n=N)
    s = 1000 * sid
    rev = dict(dt=seeded((batch, T, D), s + 31, dtype, 0.5, -1.0) if fused else
               synth.positive_step((batch, T, D), s + 31, "cuda", dtype),
               B=seeded((batch, T, N), s + 32, dtype), C=seeded((batch, T, N), s + 33, dtype),
               A=synth.a_matrix(D, N, "random", seed=s + 34).to("cuda"))
    kw, ok = {}, {}
    if fused:
        c.dev["dt"] = seeded((batch, T, D), s + 35, dtype, 0.8, -1.0)
        rev["dt_bias"] = seeded((D,), s + 36, std=0.3)
        bias = seeded((D,), s + 37, std=0.3)
        z = seeded((batch, T, D), s + 38, dtype, 1.5)
        kw = dict(dt_bias=bias, dt_softplus=True, z=z)
        ok = dict(dt_bias=to_np(bias), dt_softplus=True, z=synth.to_oracle(z))
    kw["rev"] = rev
    ok["rev"] = dict(dt=synth.to_oracle(rev["dt"]), B=synth.to_oracle(rev["B"]),
                     C=synth.to_oracle(rev["C"]), A=synth.to_oracle(rev["A"]),
                     dt_bias=to_np(rev["dt_bias"]) if "dt_bias" in rev else None)
    dy = seeded((batch, T, D), s + 21, dtype)
    db = seeded((batch, T // L + 1, D, N), s + 22)
    h0b = seeded((batch, T // L + 1, D, N), s + 23)
    _, bnd = m.train_scan(*c.args(), L, want_bounds=True, **kw)
    g = m.train_scan_bwd(*c.args(), L, bnd, dy, d_bounds=db, want_dh_init=True, **kw)
    gb = m.train_scan_blocks_bwd(*c.args(), L, h0b, dy, want_dh0_blocks=True, **kw)
    torch.cuda.synchronize()
    oa = c.oracle_args()
    r = oracle.scan_bwd(*oa, L, to_np(dy), dbounds=to_np(db), **ok)
    r["dh_init"] = r.pop("dh0")
    rb = oracle.scan_bwd(*oa, L, to_np(dy), h0_blocks=to_np(h0b), **ok)
    streams = ("dx", "ddt", "dB", "dC", "ddt_rev", "dB_rev", "dC_rev") + (("dz",) if fused else ())
    params = ("dA", "dDskip", "dA_rev") + (("d_dt_bias", "d_dt_bias_rev") if fused else ())
    label = "N=%d L=%d fused=%s" % (N, L, fused)
    check(g, r, streams, TOL[dtype], label)
    check(g, r, params + ("dh_init",), STATE_TOL, label)
    check(gb, rb, streams, TOL[dtype], label + " blocks")
    check(gb, rb, params + ("dh0_blocks",), STATE_TOL, label + " blocks")


def test_separate_operands_equal_to_the_forwards_match_the_shared_backward(dev):
    """Reverse operands identical to the forward's: each shared gradient is the
    sum of the two directions' parts of the separate-operand backward."""
    batch, T, D, L, N = 2, 256, 70, 16, 16
    c = Case(batch, T, D, torch.float32, sid=120, a_kind="random")
    rev = dict(dt=c.dev["dt"].clone(), B=c.dev["B"].clone(), C=c.dev["C"].clone(), A=c.dev["A"].clone())
    dy = seeded((batch, T, D), 120021)
    _, bnd = m.train_scan(*c.args(), L, want_bounds=True)
    g0 = m.train_scan_bwd(*c.args(), L, bnd, dy, want_dh_init=True)
    g1 = m.train_scan_bwd(*c.args(), L, bnd, dy, want_dh_init=True, rev=rev)
    torch.cuda.synchronize()
    for k, kr in (("ddt", "ddt_rev"), ("dB", "dB_rev"), ("dC", "dC_rev"), ("dA", "dA_rev")):
        assert rel_err(to_np(g1[k]) + to_np(g1[kr]), to_np(g0[k])) < 1e-4, k
    for k in ("dx", "dDskip", "dh_init"):
        assert rel_err(to_np(g1[k]), to_np(g0[k])) < 1e-4, k
