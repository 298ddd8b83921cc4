"""GPU parity of the cross-chunk carry with many chunks.

Forced 16-token chunks put hundreds of chunks on a row, so the carry runs the
segmented kernel (one wave per segment of about 12 chunks, up to 16
segments; segment maps combined through LDS; BDSSM_CARRY=tree forces it on
sequences of 64 chunks or fewer too) in each of its uses: the state-only
prefill (final state only), the prefill with outputs and train_scan (the
states entering the coarse chunks), the full-sequence scan (forward and
reverse carries) and the backward (the adjoint's reverse carry).  Every
result is checked against the oracle, with BDSSM_CARRY=serial (the
one-thread walk over the chunks) as well; the two differ only in rounding
order.  Channel counts leave the last 64-lane tile of (b, d, n) partly
filled.
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
    print("\n[parity-carry] %s" % request.node.name, flush=True)
    yield


def _h0(batch, D, n, seed):
    return synth.normal((batch, D, n), seed, "cpu", torch.float32).to("cuda").contiguous()


@pytest.mark.parametrize("carry", ["tree", "serial"])
@pytest.mark.parametrize("T,D,n,dtype,a_kind", [
    (4800, 70, 16, torch.float32, "long"),     # 300 chunks: 16 segments of 18-19 (two 8-load batches + rest)
    (4096, 64, 16, torch.float32, "default"),  # 256 chunks: 16 segments of exactly 16 (two batches)
    (1504, 37, 4, torch.bfloat16, "random"),   # 94 chunks: 8 segments of 11-12 (one batch + rest)
    (400, 130, 8, torch.float32, "default"),   # 25 chunks: 3 segments when forced
])
def test_forward_carries(dev, carry, T, D, n, dtype, a_kind, monkeypatch):
    monkeypatch.setenv("BDSSM_CHUNK", "16")
    monkeypatch.setenv("BDSSM_CARRY", carry)
    batch, L = 2, 16
    c = Case(batch, T, D, dtype, sid=91, a_kind=a_kind, n=n)
    h0 = _h0(batch, D, n, 9101)
    h_state, _ = m.prefill(*c.args(), L, h_init=h0)
    h_y, yp = m.prefill(*c.args(), L, h_init=h0, want_y=True)
    yt, bnd = m.train_scan(*c.args(), L, h_init=h0, want_bounds=True)
    yf = m.full_scan(*c.args())
    torch.cuda.synchronize()
    oa = c.oracle_args()
    r = oracle.scan(*oa, L, h0=to_np(h0), want_y=True, want_bounds=True)
    tol = TOL[dtype]
    for name, got, ref, bar in (("prefill state", h_state, r["hT"], STATE_TOL),
                                ("prefill(y) state", h_y, r["hT"], STATE_TOL),
                                ("prefill y", yp, r["y"], tol),
                                ("train_scan y", yt, r["y"], tol),
                                ("train_scan bounds", bnd, r["bounds"], STATE_TOL)):
        g = to_np(got)
        assert rel_err(g, ref) < bar, (name, worst(g, ref))
    ro = oracle.full_scan(*oa)
    assert rel_err(to_np(yf), ro) < tol, ("full_scan y", worst(to_np(yf), ro))


@pytest.mark.parametrize("carry", ["tree", "serial"])
def test_adjoint_carry(dev, carry, monkeypatch):
    """The backward's reverse carry over 200 chunks (its lowest chunk the
    last of the first coarse chunk)."""
    monkeypatch.setenv("BDSSM_CHUNK", "16")
    monkeypatch.setenv("BDSSM_COARSE_CHUNKS", "4")
    monkeypatch.setenv("BDSSM_CARRY", carry)
    batch, T, D, L = 2, 3200, 70, 16
    c = Case(batch, T, D, torch.float32, sid=92, a_kind="long")
    dy = synth.normal((batch, T, D), 9201, "cpu", torch.float32).to("cuda").contiguous()
    db = synth.normal((batch, T // L + 1, D, 16), 9202, "cpu", torch.float32).to("cuda").contiguous()
    y, bnd = m.train_scan(*c.args(), L, want_bounds=True)
    g = m.train_scan_bwd(*c.args(), L, bnd, dy, d_bounds=db, want_dh_init=True)
    torch.cuda.synchronize()
    r = oracle.scan_bwd(*c.oracle_args(), L, to_np(dy), dbounds=to_np(db))
    r["dh_init"] = r.pop("dh0")
    for k in ("dx", "ddt", "dB", "dC", "dA", "dDskip", "dh_init"):
        gk = to_np(g[k])
        assert rel_err(gk, r[k]) < TOL[torch.float32], (k, worst(gk, r[k]))


def test_tree_matches_serial(dev, monkeypatch):
    """The segmented and the one-thread carry agree to fp32 rounding on a
    long-memory problem (decays near 1 over the whole context)."""
    monkeypatch.setenv("BDSSM_CHUNK", "16")
    batch, T, D, L = 1, 8192, 96, 16
    c = Case(batch, T, D, torch.float32, sid=93, a_kind="long")
    out = {}
    for carry in ("tree", "serial"):
        monkeypatch.setenv("BDSSM_CARRY", carry)
        h, _ = m.prefill(*c.args(), L)
        yt, _ = m.train_scan(*c.args(), L)
        out[carry] = (to_np(h), to_np(yt))
    torch.cuda.synchronize()
    assert rel_err(out["tree"][0], out["serial"][0]) < 1e-5
    assert rel_err(out["tree"][1], out["serial"][1]) < 1e-5
