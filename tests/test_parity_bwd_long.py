"""GPU parity of the long-block backward (block lengths that are multiples of
16 above 16, 16 states: group_state_kernel, then bwd_pair_kernel walking each
block's 16-token groups from the right with the reverse state carried between
them) against the fp64 oracle's gradients, element by element: both training
forms, d_bounds, forced multi-chunk plans (the general adjoint pre-pass and
the carry), ragged channel counts, one-group-per-block edge cases excluded by
construction (L > 16), and the fusions.  The same cases on the general kernel
(BDSSM_BWD_KERNEL=general) must agree with it to rounding.
"""
import pytest
import torch

import mamba_selective_scan_04_amd as m
from mamba_selective_scan_04_amd import synth
from parity_util import Case, to_np
from test_parity_bwd_general import both_forms, seeded

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request, dev):
    print("\n[parity-bwd-long] %s" % request.node.name, flush=True)
    yield


CASES = [  # (L, T, D, dtype, chunk)
    (32, 512, 65, torch.bfloat16, "64"),
    (48, 480, 33, torch.float32, "64"),
    (64, 1024, 100, torch.bfloat16, "128"),
    (256, 512, 40, torch.float32, "64"),
    (32, 256, 130, torch.float32, None),
    (128, 640, 70, torch.bfloat16, "256"),
]


@pytest.mark.parametrize("L,T,D,dtype,chunk", CASES)
def test_long_block_backward(dev, L, T, D, dtype, chunk, monkeypatch):
    if chunk is not None:
        monkeypatch.setenv("BDSSM_CHUNK", chunk)
    sid = 300 + CASES.index((L, T, D, dtype, chunk))
    c = Case(2, T, D, dtype, sid=sid, a_kind="random", n=16)
    both_forms(c, L, sid, label="long L=%d" % L)


@pytest.mark.parametrize("L", [32, 96])
def test_long_block_backward_long_memory(dev, L):
    """One chunk per row, slowly decaying states: the group states carry far."""
    T, D = 4 * L, 64
    c = Case(2, T, D, torch.float32, sid=320 + L, a_kind="long", n=16)
    both_forms(c, L, 320 + L, label="long L=%d long-memory" % L)


@pytest.mark.parametrize("L", [32, 64])
def test_long_block_backward_fused(dev, L, monkeypatch):
    """softplus(dt + bias) and the silu gate: the raw dt stream's gradient,
    d_dt_bias and dz."""
    monkeypatch.setenv("BDSSM_CHUNK", "64")
    batch, T, D, dtype = 2, 512, 70, torch.bfloat16
    sid = 340 + L
    c = Case(batch, T, D, dtype, sid=sid, a_kind="random", n=16)
    c.dev["dt"] = synth.normal((batch, T, D), 1000 * sid + 11, "cpu", torch.float32, mean=-1.0,
                               std=0.8).to(dtype).to("cuda").contiguous()
    bias = seeded((D,), 1000 * sid + 12, std=0.3)
    z = seeded((batch, T, D), 1000 * sid + 13, dtype, std=1.5)
    kw = dict(dt_bias=bias, dt_softplus=True, z=z)
    ok = dict(dt_bias=to_np(bias), dt_softplus=True, z=synth.to_oracle(z))
    both_forms(c, L, sid, kw, ok, label="long fused L=%d" % L)


def test_long_block_matches_general_kernel(dev, monkeypatch):
    """The pair kernel and the general kernel on the same long-block inputs:
    the same gradients up to fp32 rounding."""
    monkeypatch.setenv("BDSSM_CHUNK", "64")
    L, T, D = 64, 512, 96
    c = Case(2, T, D, torch.float32, sid=360, a_kind="random", n=16)
    dy = seeded((2, T, D), 36001)
    db = seeded((2, T // L + 1, D, 16), 36002)
    _, bnd = m.train_scan(*c.args(), L, want_bounds=True)
    outs = []
    for kern in ("pair", "general"):
        monkeypatch.setenv("BDSSM_BWD_KERNEL", kern)
        outs.append(m.train_scan_bwd(*c.args(), L, bnd, dy, d_bounds=db, want_dh_init=True))
    torch.cuda.synchronize()
    for k in outs[0]:
        a, b = outs[0][k].float(), outs[1][k].float()
        scale = max(b.abs().max().item(), 1e-30)
        assert (a - b).abs().max().item() / scale < 2e-5, k


def test_long_block_is_deterministic(dev, monkeypatch):
    monkeypatch.setenv("BDSSM_CHUNK", "64")
    L, T, D = 32, 512, 100
    c = Case(2, T, D, torch.bfloat16, sid=370, n=16)
    dy = seeded((2, T, D), 37001, torch.bfloat16)
    _, bnd = m.train_scan(*c.args(), L, want_bounds=True)
    g1 = m.train_scan_bwd(*c.args(), L, bnd, dy, want_dh_init=True)
    g2 = m.train_scan_bwd(*c.args(), L, bnd, dy, want_dh_init=True)
    torch.cuda.synchronize()
    for k in g1:
        assert torch.equal(g1[k], g2[k]), k
