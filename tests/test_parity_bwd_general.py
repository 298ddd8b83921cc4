"""GPU parity of the backward's general path (state counts 4, 8 and 32, block
lengths outside {1, 2, 4, 8, 16} up to 256) against the fp64 oracle's
gradients, element by element: both training forms, the gradient entering
through the block states (d_bounds), forced multi-chunk plans (the general
adjoint pre-pass and the carry run), ragged channel counts, blocks longer
than one 16-token segment and blocks that end inside one, and the fusions.

The oracle receives the same input values as the GPU (read back from the
device tensors); dy, d_bounds and the two-stream block starts are seeded.
Block lengths that are multiples of 16 at 16 states normally take the pair
kernel with group states (tests/test_parity_bwd_long.py); here
BDSSM_BWD_KERNEL=general keeps them on the general kernel.
"""
import pytest
import torch

import mamba_selective_scan_04_amd as m
import oracle
from mamba_selective_scan_04_amd import synth
from parity_util import Case, STATE_TOL, TOL, rel_err, to_np, worst

pytestmark = pytest.mark.gpu

GRADS = ("dx", "ddt", "dB", "dC")
PARAM_GRADS = ("dA", "dDskip")


@pytest.fixture(autouse=True)
def _announce(request, dev):
    print("\n[parity-bwd-general] %s" % request.node.name, flush=True)
    yield


def seeded(shape, seed, dtype=torch.float32, std=1.0):
    return synth.normal(shape, seed, "cpu", dtype, std=std).to("cuda").contiguous()


def check(got, ref, names, tol, label=""):
    for k in names:
        g = to_np(got[k])
        assert g.shape == ref[k].shape, (label, k, g.shape, ref[k].shape)
        e = rel_err(g, ref[k])
        assert e < tol, (label, k, e, worst(g, ref[k]))


def both_forms(c, L, sid, kw=None, ok=None, label=""):
    kw = kw or {}
    ok = ok or {}
    batch, T, D, n, dtype = c.batch, c.T, c.D, c.n, c.dtype
    dy = seeded((batch, T, D), 1000 * sid + 21, dtype)
    db = seeded((batch, T // L + 1, D, n), 1000 * sid + 22)
    h0b = seeded((batch, T // L + 1, D, n), 1000 * sid + 23)
    _, bnd = m.train_scan(*c.args(), L, want_bounds=True, **kw)
    g = m.train_scan_bwd(*c.args(), L, bnd, dy, d_bounds=db, want_dh_init=True, **kw)
    gb = m.train_scan_blocks_bwd(*c.args(), L, h0b, dy, want_dh0_blocks=True, **kw)
    torch.cuda.synchronize()
    oa = c.oracle_args()
    r = oracle.scan_bwd(*oa, L, to_np(dy), dbounds=to_np(db), **ok)
    r["dh_init"] = r.pop("dh0")
    rb = oracle.scan_bwd(*oa, L, to_np(dy), h0_blocks=to_np(h0b), **ok)
    extra = tuple(k for k in ("dz",) if k in r)
    pextra = tuple(k for k in ("d_dt_bias",) if k in r)
    check(g, r, GRADS + extra, TOL[dtype], label)
    check(g, r, PARAM_GRADS + ("dh_init",) + pextra, STATE_TOL, label)
    check(gb, rb, GRADS + extra, TOL[dtype], label + " blocks")
    check(gb, rb, PARAM_GRADS + ("dh0_blocks",) + pextra, STATE_TOL, label + " blocks")


CASES = [  # (N, L, T, D, dtype)
    (4, 16, 256, 130, torch.bfloat16),
    (8, 16, 320, 70, torch.float32),
    (32, 16, 192, 40, torch.bfloat16),
    (16, 3, 240, 70, torch.bfloat16),
    (16, 12, 480, 100, torch.float32),
    (16, 24, 480, 70, torch.bfloat16),
    (16, 32, 512, 65, torch.bfloat16),
    (16, 48, 480, 33, torch.float32),
    (16, 100, 400, 70, torch.bfloat16),
    (16, 256, 512, 40, torch.float32),
    (8, 40, 480, 50, torch.bfloat16),
    (32, 64, 256, 24, torch.float32),
    (4, 5, 200, 130, torch.bfloat16),
]


@pytest.mark.parametrize("N,L,T,D,dtype", CASES)
def test_general_backward(dev, N, L, T, D, dtype, monkeypatch):
    """Several chunks (the adjoint pre-pass and the carry), both forms."""
    monkeypatch.setenv("BDSSM_CHUNK", "64")
    monkeypatch.setenv("BDSSM_BWD_KERNEL", "general")
    sid = 60 + CASES.index((N, L, T, D, dtype))
    c = Case(2, T, D, dtype, sid=sid, a_kind="random", n=N)
    both_forms(c, L, sid, label="N=%d L=%d" % (N, L))


@pytest.mark.parametrize("N,L", [(16, 32), (8, 16), (4, 100)])
def test_general_backward_single_chunk_long_memory(dev, N, L, monkeypatch):
    """One chunk per row (no carry), slowly decaying states."""
    monkeypatch.setenv("BDSSM_BWD_KERNEL", "general")
    T, D = 4 * L if L > 16 else 128, 64
    c = Case(2, T, D, torch.float32, sid=80 + N + L, a_kind="long", n=N)
    both_forms(c, L, 80 + N + L, label="N=%d L=%d long" % (N, L))


@pytest.mark.parametrize("N,L", [(8, 16), (16, 24), (32, 48)])
def test_general_backward_fused(dev, N, L, monkeypatch):
    """softplus(dt + bias) and the silu gate: the raw dt stream's gradient,
    d_dt_bias and dz."""
    monkeypatch.setenv("BDSSM_CHUNK", "64")
    batch, T, D, dtype = 2, {16: 256, 24: 480, 48: 480}[L], 70, torch.bfloat16
    sid = 90 + N + L
    c = Case(batch, T, D, dtype, sid=sid, a_kind="random", n=N)
    c.dev["dt"] = synth.normal((batch, T, D), 1000 * sid + 11, "cpu", torch.float32, mean=-1.0,
                               std=0.8).to(dtype).to("cuda").contiguous()
    bias = seeded((D,), 1000 * sid + 12, std=0.3)
    z = seeded((batch, T, D), 1000 * sid + 13, dtype, std=1.5)
    kw = dict(dt_bias=bias, dt_softplus=True, z=z)
    ok = dict(dt_bias=to_np(bias), dt_softplus=True, z=synth.to_oracle(z))
    both_forms(c, L, sid, kw, ok, label="fused N=%d L=%d" % (N, L))


def test_general_backward_is_deterministic(dev, monkeypatch):
    monkeypatch.setenv("BDSSM_CHUNK", "64")
    batch, T, D, L, N = 2, 480, 100, 24, 8
    c = Case(batch, T, D, torch.bfloat16, sid=98, n=N)
    dy = seeded((batch, T, D), 9801, torch.bfloat16)
    _, bnd = m.train_scan(*c.args(), L, want_bounds=True)
    g1 = m.train_scan_bwd(*c.args(), L, bnd, dy, want_dh_init=True)
    g2 = m.train_scan_bwd(*c.args(), L, bnd, dy, want_dh_init=True)
    torch.cuda.synchronize()
    for k in g1:
        assert torch.equal(g1[k], g2[k]), k


def test_general_backward_empty_sequence(dev):
    N, L = 8, 24
    c = Case(2, 0, 64, torch.float32, sid=99, n=N)
    bnd = seeded((2, 1, 64, N), 9901)
    db = seeded((2, 1, 64, N), 9902)
    dy = torch.empty(2, 0, 64, device="cuda")
    g = m.train_scan_bwd(*c.args(), L, bnd, dy, d_bounds=db, want_dh_init=True)
    torch.cuda.synchronize()
    assert torch.count_nonzero(g["dA"]) == 0 and g["dA"].shape == (64, N)
    assert torch.equal(g["dh_init"], db[:, 0])


PAIR_CASES = [  # (N, L, T, D, dtype): the pair kernel at other state counts
    (4, 16, 256, 130, torch.bfloat16),
    (8, 16, 336, 70, torch.float32),
    (32, 16, 192, 40, torch.bfloat16),
    (32, 4, 200, 33, torch.float32),
    (8, 2, 100, 65, torch.bfloat16),
    (4, 1, 37, 130, torch.float32),
]


@pytest.mark.parametrize("N,L,T,D,dtype", PAIR_CASES)
def test_pair_backward_state_counts(dev, N, L, T, D, dtype, monkeypatch):
    """bwd_pair_kernel at 4, 8 and 32 states (the default for block lengths
    dividing 16): several chunks, ragged channel tiles and last groups, both
    forms."""
    monkeypatch.setenv("BDSSM_CHUNK", "64")
    monkeypatch.setenv("BDSSM_COARSE_CHUNKS", "3")
    sid = 80 + PAIR_CASES.index((N, L, T, D, dtype))
    c = Case(2, T, D, dtype, sid=sid, a_kind="random", n=N)
    both_forms(c, L, sid, label="pair N=%d L=%d" % (N, L))


@pytest.mark.parametrize("N", [4, 8, 32])
def test_pair_backward_state_counts_fused(dev, N, monkeypatch):
    """The fused pair kernel (softplus with bias, gate) at 4, 8 and 32 states."""
    monkeypatch.setenv("BDSSM_CHUNK", "64")
    batch, T, D, L = 2, 200, 70, 8
    c = Case(batch, T, D, torch.bfloat16, sid=90 + N, a_kind="random", n=N)
    c.dev["dt"] = synth.normal((batch, T, D), 1000 * (90 + N) + 11, "cpu", torch.float32, mean=-1.0,
                               std=0.8).to(torch.bfloat16).to("cuda").contiguous()
    bias = seeded((D,), 1000 * (90 + N) + 12, std=0.3)
    z = seeded((batch, T, D), 1000 * (90 + N) + 13, torch.bfloat16, std=1.5)
    kw = dict(dt_softplus=True, dt_bias=bias, z=z)
    ok = dict(dt_softplus=True, dt_bias=to_np(bias), z=synth.to_oracle(z))
    both_forms(c, L, 90 + N, kw, ok, label="pair fused N=%d" % N)
