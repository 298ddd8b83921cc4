"""GPU parity: every entry point of the HIP library against the fp64 oracle,
element by element, on seeded inputs.  Sizes span several 64-channel tiles,
several time chunks and ragged tails (channels not a multiple of 64, the last
16-token group partly filled).  Full-size workloads are checked on sampled
channels in test_parity_fullsize.py.
"""
import os

import numpy as np
import pytest
import torch

import mamba_selective_scan_04_amd as m
import oracle
from parity_util import Case, N, STATE_TOL, TOL, rel_err, to_np, worst

pytestmark = pytest.mark.gpu


def _sync():
    torch.cuda.synchronize()


@pytest.fixture(autouse=True)
def _announce(request, dev):
    print("\n[parity] %s" % request.node.name, flush=True)
    yield


# ------------------------------------------------------------- tiny fp32 workload

def test_tiny_fp32_workload(dev):
    """batch 1, d_inner 64, d_state 16, 256 tokens, block 16, fp32: prefill of
    240 tokens, one block step, commit, and the training / baseline forms."""
    c = Case(1, 256, 64, torch.float32, sid=1)
    L, P = 16, 240
    seg = c.segment(0, P)
    h, _ = m.prefill(*seg, L)
    blk = c.segment(P, P + L)
    y = m.block_step(h, *blk)
    h_before = h.clone()
    _, yc = m.commit(h, *blk, want_y=True)
    yt, bnd = m.train_scan(*c.args(), L, want_bounds=True)
    yfull = m.full_scan(*c.args())
    _sync()
    oa = c.oracle_args(0, P)
    ho, _ = oracle.prefill(*oa, L)
    ob = c.oracle_args(P, P + L)
    yo = oracle.block_step(ho, *ob)
    ho2, yco = oracle.commit(ho, *ob, want_y=True)
    full = c.oracle_args()
    yto, bo = oracle.train_scan(*full, L, want_bounds=True)
    yfo = oracle.full_scan(*full)
    assert rel_err(to_np(h_before), ho) < STATE_TOL
    assert rel_err(to_np(y), yo) < TOL[torch.float32]
    assert rel_err(to_np(yc), yco) < TOL[torch.float32]
    assert rel_err(to_np(h), ho2) < STATE_TOL
    assert rel_err(to_np(yt), yto) < TOL[torch.float32]
    assert rel_err(to_np(bnd), bo) < STATE_TOL
    assert rel_err(to_np(yfull), yfo) < TOL[torch.float32]
    # the block step equals the last block of the training form (exact caching)
    assert rel_err(to_np(y), yto[:, P:]) < TOL[torch.float32]


# ----------------------------------------------------- medium bf16, ragged, chunked

# the bidirectional pass on bidir_pair_kernel (two states per lane, the
# default) and on bidir_wave_kernel (four states per lane)
BIDIR = ["pair", "wave"]


@pytest.mark.parametrize("bidir", BIDIR)
@pytest.mark.parametrize("a_kind", ["default", "random", "long"])
def test_bf16_medium_all_forms(dev, a_kind, bidir, monkeypatch):
    """batch 2, 200 channels (three full 64-lane tiles and a ragged one; six
    full 32-channel tiles and a ragged one), 2048 tokens; chunk length forced
    to 128 so every chunked path runs."""
    monkeypatch.setenv("BDSSM_CHUNK", "128")
    monkeypatch.setenv("BDSSM_BIDIR_KERNEL", bidir)
    c = Case(2, 2048, 200, torch.bfloat16, sid=8, a_kind=a_kind)
    L = 16
    tol = TOL[torch.bfloat16]
    h, yp = m.prefill(*c.args(), L, want_y=True)
    h2, _ = m.prefill(*c.args(), L)
    yt, bnd = m.train_scan(*c.args(), L, want_bounds=True)
    yf = m.full_scan(*c.args())
    _sync()
    oa = c.oracle_args()
    r = oracle.scan(*oa, L, want_y=True, want_bounds=True)
    yfo = oracle.full_scan(*oa)
    assert rel_err(to_np(h), r["hT"]) < STATE_TOL
    assert rel_err(to_np(h2), r["hT"]) < STATE_TOL
    assert rel_err(to_np(yp), r["y"]) < tol
    assert rel_err(to_np(yt), r["y"]) < tol
    assert rel_err(to_np(bnd), r["bounds"]) < STATE_TOL, worst(to_np(bnd), r["bounds"])
    assert rel_err(to_np(yf), yfo) < tol
    # bf16 outputs within one bf16 rounding of the oracle's value
    ref = torch.from_numpy(r["y"]).float().to(torch.bfloat16).float().numpy()
    diff = np.abs(to_np(yt) - ref)
    ulp = np.abs(ref) * 2.0 ** -7 + 1e-30
    assert np.mean(diff <= ulp) > 0.999


def test_fp32_zero_A_and_initial_state(dev, monkeypatch):
    """A = 0 (no decay, long cumulative sums) with a nonzero initial state."""
    monkeypatch.setenv("BDSSM_CHUNK", "64")
    c = Case(2, 512, 96, torch.float32, sid=9, a_kind="zero")
    h0 = torch.randn(2, 96, N, generator=torch.Generator().manual_seed(3)).to(dev)
    L = 16
    h, yp = m.prefill(*c.args(), L, h_init=h0, want_y=True)
    yt, _ = m.train_scan(*c.args(), L, h_init=h0)
    _sync()
    r = oracle.scan(*c.oracle_args(), L, h0=to_np(h0), want_y=True)
    assert rel_err(to_np(h), r["hT"]) < STATE_TOL
    assert rel_err(to_np(yp), r["y"]) < TOL[torch.float32]
    assert rel_err(to_np(yt), r["y"]) < TOL[torch.float32]


@pytest.mark.parametrize("bidir", BIDIR)
@pytest.mark.parametrize("L,T", [(1, 37), (2, 50), (4, 36), (8, 40), (8, 8), (16, 48)])
def test_block_lengths_and_ragged_groups(dev, L, T, bidir, monkeypatch):
    """Every supported block length, with sequence lengths that leave the last
    16-token group partly filled."""
    monkeypatch.setenv("BDSSM_BIDIR_KERNEL", bidir)
    c = Case(1, T, 70, torch.float32, sid=10, a_kind="random")
    yt, bnd = m.train_scan(*c.args(), L, want_bounds=True)
    blk = c.segment(T - L, T)
    hpre, _ = m.prefill(*c.segment(0, T - L), L)
    yb = m.block_step(hpre, *blk)
    _sync()
    r = oracle.scan(*c.oracle_args(), L, want_y=True, want_bounds=True)
    assert rel_err(to_np(yt), r["y"]) < TOL[torch.float32]
    assert rel_err(to_np(bnd), r["bounds"]) < STATE_TOL
    assert rel_err(to_np(yb), r["y"][:, T - L:]) < TOL[torch.float32]


def test_chunk_length_invariance(dev, monkeypatch):
    c = Case(1, 1024, 128, torch.float32, sid=11, a_kind="long")
    outs = []
    for ch in ("16", "48", "256", "100000"):
        monkeypatch.setenv("BDSSM_CHUNK", ch)
        yt, _ = m.train_scan(*c.args(), 16)
        h, _ = m.prefill(*c.args(), 16)
        outs.append((to_np(yt), to_np(h)))
    _sync()
    r = oracle.scan(*c.oracle_args(), 16, want_y=True)
    for yt, h in outs:
        assert rel_err(yt, r["y"]) < TOL[torch.float32]
        assert rel_err(h, r["hT"]) < STATE_TOL
        assert rel_err(yt, outs[0][0]) < 1e-4


# ------------------------------------------------------------------ invariants

def test_exact_caching_on_gpu(dev):
    """The cache after prefill(P) and commits of b1..b3 matches prefill over
    P|b1|b2|b3; block steps never modify the cache; a cache saved to the host
    and restored gives bit-identical block outputs."""
    L = 16
    for a_kind in ("default", "long"):
        c = Case(2, 64 * L, 130, torch.bfloat16, sid=12, a_kind=a_kind)
        P = 60 * L
        h, _ = m.prefill(*c.segment(0, P), L)
        for k in range(3):
            blk = c.segment(P + k * L, P + (k + 1) * L)
            before = h.clone()
            y1 = m.block_step(h, *blk)
            y2 = m.block_step(h, *blk)
            _sync()
            assert torch.equal(before, h)
            assert torch.equal(y1, y2)
            saved = h.cpu()
            restored = saved.to(dev)
            y3 = m.block_step(restored, *blk)
            _sync()
            assert torch.equal(y1, y3)
            m.commit(h, *blk)
        hall, _ = m.prefill(*c.segment(0, P + 3 * L), L)
        _sync()
        ho, _ = oracle.prefill(*c.oracle_args(0, P + 3 * L), L)
        assert rel_err(to_np(h), ho) < STATE_TOL
        assert rel_err(to_np(hall), ho) < STATE_TOL


def test_block_locality_on_gpu(dev, monkeypatch):
    """Perturbing tokens after block k leaves block k's training-form outputs
    bitwise unchanged (the reverse is confined to the block); the full-sequence
    baseline is not prefix-only."""
    monkeypatch.setenv("BDSSM_CHUNK", "64")
    L = 16
    c = Case(1, 512, 100, torch.float32, sid=13, a_kind="long")
    y0, _ = m.train_scan(*c.args(), L)
    f0 = m.full_scan(*c.args())
    k = 20
    x2 = c.dev["x"].clone()
    x2[:, (k + 1) * L:] += 1.0
    args2 = (x2,) + c.args()[1:]
    y2, _ = m.train_scan(*args2, L)
    f2 = m.full_scan(*args2)
    _sync()
    assert torch.equal(y0[:, :(k + 1) * L], y2[:, :(k + 1) * L])
    assert not torch.equal(y0[:, (k + 1) * L:], y2[:, (k + 1) * L:])
    assert not torch.equal(f0[:, :L], f2[:, :L])


def test_determinism(dev, monkeypatch):
    monkeypatch.setenv("BDSSM_CHUNK", "128")
    c = Case(2, 1024, 192, torch.bfloat16, sid=14, a_kind="random")
    a = [m.train_scan(*c.args(), 16)[0], m.prefill(*c.args(), 16)[0], m.full_scan(*c.args())]
    b = [m.train_scan(*c.args(), 16)[0], m.prefill(*c.args(), 16)[0], m.full_scan(*c.args())]
    _sync()
    for u, v in zip(a, b):
        assert torch.equal(u, v)


# ------------------------------------------------------------------ edge cases

@pytest.mark.parametrize("D", [1, 63, 65])
def test_small_and_ragged_channel_counts(dev, D):
    c = Case(3, 64, D, torch.float32, sid=15, a_kind="random")
    yt, _ = m.train_scan(*c.args(), 16)
    h, _ = m.prefill(*c.args(), 16)
    yf = m.full_scan(*c.args())
    _sync()
    r = oracle.scan(*c.oracle_args(), 16, want_y=True)
    assert rel_err(to_np(yt), r["y"]) < TOL[torch.float32]
    assert rel_err(to_np(h), r["hT"]) < STATE_TOL
    assert rel_err(to_np(yf), oracle.full_scan(*c.oracle_args())) < TOL[torch.float32]


def test_empty_inputs(dev):
    x = torch.zeros(2, 0, 64, device=dev)
    Bm = torch.zeros(2, 0, N, device=dev)
    A = -torch.ones(64, N, device=dev)
    Ds = torch.zeros(64, device=dev)
    h0 = torch.randn(2, 64, N, device=dev)
    h, _ = m.prefill(x, x, Bm, Bm, A, Ds, 16, h_init=h0)
    _, bnd = m.train_scan(x, x, Bm, Bm, A, Ds, 16, h_init=h0, want_bounds=True)
    y = m.full_scan(x, x, Bm, Bm, A, Ds)
    _sync()
    assert torch.equal(h, h0)
    assert torch.equal(bnd[:, 0], h0)
    assert y.shape == (2, 0, 64)


def test_in_place_prefill_continuation(dev):
    """prefill may take its initial state from the buffer it writes."""
    c = Case(1, 512, 64, torch.bfloat16, sid=16)
    h, _ = m.prefill(*c.segment(0, 256), 16)
    m.prefill(*c.segment(256, 512), 16, h_init=h, h_cache=h)
    _sync()
    ho, _ = oracle.prefill(*c.oracle_args(), 16)
    assert rel_err(to_np(h), ho) < STATE_TOL


def test_graph_replay_matches_eager(dev):
    """The inference calls can be captured in a HIP graph (no memset or
    allocation inside): replays, with eager work and synchronisations in
    between, reproduce the eager results bit for bit every time."""
    c = Case(2, 16 * 40, 130, torch.bfloat16, sid=17, a_kind="random")
    L, P = 16, 16 * 36
    h, _ = m.prefill(*c.segment(0, P), L)
    blocks = [c.segment(P + k * L, P + (k + 1) * L) for k in range(4)]
    # eager reference: 3 block steps on block 0, commit block 0, 1 step on block 1
    h_ref = h.clone()
    ys_ref = [m.block_step(h_ref, *blocks[0]) for _ in range(3)]
    m.commit(h_ref, *blocks[0])
    y_next_ref = m.block_step(h_ref, *blocks[1])
    torch.cuda.synchronize()
    hg = torch.empty_like(h)
    ys = [torch.empty_like(ys_ref[0]) for _ in range(3)]
    y_next = torch.empty_like(y_next_ref)
    g = torch.cuda.CUDAGraph()
    hg.copy_(h)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for i in range(3):
            m.block_step(hg, *blocks[0], y=ys[i])
        m.commit(hg, *blocks[0])
        m.block_step(hg, *blocks[1], y=y_next)
    for rep in range(4):
        hg.copy_(h)                               # eager work between replays
        _ = m.block_step(h, *blocks[2])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i in range(3):
            assert torch.equal(ys[i], ys_ref[i]), rep
        assert torch.equal(hg, h_ref), rep
        assert torch.equal(y_next, y_next_ref), rep


# ---------------------------------------------------- two-stream training form

@pytest.mark.parametrize("bidir", BIDIR)
@pytest.mark.parametrize("L,T,D,dtype", [(16, 512, 130, torch.bfloat16), (8, 200, 70, torch.float32),
                                         (4, 36, 64, torch.float32), (1, 37, 65, torch.float32),
                                         (2, 50, 33, torch.bfloat16)])
def test_train_blocks_against_oracle(dev, L, T, D, dtype, bidir, monkeypatch):
    """Every block from its own (seeded, synthetic) start state."""
    from mamba_selective_scan_04_amd import synth
    monkeypatch.setenv("BDSSM_BIDIR_KERNEL", bidir)
    c = Case(2, T, D, dtype, sid=18, a_kind="random")
    h0b = synth.normal((2, T // L + 1, D, N), 1000 * 18 + 7).to(dev)
    y = m.train_scan_blocks(*c.args(), L, h0b)
    _sync()
    yo = oracle.train_blocks(*c.oracle_args(), L, to_np(h0b))
    assert rel_err(to_np(y), yo) < TOL[dtype], worst(to_np(y), yo)


@pytest.mark.parametrize("n", [16, 32])
@pytest.mark.parametrize("L", [8, 16])
@pytest.mark.parametrize("T", [16, 17, 33, 48, 64, 80, 101])
def test_pair_group_pairs_and_ragged_tails(dev, T, L, n):
    """bidir_pair_kernel runs two 16-token groups per barrier at 16 and 32
    states: sequences of 1 to 7 groups (an odd last group, a partial last
    group, an even count), both training forms, against the oracle."""
    from mamba_selective_scan_04_amd import synth
    if T % L:
        T = (T // L + 1) * L
    sid = 60 + T + L + n
    c = Case(2, T, 40, torch.float32, sid=sid, a_kind="random", n=n)
    h0 = synth.normal((2, 40, n), 1000 * sid + 5).to(dev)
    y, bnd = m.train_scan(*c.args(), L, h_init=h0, want_bounds=True)
    h0b = synth.normal((2, T // L + 1, 40, n), 1000 * sid + 7).to(dev)
    yb = m.train_scan_blocks(*c.args(), L, h0b)
    _sync()
    yo, bo = oracle.train_scan(*c.oracle_args(), L, h_init=to_np(h0), want_bounds=True)
    assert rel_err(to_np(y), yo) < TOL[torch.float32], worst(to_np(y), yo)
    assert rel_err(to_np(bnd), bo) < STATE_TOL
    ybo = oracle.train_blocks(*c.oracle_args(), L, to_np(h0b))
    assert rel_err(to_np(yb), ybo) < TOL[torch.float32], worst(to_np(yb), ybo)


def test_train_blocks_with_clean_bounds_matches_continuous(dev):
    """Passing the stream's own boundary states (from train_scan) reproduces
    train_scan's output: the noisy-stream form equals the clean form when the
    noisy tokens are the clean ones."""
    c = Case(4, 2048, 192, torch.bfloat16, sid=19, a_kind="long")
    y, bnd = m.train_scan(*c.args(), 16, want_bounds=True)
    yb = m.train_scan_blocks(*c.args(), 16, bnd)
    _sync()
    assert rel_err(to_np(yb), to_np(y)) < TOL[torch.bfloat16]


@pytest.mark.parametrize("kernel", ["lane", "wave"])
@pytest.mark.parametrize("n,L,D,dtype", [(16, 16, 130, torch.bfloat16), (16, 5, 70, torch.float32),
                                         (4, 16, 65, torch.bfloat16), (32, 12, 33, torch.float32),
                                         (8, 1, 200, torch.bfloat16)])
def test_single_block_kernels(dev, kernel, n, L, D, dtype, monkeypatch):
    """block_step and commit (with and without y) on either single-block kernel
    (one lane per (channel, state), or the bidirectional / chunk kernels),
    with and without the step-size and gate fusions, against the oracle."""
    from mamba_selective_scan_04_amd import synth
    monkeypatch.setenv("BDSSM_BLOCK_KERNEL", kernel)
    batch, P = 2, 4 * L
    c = Case(batch, P + L, D, dtype, sid=12, a_kind="random", n=n)
    h, _ = m.prefill(*c.segment(0, P), L)
    blk = c.segment(P, P + L)
    ho, _ = oracle.prefill(*c.oracle_args(0, P), L)
    ob = c.oracle_args(P, P + L)
    for fused in (False, True):
        kw, ok = {}, {}
        if fused:
            bias = synth.normal((D,), 1201, "cuda", torch.float32, std=0.3)
            z = synth.normal((batch, L, D), 1202, "cuda", dtype, std=1.5)
            kw = dict(dt_bias=bias, dt_softplus=True, z=z)
            ok = dict(dt_bias=to_np(bias), dt_softplus=True, z=synth.to_oracle(z))
        y = m.block_step(h, *blk, **kw)
        hc = h.clone()
        _, yc = m.commit(hc, *blk, want_y=True, **kw)
        hc2 = h.clone()
        m.commit(hc2, *blk, **{k: v for k, v in kw.items() if k != "z"})
        _sync()
        tol = TOL[dtype]
        assert rel_err(to_np(y), oracle.block_step(ho, *ob, **ok)) < tol, (fused, "block_step")
        hco, yco = oracle.commit(ho, *ob, want_y=True, **ok)
        assert rel_err(to_np(yc), yco) < tol, (fused, "commit y")
        assert rel_err(to_np(hc), hco) < STATE_TOL, (fused, "commit state")
        ok2 = {k: v for k, v in ok.items() if k != "z"}
        hco2, _ = oracle.commit(ho, *ob, **ok2)
        assert rel_err(to_np(hc2), hco2) < STATE_TOL, (fused, "commit state, no y")


def test_bound_calls_match_plain_calls(dev):
    """BoundCall (checked and marshalled once, launched many times) enqueues
    the same work as the plain binding call: block_step and commit, plain and
    fused, bit for bit, also after the inputs' contents change."""
    from mamba_selective_scan_04_amd import synth
    batch, L, D, P = 4, 16, 200, 64
    c = Case(batch, P + L, D, torch.bfloat16, sid=24, a_kind="random")
    h, _ = m.prefill(*c.segment(0, P), L)
    blk = c.segment(P, P + L)
    bias = synth.normal((D,), 2401, "cuda", torch.float32, std=0.3)
    z = synth.normal((batch, L, D), 2402, "cuda", torch.bfloat16)
    for kw in ({}, dict(dt_bias=bias, dt_softplus=True, z=z)):
        y_ref = m.block_step(h, *blk, **kw)
        y = torch.empty_like(y_ref)
        call = m.bind_block_step(h, *blk, y, **kw)
        call()
        _sync()
        assert torch.equal(y, y_ref)
        blk[0].mul_(-0.5)                       # new contents, same storage
        y_ref = m.block_step(h, *blk, **kw)
        call()
        _sync()
        assert torch.equal(y, y_ref)
        ckw = {k: v for k, v in kw.items() if k != "z"}
        h_ref = h.clone()
        m.commit(h_ref, *blk, **ckw)
        hb = h.clone()
        m.bind_commit(hb, *blk, **ckw)()
        _sync()
        assert torch.equal(hb, h_ref)
