"""GPU parity of the backward entry points (train_scan_bwd,
train_scan_blocks_bwd) against the fp64 oracle's gradients, element by
element, on seeded inputs: several 64-channel tiles, ragged channel counts,
ragged 16-token groups, every supported block length, forced multi-chunk
plans (so the adjoint carry across chunks runs), the gradient flowing in
through the block states (d_bounds), the two-stream form and the all-block
chain that joins them.

The oracle receives the same input values as the GPU (read back from the
device tensors); it recomputes its own forward states.  dy, d_bounds and the
two-stream block starts are seeded inputs, not GPU outputs.
"""
import numpy as np
import pytest
import torch

import mamba_selective_scan_04_amd as m
import oracle
from mamba_selective_scan_04_amd import synth
from parity_util import Case, N, STATE_TOL, TOL, rel_err, to_np, worst

pytestmark = pytest.mark.gpu

GRADS = ("dx", "ddt", "dB", "dC")          # stream dtype
PARAM_GRADS = ("dA", "dDskip")             # fp32


@pytest.fixture(autouse=True)
def _announce(request, dev):
    print("\n[parity-bwd] %s" % request.node.name, flush=True)
    yield


def seeded(shape, seed, dtype=torch.float32, std=1.0):
    return synth.normal(shape, seed, "cpu", dtype, std=std).to("cuda").contiguous()


def check(got, ref, names, tol, label=""):
    for k in names:
        g = to_np(got[k])
        assert g.shape == ref[k].shape, (k, g.shape, ref[k].shape)
        e = rel_err(g, ref[k])
        assert e < tol, (label, k, e, worst(g, ref[k]))


def run_continuous(c, L, dy, dbounds=None, want_dh=True):
    y, bnd = m.train_scan(*c.args(), L, want_bounds=True)
    g = m.train_scan_bwd(*c.args(), L, bnd, dy, d_bounds=dbounds, want_dh_init=want_dh)
    torch.cuda.synchronize()
    return g


def oracle_continuous(c, L, dy, dbounds=None):
    r = oracle.scan_bwd(*c.oracle_args(), L, to_np(dy),
                        dbounds=None if dbounds is None else to_np(dbounds))
    r["dh_init"] = r.pop("dh0")
    return r


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("with_bounds", [False, True])
def test_train_scan_bwd_single_chunk(dev, dtype, with_bounds):
    batch, T, D, L = 2, 256, 64, 16
    c = Case(batch, T, D, dtype, sid=31)
    dy = seeded((batch, T, D), 3101, dtype)
    db = seeded((batch, T // L + 1, D, N), 3102) if with_bounds else None
    g = run_continuous(c, L, dy, db)
    r = oracle_continuous(c, L, dy, db)
    check(g, r, GRADS, TOL[dtype], "single")
    check(g, r, PARAM_GRADS + ("dh_init",), STATE_TOL, "single")


@pytest.mark.parametrize("a_kind", ["default", "random", "long"])
def test_train_scan_bwd_multi_chunk_bf16(dev, a_kind, monkeypatch):
    """Forced small chunks: the adjoint aggregates and the reverse carry run,
    and the backward pass walks several coarse chunks."""
    monkeypatch.setenv("BDSSM_CHUNK", "64")
    monkeypatch.setenv("BDSSM_COARSE_CHUNKS", "5")
    batch, T, D, L = 2, 1024, 130, 16
    c = Case(batch, T, D, torch.bfloat16, sid=32, a_kind=a_kind)
    dy = seeded((batch, T, D), 3201, torch.bfloat16)
    db = seeded((batch, T // L + 1, D, N), 3202)
    g = run_continuous(c, L, dy, db)
    r = oracle_continuous(c, L, dy, db)
    check(g, r, GRADS, TOL[torch.bfloat16], a_kind)
    check(g, r, PARAM_GRADS + ("dh_init",), STATE_TOL, a_kind)


def test_train_scan_bwd_multi_chunk_fp32(dev, monkeypatch):
    monkeypatch.setenv("BDSSM_CHUNK", "48")
    monkeypatch.setenv("BDSSM_COARSE_CHUNKS", "3")
    batch, T, D, L = 1, 400, 70, 8
    c = Case(batch, T, D, torch.float32, sid=33, a_kind="random")
    dy = seeded((batch, T, D), 3301)
    db = seeded((batch, T // L + 1, D, N), 3302)
    g = run_continuous(c, L, dy, db)
    r = oracle_continuous(c, L, dy, db)
    check(g, r, GRADS + PARAM_GRADS + ("dh_init",), TOL[torch.float32], "fp32 multi")


@pytest.mark.parametrize("L,T", [(1, 40), (2, 50), (4, 36), (8, 40), (16, 48)])
def test_train_scan_bwd_block_lengths_and_ragged_groups(dev, L, T):
    batch, D = 2, 64
    c = Case(batch, T, D, torch.float32, sid=34, a_kind="random")
    dy = seeded((batch, T, D), 3400 + L)
    db = seeded((batch, T // L + 1, D, N), 3450 + L)
    g = run_continuous(c, L, dy, db)
    r = oracle_continuous(c, L, dy, db)
    check(g, r, GRADS + PARAM_GRADS + ("dh_init",), TOL[torch.float32], "L=%d" % L)


@pytest.mark.parametrize("D", [1, 17, 65, 200])
def test_train_scan_bwd_ragged_channels(dev, D):
    batch, T, L = 2, 64, 16
    c = Case(batch, T, D, torch.float32, sid=35)
    dy = seeded((batch, T, D), 3500 + D)
    g = run_continuous(c, L, dy)
    r = oracle_continuous(c, L, dy)
    check(g, r, GRADS + PARAM_GRADS + ("dh_init",), TOL[torch.float32], "D=%d" % D)


@pytest.mark.parametrize("dtype,L,T,D", [(torch.float32, 16, 256, 64), (torch.bfloat16, 16, 512, 130),
                                         (torch.float32, 4, 72, 70), (torch.float32, 8, 40, 64)])
def test_train_scan_blocks_bwd(dev, dtype, L, T, D):
    batch = 2
    c = Case(batch, T, D, dtype, sid=36, a_kind="random")
    h0b = seeded((batch, T // L + 1, D, N), 3601)
    dy = seeded((batch, T, D), 3602, dtype)
    g = m.train_scan_blocks_bwd(*c.args(), L, h0b, dy, want_dh0_blocks=True)
    torch.cuda.synchronize()
    r = oracle.scan_bwd(*c.oracle_args(), L, to_np(dy), h0_blocks=to_np(h0b))
    check(g, r, GRADS, TOL[dtype], "blocks")
    check(g, r, PARAM_GRADS + ("dh0_blocks",), STATE_TOL, "blocks")


def test_all_block_chain(dev, monkeypatch):
    """Clean stream -> block states -> noisy stream; the noisy stream's
    block-start gradients flow back into the clean stream as d_bounds."""
    monkeypatch.setenv("BDSSM_CHUNK", "64")
    batch, T, D, L = 2, 512, 96, 16
    dtype = torch.bfloat16
    clean = Case(batch, T, D, dtype, sid=37, a_kind="random")
    noisy = Case(batch, T, D, dtype, sid=37, a_kind="random", k0=50)
    A, Ds = clean.dev["A"], clean.dev["Dskip"]
    nargs = (noisy.dev["x"], noisy.dev["dt"], noisy.dev["B"], noisy.dev["C"], A, Ds)
    dyc = seeded((batch, T, D), 3701, dtype)
    dyn = seeded((batch, T, D), 3702, dtype)
    _, bnd = m.train_scan(*clean.args(), L, want_bounds=True)
    gn = m.train_scan_blocks_bwd(*nargs, L, bnd, dyn, want_dh0_blocks=True)
    gc = m.train_scan_bwd(*clean.args(), L, bnd, dyc, d_bounds=gn["dh0_blocks"], want_dh_init=True)
    torch.cuda.synchronize()

    oc = clean.oracle_args()
    on = noisy.oracle_args()[:4] + oc[4:]
    bo = oracle.scan(*oc, L, want_y=False, want_bounds=True)["bounds"]
    rn = oracle.scan_bwd(*on, L, to_np(dyn), h0_blocks=bo)
    rc = oracle.scan_bwd(*oc, L, to_np(dyc), dbounds=rn["dh0_blocks"])
    rc["dh_init"] = rc.pop("dh0")
    check(gn, rn, GRADS, TOL[dtype], "noisy")
    check(gc, rc, GRADS, TOL[dtype], "clean")
    check(gn, rn, PARAM_GRADS + ("dh0_blocks",), STATE_TOL, "noisy")
    check(gc, rc, PARAM_GRADS + ("dh_init",), STATE_TOL, "clean")


def test_bwd_is_deterministic(dev, monkeypatch):
    monkeypatch.setenv("BDSSM_CHUNK", "64")
    monkeypatch.setenv("BDSSM_COARSE_CHUNKS", "4")
    batch, T, D, L = 2, 512, 130, 16
    c = Case(batch, T, D, torch.bfloat16, sid=38)
    dy = seeded((batch, T, D), 3801, torch.bfloat16)
    _, bnd = m.train_scan(*c.args(), L, want_bounds=True)
    g1 = m.train_scan_bwd(*c.args(), L, bnd, dy, want_dh_init=True)
    g2 = m.train_scan_bwd(*c.args(), L, bnd, dy, want_dh_init=True)
    torch.cuda.synchronize()
    for k in g1:
        assert torch.equal(g1[k], g2[k]), k


def test_bwd_empty_sequence(dev):
    c = Case(2, 0, 64, torch.float32, sid=39)
    bnd = seeded((2, 1, 64, N), 3901)
    dy = torch.empty(2, 0, 64, device="cuda")
    db = seeded((2, 1, 64, N), 3902)
    g = m.train_scan_bwd(*c.args(), 16, bnd, dy, d_bounds=db, want_dh_init=True)
    torch.cuda.synchronize()
    assert torch.count_nonzero(g["dA"]) == 0 and torch.count_nonzero(g["dDskip"]) == 0
    assert torch.equal(g["dh_init"], db[:, 0])


@pytest.mark.parametrize("kernel", ["pair", "wave"])
@pytest.mark.parametrize("L", [2, 4, 8, 16])
def test_both_backward_kernels(dev, kernel, L, monkeypatch):
    """Each block-local backward kernel (two states per lane with the whole
    group in registers, or four states per lane with segment recomputation),
    forced whatever the block length would pick, in both training forms with
    several coarse chunks, ragged channels and a ragged last group."""
    monkeypatch.setenv("BDSSM_BWD_KERNEL", kernel)
    monkeypatch.setenv("BDSSM_CHUNK", "64")
    monkeypatch.setenv("BDSSM_COARSE_CHUNKS", "3")
    batch, D = 2, 100
    T = 456 if L < 16 else 464          # a ragged last 16-token group where L allows
    c = Case(batch, T, D, torch.bfloat16, sid=39, a_kind="random")
    dy = seeded((batch, T, D), 3950 + L, torch.bfloat16)
    db = seeded((batch, T // L + 1, D, N), 3960 + L)
    g = run_continuous(c, L, dy, db)
    r = oracle_continuous(c, L, dy, db)
    check(g, r, GRADS, TOL[torch.bfloat16], kernel)
    check(g, r, PARAM_GRADS + ("dh_init",), STATE_TOL, kernel)
    h0b = seeded((batch, T // L + 1, D, N), 3970 + L)
    gb = m.train_scan_blocks_bwd(*c.args(), L, h0b, dy, want_dh0_blocks=True)
    torch.cuda.synchronize()
    rb = oracle.scan_bwd(*c.oracle_args(), L, to_np(dy), h0_blocks=to_np(h0b))
    check(gb, rb, GRADS, TOL[torch.bfloat16], kernel + " blocks")
    check(gb, rb, PARAM_GRADS + ("dh0_blocks",), STATE_TOL, kernel + " blocks")


@pytest.mark.parametrize("L", [16, 32, 64])
def test_training_step_graph_replays_match_eager(dev, L, monkeypatch):
    """The whole all-block training step (both forms, forward and backward,
    caller workspaces) captured in one HIP graph: every replay, with eager
    work in between, reproduces the eager gradients bit for bit (the library
    records no memset nodes and allocates nothing).  L = 32 and 64 run the
    long-block kernels (segmented forward, group states, pair backward)."""
    monkeypatch.setenv("BDSSM_CHUNK", "64")
    batch, T, D = 2, 512, 96
    c = Case(batch, T, D, torch.bfloat16, sid=40, a_kind="random")
    dy = seeded((batch, T, D), 4001, torch.bfloat16)
    y = torch.empty_like(c.dev["x"])
    bnd = torch.empty(batch, T // L + 1, D, N, device="cuda")
    ws = torch.empty(max(1, m.workspace_bytes(batch, D, T, m.OP_TRAIN, L, N, torch.bfloat16)),
                     dtype=torch.uint8, device="cuda")
    wsb = torch.empty(m.workspace_bytes(batch, D, T, m.OP_TRAIN_BWD, L, N, torch.bfloat16),
                      dtype=torch.uint8, device="cuda")
    wsbb = torch.empty(m.workspace_bytes(batch, D, T, m.OP_BLOCKS_BWD, L, N, torch.bfloat16),
                       dtype=torch.uint8, device="cuda")

    def step():
        m.train_scan(*c.args(), L, y=y, h_bounds=bnd, ws=ws)
        gn = m.train_scan_blocks_bwd(*c.args(), L, bnd, dy, want_dh0_blocks=True, ws=wsbb)
        gc = m.train_scan_bwd(*c.args(), L, bnd, dy, d_bounds=gn["dh0_blocks"], want_dh_init=True, ws=wsb)
        return gn, gc

    ref_n, ref_c = step()
    torch.cuda.synchronize()
    ref = {("n", k): v.clone() for k, v in ref_n.items() if v is not None}
    ref.update({("c", k): v.clone() for k, v in ref_c.items() if v is not None})
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out_n, out_c = step()
    for _ in range(3):
        g.replay()
        torch.cuda.synchronize()
        for (form, k), v in ref.items():
            got = (out_n if form == "n" else out_c)[k]
            assert torch.equal(got, v), (form, k)
        step()                                     # eager work between the replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("fill", ["1", "0"])
def test_training_plans_default_chunks(dev, fill, monkeypatch):
    """Default plans (nothing forced) at a shape where the training plans
    cut the fine chunks shorter than the inference plan's (batch 4, 1536
    channels, 2048 tokens: 128 chunks of 16 tokens instead of 64 of 32, four
    coarse chunks): train_scan with its block states and train_scan_bwd with
    d_bounds against the oracle, with the shorter chunks and without them
    (BDSSM_FILL_PREPASS=0)."""
    monkeypatch.setenv("BDSSM_FILL_PREPASS", fill)
    batch, T, D, L = 4, 2048, 1536, 16
    c = Case(batch, T, D, torch.bfloat16, sid=3900, a_kind="random", device=dev, gen_device=dev)
    dy = synth.normal((batch, T, D), 3901, dev, torch.bfloat16)
    db = synth.normal((batch, T // L + 1, D, N), 3902, dev, torch.float32)
    y, bnd = m.train_scan(*c.args(), L, want_bounds=True)
    g = m.train_scan_bwd(*c.args(), L, bnd, dy, d_bounds=db, want_dh_init=True)
    torch.cuda.synchronize()
    ch = list(range(0, D, 97)) + [D - 1]
    oa = c.oracle_args(chans=ch)
    idx = torch.as_tensor(ch, device=dev)
    sel = lambda t: to_np(t.index_select(2, idx))
    r = oracle.scan(*oa, L, want_y=True, want_bounds=True)
    assert rel_err(sel(y), r["y"]) < TOL[torch.bfloat16], worst(sel(y), r["y"])
    assert rel_err(sel(bnd), r["bounds"]) < STATE_TOL, worst(sel(bnd), r["bounds"])
    rb = oracle.scan_bwd(*oa, L, sel(dy), dbounds=sel(db))
    for k in ("dx", "ddt"):
        assert rel_err(sel(g[k]), rb[k]) < TOL[torch.bfloat16], (k, worst(sel(g[k]), rb[k]))
    ga = to_np(g["dA"].index_select(0, idx))
    assert rel_err(ga, rb["dA"]) < STATE_TOL, worst(ga, rb["dA"])
    gh = to_np(g["dh_init"].index_select(1, idx))
    assert rel_err(gh, rb["dh0"]) < STATE_TOL, worst(gh, rb["dh0"])
