"""GPU parity of the block lengths outside {1, 2, 4, 8, 16} (block_bidir_kernel:
one lane per channel, each block's forward output staged in LDS, blocks
longer than 64 tokens finished in 64-token segments) on every
forward entry point, against the fp64 oracle, element by element: lengths
that are not powers of two, multiples of 16, the largest supported (256),
ragged channel counts, forced multi-chunk plans (chunks rounded up to whole
blocks, so the forward carry runs), the two-stream form, the fusions and
separate reverse operands.  Also the regression case of a reverse step-size
bias given without a forward one, on both bidirectional kernels.
"""
import pytest
import torch

import mamba_selective_scan_04_amd as m
import oracle
from mamba_selective_scan_04_amd import synth
from parity_util import Case, N, STATE_TOL, TOL, rel_err, to_np, worst

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request, dev):
    print("\n[parity-blocklen] %s" % request.node.name, flush=True)
    yield


def close(got, ref, tol, what):
    g = to_np(got)
    assert g.shape == ref.shape, (what, g.shape, ref.shape)
    e = rel_err(g, ref)
    assert e < tol, (what, e, worst(g, ref))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("L,T,D", [(3, 96, 70), (5, 200, 64), (12, 240, 130), (24, 480, 96),
                                   (32, 512, 200), (48, 480, 64), (100, 400, 65), (256, 768, 96)])
def test_training_forms(dev, dtype, L, T, D, monkeypatch):
    """train_scan (with block states) and the two-stream form, several chunks."""
    monkeypatch.setenv("BDSSM_CHUNK", "64")
    batch = 2
    c = Case(batch, T, D, dtype, sid=61, a_kind="random")
    y, bnd = m.train_scan(*c.args(), L, want_bounds=True)
    h0b = synth.normal((batch, T // L + 1, D, N), 6101, "cuda")
    yb = m.train_scan_blocks(*c.args(), L, h0b)
    torch.cuda.synchronize()
    oa = c.oracle_args()
    yo, bo = oracle.train_scan(*oa, L, want_bounds=True)
    ybo = oracle.train_blocks(*oa, L, to_np(h0b))
    close(y, yo, TOL[dtype], "train_scan y")
    close(bnd, bo, STATE_TOL, "h_bounds")
    close(yb, ybo, TOL[dtype], "train_scan_blocks y")


@pytest.mark.parametrize("a_kind", ["default", "long"])
def test_training_single_chunk_with_h_init(dev, a_kind):
    """One chunk (no carry), a given start state, long-memory A."""
    batch, T, D, L = 2, 192, 128, 32
    c = Case(batch, T, D, torch.float32, sid=62, a_kind=a_kind)
    h0 = synth.normal((batch, D, N), 6201, "cuda")
    y, bnd = m.train_scan(*c.args(), L, h_init=h0, want_bounds=True)
    torch.cuda.synchronize()
    yo, bo = oracle.train_scan(*c.oracle_args(), L, h_init=to_np(h0), want_bounds=True)
    close(y, yo, TOL[torch.float32], "y")
    close(bnd, bo, STATE_TOL, "h_bounds")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("L", [6, 32, 64, 256])
def test_inference_cycle(dev, dtype, L, monkeypatch):
    """prefill (state only and with y) over a multi-chunk context, block step,
    commit with and without y; the block step equals the training form's
    last block (exact caching)."""
    monkeypatch.setenv("BDSSM_CHUNK", "64")
    batch, D = 2, 130
    P = 6 * L if L <= 64 else 2 * L
    T = P + 2 * L
    c = Case(batch, T, D, dtype, sid=63, a_kind="random")
    h, yp = m.prefill(*c.segment(0, P), L, want_y=True)
    h2, _ = m.prefill(*c.segment(0, P), L)
    ys = m.block_step(h, *c.segment(P, P + L))
    hc = h.clone()
    _, yc = m.commit(hc, *c.segment(P, P + L), want_y=True)
    hc2 = hc.clone()
    m.commit(hc2, *c.segment(P + L, T))
    yt, _ = m.train_scan(*c.segment(0, P + L), L)
    torch.cuda.synchronize()
    tol = TOL[dtype]
    ho, ypo = oracle.prefill(*c.oracle_args(0, P), L, want_y=True)
    close(h, ho, STATE_TOL, "prefill state")
    close(h2, ho, STATE_TOL, "prefill state (state only)")
    close(yp, ypo, tol, "prefill y")
    yso = oracle.block_step(ho, *c.oracle_args(P, P + L))
    close(ys, yso, tol, "block_step y")
    hco, yco = oracle.commit(ho, *c.oracle_args(P, P + L), want_y=True)
    close(yc, yco, tol, "commit y")
    close(hc, hco, STATE_TOL, "commit state")
    hco2, _ = oracle.commit(hco, *c.oracle_args(P + L, T))
    close(hc2, hco2, STATE_TOL, "commit state (no y)")
    close(ys, to_np(yt)[:, P:], tol, "block_step vs train_scan's last block")


@pytest.mark.parametrize("D", [1, 63, 64, 65])
def test_ragged_channels(dev, D):
    batch, T, L = 3, 96, 24
    c = Case(batch, T, D, torch.float32, sid=64, a_kind="random")
    y, bnd = m.train_scan(*c.args(), L, want_bounds=True)
    torch.cuda.synchronize()
    yo, bo = oracle.train_scan(*c.oracle_args(), L, want_bounds=True)
    close(y, yo, TOL[torch.float32], "y")
    close(bnd, bo, STATE_TOL, "h_bounds")


def test_block_equal_to_sequence_is_the_full_scan(dev):
    """L = T: the in-block reverse covers the whole sequence, as the baseline."""
    batch, T, D = 2, 192, 96
    c = Case(batch, T, D, torch.float32, sid=65, a_kind="random")
    y, _ = m.train_scan(*c.args(), T)
    yf = m.full_scan(*c.args())
    torch.cuda.synchronize()
    yo = oracle.full_scan(*c.oracle_args())
    close(y, yo, TOL[torch.float32], "train_scan L = T")
    close(yf, yo, TOL[torch.float32], "full_scan")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("mode", ["softplus_bias", "bias"])
def test_fusions(dev, dtype, mode, monkeypatch):
    """dt = softplus(dt_raw + bias) or dt_raw + bias, gate silu(z), L = 40."""
    monkeypatch.setenv("BDSSM_CHUNK", "64")
    batch, T, D, L = 2, 400, 100, 40
    c = Case(batch, T, D, dtype, sid=66, a_kind="random")
    mean = -1.0 if mode == "softplus_bias" else 1.0
    std = 0.5 if mode == "softplus_bias" else 0.1
    c.dev["dt"] = synth.normal((batch, T, D), 6601, "cpu", torch.float32, mean=mean,
                               std=std).to(dtype).to("cuda").contiguous()
    bias = synth.normal((D,), 6602, "cuda", torch.float32, std=0.3 if mode == "softplus_bias" else 0.05)
    z = synth.normal((batch, T, D), 6603, "cuda", dtype, std=2.0)
    kw = dict(dt_bias=bias, dt_softplus=mode == "softplus_bias", z=z)
    ok = dict(dt_bias=to_np(bias), dt_softplus=kw["dt_softplus"], z=synth.to_oracle(z))
    y, bnd = m.train_scan(*c.args(), L, want_bounds=True, **kw)
    h0b = synth.normal((batch, T // L + 1, D, N), 6604, "cuda")
    yb = m.train_scan_blocks(*c.args(), L, h0b, **kw)
    torch.cuda.synchronize()
    oa = c.oracle_args()
    yo, bo = oracle.train_scan(*oa, L, want_bounds=True, **ok)
    ybo = oracle.train_blocks(*oa, L, to_np(h0b), **ok)
    close(y, yo, TOL[dtype], "y")
    close(bnd, bo, STATE_TOL, "h_bounds")
    close(yb, ybo, TOL[dtype], "two-stream y")


def _rev_operands(batch, T, D, dtype, sid, with_bias):
    rev = dict(dt=synth.positive_step((batch, T, D), 1000 * sid + 80, "cpu", dtype),
               B=synth.normal((batch, T, N), 1000 * sid + 81, "cpu", dtype),
               C=synth.normal((batch, T, N), 1000 * sid + 82, "cpu", dtype),
               A=synth.a_matrix(D, N, "random", seed=1000 * sid + 83))
    rev = {k: v.to("cuda").contiguous() for k, v in rev.items()}
    if with_bias:
        rev["dt_bias"] = synth.normal((D,), 1000 * sid + 84, "cuda", torch.float32, std=0.05)
    return rev


def _rev_oracle(rev):
    out = dict(dt=synth.to_oracle(rev["dt"]), B=synth.to_oracle(rev["B"]),
               C=synth.to_oracle(rev["C"]), A=synth.to_oracle(rev["A"]))
    if "dt_bias" in rev:
        out["dt_bias"] = to_np(rev["dt_bias"])
    return out


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_reverse_operands(dev, dtype, monkeypatch):
    monkeypatch.setenv("BDSSM_CHUNK", "64")
    batch, T, D, L = 2, 384, 96, 48
    c = Case(batch, T, D, dtype, sid=67, a_kind="random")
    rev = _rev_operands(batch, T, D, dtype, 67, with_bias=False)
    y, bnd = m.train_scan(*c.args(), L, want_bounds=True, rev=rev)
    h0b = synth.normal((batch, T // L + 1, D, N), 6701, "cuda")
    yb = m.train_scan_blocks(*c.args(), L, h0b, rev=rev)
    torch.cuda.synchronize()
    oa = c.oracle_args()
    ro = _rev_oracle(rev)
    yo, bo = oracle.train_scan(*oa, L, want_bounds=True, rev=ro)
    ybo = oracle.train_blocks(*oa, L, to_np(h0b), rev=ro)
    close(y, yo, TOL[dtype], "y")
    close(bnd, bo, STATE_TOL, "h_bounds")
    close(yb, ybo, TOL[dtype], "two-stream y")


@pytest.mark.parametrize("L", [16, 4, 20])
def test_reverse_bias_without_forward_bias(dev, L, monkeypatch):
    """Separate reverse operands with a reverse step-size bias and no forward
    bias (no softplus): the reverse bias must still be added."""
    monkeypatch.setenv("BDSSM_CHUNK", "64")
    batch, T, D = 2, 320, 80
    dtype = torch.float32
    c = Case(batch, T, D, dtype, sid=68, a_kind="random")
    rev = _rev_operands(batch, T, D, dtype, 68, with_bias=True)
    y, _ = m.train_scan(*c.args(), L, rev=rev)
    h0b = synth.normal((batch, T // L + 1, D, N), 6801, "cuda")
    yb = m.train_scan_blocks(*c.args(), L, h0b, rev=rev)
    yf = m.full_scan(*c.args(), rev=rev)
    torch.cuda.synchronize()
    oa = c.oracle_args()
    ro = _rev_oracle(rev)
    close(y, oracle.train_scan(*oa, L, rev=ro)[0], TOL[dtype], "train_scan y")
    close(yb, oracle.train_blocks(*oa, L, to_np(h0b), rev=ro), TOL[dtype], "two-stream y")
    close(yf, oracle.full_scan(*oa, rev=ro), TOL[dtype], "full_scan y")


QUAD = [  # (L, N, dtype, variant)
    (128, 16, torch.bfloat16, "plain"),
    (128, 8, torch.float32, "plain"),
    (96, 32, torch.bfloat16, "plain"),
    (128, 4, torch.float32, "plain"),
    (128, 16, torch.bfloat16, "fused"),
    (128, 16, torch.float32, "rev"),
    (24, 16, torch.bfloat16, "plain"),
]


@pytest.mark.parametrize("seg", ["0", "64", "24"])
@pytest.mark.parametrize("L,N_,dtype,variant", QUAD)
def test_long_block_forward_segments(dev, seg, L, N_, dtype, variant, monkeypatch):
    """block_bidir_kernel's segments (the reverse state entering each segment
    formed again from the block's end) on both training forms: the default
    length (32 tokens, 64 at N = 32), 64-token segments (L = 96: a 32-token
    last segment) and 24-token ones (L = 128:
    five and a ragged 8-token last one; L = 24: one), several chunks, 70
    channels, 4 to 32 states, the fusions and separate reverse operands."""
    monkeypatch.setenv("BDSSM_CHUNK", "64")
    monkeypatch.setenv("BDSSM_SEG", seg)
    # multiples of 16 take bidir_pair_kernel by default: keep them on
    # block_bidir_kernel here
    monkeypatch.setenv("BDSSM_BIDIR_KERNEL", "wave")
    batch, T, D = 2, {128: 512, 96: 384, 24: 480}[L], 70
    sid = 400 + QUAD.index((L, N_, dtype, variant))
    c = Case(batch, T, D, dtype, sid=sid, a_kind="random", n=N_)
    kw, ok = {}, {}
    if variant == "fused":
        c.dev["dt"] = synth.normal((batch, T, D), 1000 * sid + 1, "cpu", torch.float32, mean=-1.0,
                                   std=0.5).to(dtype).to("cuda").contiguous()
        bias = synth.normal((D,), 1000 * sid + 2, "cuda", torch.float32, std=0.3)
        z = synth.normal((batch, T, D), 1000 * sid + 3, "cuda", dtype, std=2.0)
        kw = dict(dt_bias=bias, dt_softplus=True, z=z)
        ok = dict(dt_bias=to_np(bias), dt_softplus=True, z=synth.to_oracle(z))
    elif variant == "rev":
        rev = _rev_operands(batch, T, D, dtype, sid, with_bias=False)
        kw, ok = dict(rev=rev), dict(rev=_rev_oracle(rev))
    y, bnd = m.train_scan(*c.args(), L, want_bounds=True, **kw)
    h0b = synth.normal((batch, T // L + 1, D, N_), 1000 * sid + 4, "cuda")
    yb = m.train_scan_blocks(*c.args(), L, h0b, **kw)
    torch.cuda.synchronize()
    oa = c.oracle_args()
    yo, bo = oracle.train_scan(*oa, L, want_bounds=True, **ok)
    ybo = oracle.train_blocks(*oa, L, to_np(h0b), **ok)
    label = "seg %s L=%d N=%d %s" % (seg, L, N_, variant)
    close(y, yo, TOL[dtype], label + " y")
    close(bnd, bo, STATE_TOL, label + " h_bounds")
    close(yb, ybo, TOL[dtype], label + " two-stream y")


SPLIT = [  # (L, N, dtype, variant)
    (32, 16, torch.bfloat16, "plain"),
    (100, 8, torch.float32, "fused"),
    (256, 16, torch.bfloat16, "rev"),
    (48, 4, torch.float32, "plain"),
    (17, 16, torch.float32, "fused"),
    (64, 16, torch.bfloat16, "bias"),      # dt + bias without softplus
    (200, 16, torch.float32, "revbias"),   # reverse operands with their own bias, no forward bias
    (64, 8, torch.bfloat16, "revbias"),
]


@pytest.mark.parametrize("split", ["1", "0"])
@pytest.mark.parametrize("L,N_,dtype,variant", SPLIT)
def test_single_block_long(dev, split, L, N_, dtype, variant, monkeypatch):
    """The block step and the commit with outputs on one block longer than 16
    tokens: above 32 tokens block_split_kernel (the block's tokens over up to
    8 waves, segment states combined in LDS; the commit's cache read and
    written in place), else and when forced off block_bidir_kernel; 4 to 16
    states, 130 channels, the fusions and separate reverse operands, against
    the oracle from a seeded cache."""
    monkeypatch.setenv("BDSSM_SPLIT", split)
    batch, D = 2, 130
    sid = 420 + SPLIT.index((L, N_, dtype, variant))
    c = Case(batch, L, D, dtype, sid=sid, a_kind="random", n=N_)
    kw, ok = {}, {}
    if variant == "fused":
        c.dev["dt"] = synth.normal((batch, L, D), 1000 * sid + 1, "cpu", torch.float32, mean=-1.0,
                                   std=0.5).to(dtype).to("cuda").contiguous()
        bias = synth.normal((D,), 1000 * sid + 2, "cuda", torch.float32, std=0.3)
        z = synth.normal((batch, L, D), 1000 * sid + 3, "cuda", dtype, std=2.0)
        kw = dict(dt_bias=bias, dt_softplus=True, z=z)
        ok = dict(dt_bias=to_np(bias), dt_softplus=True, z=synth.to_oracle(z))
    elif variant == "bias":
        bias = synth.normal((D,), 1000 * sid + 2, "cuda", torch.float32, std=0.05)
        kw, ok = dict(dt_bias=bias), dict(dt_bias=to_np(bias))
    elif variant in ("rev", "revbias"):
        rev = _rev_operands(batch, L, D, dtype, sid, with_bias=variant == "revbias")
        if N_ != N:
            rev["B"], rev["C"] = rev["B"][..., :N_].contiguous(), rev["C"][..., :N_].contiguous()
            rev["A"] = rev["A"][:, :N_].contiguous()
        kw, ok = dict(rev=rev), dict(rev=_rev_oracle(rev))
    h = synth.normal((batch, D, N_), 1000 * sid + 5, "cuda", std=0.5)
    ys = m.block_step(h, *c.args()[:6], **kw)
    hc = h.clone()
    _, yc = m.commit(hc, *c.args()[:6], want_y=True, **kw)
    torch.cuda.synchronize()
    oa = c.oracle_args()
    ho = to_np(h)
    label = "split %s L=%d N=%d %s" % (split, L, N_, variant)
    close(ys, oracle.block_step(ho, *oa[:6], **ok), TOL[dtype], label + " block_step y")
    hco, yco = oracle.commit(ho, *oa[:6], want_y=True, **ok)
    close(yc, yco, TOL[dtype], label + " commit y")
    close(hc, hco, STATE_TOL, label + " commit state")


PAIR_LONG = [  # (L, N, T, D, dtype, variant): bidir_pair_kernel's long-block mode
    (32, 16, 512, 70, torch.bfloat16, "plain"),
    (48, 16, 480, 33, torch.float32, "plain"),
    (256, 16, 768, 96, torch.bfloat16, "plain"),
    (128, 32, 512, 40, torch.float32, "plain"),
    (64, 8, 512, 130, torch.bfloat16, "plain"),
    (96, 4, 384, 200, torch.float32, "plain"),
    (64, 16, 512, 70, torch.bfloat16, "fused"),
    (32, 32, 256, 24, torch.bfloat16, "fused"),
]


@pytest.mark.parametrize("L,N_,T,D,dtype,variant", PAIR_LONG)
def test_pair_long_blocks(dev, L, N_, T, D, dtype, variant, monkeypatch):
    """Blocks longer than one 16-token group in the two-state forward (each
    block's right-to-left state walk, then its groups left to right): both
    training forms with several chunks, the prefill with y, ragged channel
    tiles, 4 to 32 states and the fusions, against the oracle."""
    monkeypatch.setenv("BDSSM_CHUNK", "64")
    batch = 2
    sid = 420 + PAIR_LONG.index((L, N_, T, D, dtype, variant))
    c = Case(batch, T, D, dtype, sid=sid, a_kind="random", n=N_)
    kw, ok = {}, {}
    if variant == "fused":
        c.dev["dt"] = synth.normal((batch, T, D), 1000 * sid + 1, "cpu", torch.float32, mean=-1.0,
                                   std=0.5).to(dtype).to("cuda").contiguous()
        bias = synth.normal((D,), 1000 * sid + 2, "cuda", torch.float32, std=0.3)
        z = synth.normal((batch, T, D), 1000 * sid + 3, "cuda", dtype, std=2.0)
        kw = dict(dt_bias=bias, dt_softplus=True, z=z)
        ok = dict(dt_bias=to_np(bias), dt_softplus=True, z=synth.to_oracle(z))
    y, bnd = m.train_scan(*c.args(), L, want_bounds=True, **kw)
    h0b = synth.normal((batch, T // L + 1, D, N_), 1000 * sid + 4, "cuda")
    yb = m.train_scan_blocks(*c.args(), L, h0b, **kw)
    h, yp = m.prefill(*c.args(), L, want_y=True, **kw)
    torch.cuda.synchronize()
    oa = c.oracle_args()
    yo, bo = oracle.train_scan(*oa, L, want_bounds=True, **ok)
    ybo = oracle.train_blocks(*oa, L, to_np(h0b), **ok)
    label = "pair long L=%d N=%d %s" % (L, N_, variant)
    close(y, yo, TOL[dtype], label + " y")
    close(bnd, bo, STATE_TOL, label + " h_bounds")
    close(yb, ybo, TOL[dtype], label + " two-stream y")
    close(yp, yo, TOL[dtype], label + " prefill y")
    close(h, bo[:, -1], STATE_TOL, label + " prefill state")
