"""Pins for the fp64 CPU oracle, checked against things other than itself:
an O(T^2) materialised form, library routines on special cases (cumsum, flip),
closed forms, a hand-derived worked example, invariants of the method (exact
caching, block locality) and brute force on tiny inputs.

Each pin is chosen so that a plausible slip in the oracle (a dropped term, a
wrong sign, an off-by-one in the reverse, swapped B/C, a transposed A, a
missing initial state) fails at least one of them.
"""
import json
import os

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def softplus(z):
    return np.log1p(np.exp(z))


def rand_inputs(rng, batch, T, D, N, a_kind="random"):
    x = rng.standard_normal((batch, T, D)).astype(np.float32)
    dt = softplus(rng.normal(-1.0, 0.5, (batch, T, D))).astype(np.float32)
    B = rng.standard_normal((batch, T, N)).astype(np.float32)
    C = rng.standard_normal((batch, T, N)).astype(np.float32)
    if a_kind == "random":
        A = (-np.exp(rng.uniform(np.log(0.01), np.log(16.0), (D, N)))).astype(np.float32)
    elif a_kind == "long":
        A = np.broadcast_to(-1e-3 * np.arange(1, N + 1, dtype=np.float32), (D, N)).copy()
    elif a_kind == "zero":
        A = np.zeros((D, N), np.float32)
    else:
        A = np.broadcast_to(-np.arange(1, N + 1, dtype=np.float32), (D, N)).copy()
    Dskip = rng.standard_normal(D).astype(np.float32)
    return x, dt, B, C, A, Dskip


def brute_force(x, dt, B, C, A, Dskip, L, h0):
    """Materialised O(T^2) form with the decay written through cumulative sums
    of dt (no recurrence): the coefficient of token s's injection in the
    forward state at t >= s is exp(A * sum_{k=s+1..t} dt_k); in the reverse
    state at t <= s (same block) it is exp(A * sum_{k=t..s-1} dt_k)."""
    x, dt, B, C = (np.asarray(a, np.float64) for a in (x, dt, B, C))
    A = np.asarray(A, np.float64)
    batch, T, D = x.shape
    N = A.shape[1]
    y = np.zeros((batch, T, D))
    hT = np.zeros((batch, D, N))
    for b in range(batch):
        for d in range(D):
            S = np.concatenate([[0.0], np.cumsum(dt[b, :, d])])   # S[t+1] = sum_{k<=t}
            u = dt[b, :, d, None] * B[b] * x[b, :, d, None]       # [T, N]
            for t in range(T):
                hf = np.exp(A[d] * (S[t + 1] - S[0])) * h0[b, d]
                for s in range(t + 1):
                    hf = hf + np.exp(A[d] * (S[t + 1] - S[s + 1])) * u[s]
                k0 = (t // L) * L
                hr = np.zeros(N)
                for s in range(t, k0 + L):
                    hr = hr + np.exp(A[d] * (S[s] - S[t])) * u[s]
                y[b, t, d] = C[b, t] @ (hf + hr) + Dskip[d] * x[b, t, d]
                if t == T - 1:
                    hT[b, d] = hf
    return y, hT


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


@pytest.mark.parametrize("L", [1, 4, 8, 24])
def test_brute_force_tiny(L):
    rng = np.random.default_rng(10 + L)
    # D != N and B != C so that a transposed A or swapped B/C shows up
    x, dt, B, C, A, Dskip = rand_inputs(rng, 2, 24, 3, 5)
    h0 = rng.standard_normal((2, 3, 5))
    r = oracle.scan(x, dt, B, C, A, Dskip, L, h0=h0)
    yb, hb = brute_force(x, dt, B, C, A, Dskip, L, h0)
    assert rel(r["y"], yb) < 1e-12
    assert rel(r["hT"], hb) < 1e-12


def test_zero_A_is_cumsum():
    """A = 0: every decay is 1, so the forward state is h0 plus the running sum
    of injections and the reverse state is the in-block suffix sum."""
    rng = np.random.default_rng(1)
    batch, T, D, N, L = 2, 32, 4, 6, 8
    x, dt, B, C, _, Dskip = rand_inputs(rng, batch, T, D, N)
    A = np.zeros((D, N), np.float32)
    h0 = rng.standard_normal((batch, D, N))
    r = oracle.scan(x, dt, B, C, A, Dskip, L, h0=h0, want_parts=True)
    u = (dt.astype(np.float64)[..., None] * x.astype(np.float64)[..., None]
         * B.astype(np.float64)[:, :, None, :])                    # [b,T,D,N]
    hf = h0[:, None] + np.cumsum(u, axis=1)
    ub = u.reshape(batch, T // L, L, D, N)
    hr = np.flip(np.cumsum(np.flip(ub, axis=2), axis=2), axis=2).reshape(batch, T, D, N)
    Cd = C.astype(np.float64)[:, :, None, :]
    assert rel(r["yf"], (Cd * hf).sum(-1)) < 1e-12
    assert rel(r["yr"], (Cd * hr).sum(-1)) < 1e-12
    assert rel(r["y"], (Cd * (hf + hr)).sum(-1) + Dskip.astype(np.float64) * x.astype(np.float64)) < 1e-12
    assert rel(r["hT"], hf[:, -1]) < 1e-12


def test_zero_step_keeps_state():
    """dt = 0: no decay and no injection, so the state stays h0 and
    y = C . h0 + Dskip * x (the reverse state stays zero)."""
    rng = np.random.default_rng(2)
    x, dt, B, C, A, Dskip = rand_inputs(rng, 1, 16, 3, 4)
    dt[:] = 0
    h0 = rng.standard_normal((1, 3, 4))
    r = oracle.scan(x, dt, B, C, A, Dskip, 16, h0=h0)
    want = np.einsum("btn,bdn->btd", C.astype(np.float64), h0) + Dskip * x.astype(np.float64)
    assert rel(r["y"], want) < 1e-14
    assert np.array_equal(r["hT"], h0)


def test_instant_forgetting():
    """A = -1e6: every decay underflows to exactly 0, so both directions hold
    only the current token's injection: y = 2 C.u + Dskip x, hT = u_last."""
    rng = np.random.default_rng(3)
    x, dt, B, C, A, Dskip = rand_inputs(rng, 1, 16, 3, 4)
    A[:] = -1e6
    r = oracle.scan(x, dt, B, C, A, Dskip, 8, h0=rng.standard_normal((1, 3, 4)))
    u = dt.astype(np.float64)[..., None] * x.astype(np.float64)[..., None] * B.astype(np.float64)[:, :, None, :]
    want = 2 * (C.astype(np.float64)[:, :, None, :] * u).sum(-1) + Dskip * x.astype(np.float64)
    assert rel(r["y"], want) < 1e-14
    assert rel(r["hT"], u[:, -1]) < 1e-14


def test_constant_inputs_geometric_series():
    """Constant dt, x, B, C: with a = exp(dt A), u = dt B x,
    hf_t = a^(t+1) h0 + u (1 - a^(t+1)) / (1 - a) and, m tokens from t to the
    block end inclusive, hr_t = u (1 - a^m) / (1 - a)."""
    T, D, N, L = 32, 2, 3, 8
    x = np.full((1, T, D), 0.75, np.float32)
    dt = np.full((1, T, D), 0.25, np.float32)
    B = np.tile(np.array([1.0, -0.5, 2.0], np.float32), (1, T, 1))
    C = np.tile(np.array([0.5, 1.5, -1.0], np.float32), (1, T, 1))
    A = np.array([[-1.0, -0.5, -3.0], [-2.0, -0.1, -1.0]], np.float32)
    Dskip = np.array([0.3, -0.7], np.float32)
    h0 = np.array([[[1.0, 2.0, -1.0], [0.5, -0.5, 0.25]]])
    r = oracle.scan(x, dt, B, C, A, Dskip, L, h0=h0)
    a = np.exp(0.25 * A.astype(np.float64))                     # [D,N]
    u = 0.25 * B[0, 0].astype(np.float64)[None, :] * 0.75        # [1,N] -> same for all d
    want = np.zeros((T, D))
    for t in range(T):
        hf = a ** (t + 1) * h0[0] + u * (1 - a ** (t + 1)) / (1 - a)
        m = (t // L) * L + L - t
        hr = u * (1 - a ** m) / (1 - a)
        want[t] = (hf + hr) @ C[0, 0].astype(np.float64) + Dskip.astype(np.float64) * 0.75
    assert rel(r["y"][0], want) < 1e-13


def test_reverse_is_flipped_forward():
    """With one segment (L = T) and h0 = 0, the reverse part equals the forward
    part computed on time-flipped inputs, flipped back."""
    rng = np.random.default_rng(4)
    x, dt, B, C, A, Dskip = rand_inputs(rng, 2, 40, 3, 5)
    r = oracle.scan(x, dt, B, C, A, Dskip, 40, want_parts=True)
    fl = [np.ascontiguousarray(a[:, ::-1]) for a in (x, dt, B, C)]
    rf = oracle.scan(*fl, A, Dskip, 40, want_parts=True)
    assert np.array_equal(r["yr"], rf["yf"][:, ::-1])
    assert np.array_equal(r["yf"], rf["yr"][:, ::-1])


def test_unit_blocks_reverse_is_injection():
    """L = 1: the reverse state at t is exactly token t's injection."""
    rng = np.random.default_rng(5)
    x, dt, B, C, A, Dskip = rand_inputs(rng, 1, 12, 3, 4)
    r = oracle.scan(x, dt, B, C, A, Dskip, 1, want_parts=True)
    u = dt.astype(np.float64)[..., None] * B.astype(np.float64)[:, :, None, :] * x.astype(np.float64)[..., None]
    assert rel(r["yr"], (C.astype(np.float64)[:, :, None, :] * u).sum(-1)) < 1e-15


def test_linear_in_x():
    rng = np.random.default_rng(6)
    x1, dt, B, C, A, Dskip = rand_inputs(rng, 1, 32, 4, 6)
    x2 = rng.standard_normal(x1.shape).astype(np.float32)
    xs = (np.float32(0.5) * x1 + np.float32(-2.0) * x2)
    y1 = oracle.scan(x1, dt, B, C, A, Dskip, 8)["y"]
    y2 = oracle.scan(x2, dt, B, C, A, Dskip, 8)["y"]
    ys = oracle.scan(xs, dt, B, C, A, Dskip, 8)["y"]
    # xs is rounded to fp32; that rounding is far below the tolerance used
    assert rel(ys, 0.5 * y1 - 2.0 * y2) < 1e-6


def test_bf16_widening_is_exact():
    """bf16 inputs (raw bit patterns) give bit-identical results to the same
    values passed as fp32."""
    rng = np.random.default_rng(7)
    arrs = rand_inputs(rng, 1, 16, 3, 4)
    f32 = []
    b16 = []
    for a in arrs[:4]:
        bits = (a.view(np.uint32) >> 16).astype(np.uint16)        # truncate to bf16
        b16.append(bits)
        f32.append((bits.astype(np.uint32) << 16).view(np.float32))
    ra = oracle.scan(*f32, arrs[4], arrs[5], 8)
    rb = oracle.scan(*b16, arrs[4], arrs[5], 8)
    assert np.array_equal(ra["y"], rb["y"]) and np.array_equal(ra["hT"], rb["hT"])


def test_worked_example_by_hand():
    """Hand-derived fixture (tests/golden/worked_example.json): two tokens, one
    channel, two states, dt = ln 2 so that the decays are exact powers of 1/2."""
    with open(os.path.join(HERE, "golden", "worked_example.json")) as f:
        g = json.load(f)
    arr = lambda k, sh: np.array(g["inputs"][k], np.float32).reshape(sh)
    T, N = 2, 2
    x = arr("x", (1, T, 1))
    dt = np.full((1, T, 1), np.log(2.0), np.float32)
    B = arr("B", (1, T, N))
    C = arr("C", (1, T, N))
    A = arr("A", (1, N))
    Dskip = arr("Dskip", (1,))
    h0 = np.array(g["inputs"]["h0"], np.float64).reshape(1, 1, N)
    dtv = float(dt[0, 0, 0])                       # ln 2 rounded to fp32
    for case in g["cases"]:
        r = oracle.scan(x, dt, B, C, A, Dskip, case["L"], h0=h0)
        # the fixture states y in units of dt plus constants, see the json
        want_y = np.array(case["y_dt_coeff"]) * dtv + np.array(case["y_const"])
        # decays are exp(dtv * A); the fixture assumes exact 1/2, 1/4: allow
        # for ln2's fp32 rounding (relative 3e-8 in the exponent)
        assert rel(r["y"][0, :, 0], want_y) < 1e-6, case
        want_h = np.array(case["hT_dt_coeff"]) * dtv + np.array(case["hT_const"])
        assert rel(r["hT"][0, 0], want_h) < 1e-6, case


# ---------------------------------------------------------------- invariants

def test_exact_caching_prefill_commit_chain():
    """The cache depends on the clean prefix alone: prefill(P) followed by
    commits of b1, b2 equals prefill(P|b1|b2), and block_step on top of the
    cache equals the last block of the training form over the whole row.
    In the oracle these are bitwise equalities (identical operation order)."""
    for kind in ("default", "long", "zero"):
        rng = np.random.default_rng(8)
        L = 8
        x, dt, B, C, A, Dskip = rand_inputs(rng, 2, 5 * L, 3, 4, a_kind=kind)
        P = 3 * L
        seg = lambda a, s, e: np.ascontiguousarray(a[:, s:e])
        h, _ = oracle.prefill(seg(x, 0, P), seg(dt, 0, P), seg(B, 0, P), seg(C, 0, P), A, Dskip, L)
        h1, _ = oracle.commit(h, seg(x, P, P + L), seg(dt, P, P + L), seg(B, P, P + L),
                              seg(C, P, P + L), A, Dskip)
        h2, _ = oracle.commit(h1, seg(x, P + L, P + 2 * L), seg(dt, P + L, P + 2 * L),
                              seg(B, P + L, P + 2 * L), seg(C, P + L, P + 2 * L), A, Dskip)
        hall, _ = oracle.prefill(x, dt, B, C, A, Dskip, L)
        assert np.array_equal(h2, hall)
        # chained prefill through h_init
        ha, _ = oracle.prefill(seg(x, 0, L), seg(dt, 0, L), seg(B, 0, L), seg(C, 0, L), A, Dskip, L)
        hb, _ = oracle.prefill(seg(x, L, 5 * L), seg(dt, L, 5 * L), seg(B, L, 5 * L),
                               seg(C, L, 5 * L), A, Dskip, L, h_init=ha)
        assert np.array_equal(hb, hall)
        # block step on the cache == last block of the training form
        yb = oracle.block_step(h1, seg(x, P + L, P + 2 * L), seg(dt, P + L, P + 2 * L),
                               seg(B, P + L, P + 2 * L), seg(C, P + L, P + 2 * L), A, Dskip)
        yt, bounds = oracle.train_scan(seg(x, 0, P + 2 * L), seg(dt, 0, P + 2 * L),
                                       seg(B, 0, P + 2 * L), seg(C, 0, P + 2 * L), A, Dskip, L,
                                       want_bounds=True)
        assert np.array_equal(yb, yt[:, P + L:])
        # commit with y == block step on the same inputs
        _, yc = oracle.commit(h1, seg(x, P + L, P + 2 * L), seg(dt, P + L, P + 2 * L),
                              seg(B, P + L, P + 2 * L), seg(C, P + L, P + 2 * L), A, Dskip,
                              want_y=True)
        assert np.array_equal(yc, yb)
        # prefill with y == training form on the same tokens
        _, yp = oracle.prefill(seg(x, 0, P), seg(dt, 0, P), seg(B, 0, P), seg(C, 0, P), A, Dskip,
                               L, want_y=True)
        assert np.array_equal(yp, yt[:, :P])
        # boundary states are the caches of every prefix
        assert np.array_equal(bounds[:, 3], h)
        assert np.array_equal(bounds[:, 4], h1)
        assert np.array_equal(bounds[:, 0], np.zeros_like(h))


def test_block_locality():
    """The reverse scan is confined to the active block: perturbing any token
    after block k leaves block k's outputs bitwise unchanged; perturbing token
    s inside block k changes y at earlier tokens of that block but at no token
    of an earlier block."""
    rng = np.random.default_rng(9)
    L = 8
    x, dt, B, C, A, Dskip = rand_inputs(rng, 1, 4 * L, 3, 4, a_kind="long")
    y0, _ = oracle.train_scan(x, dt, B, C, A, Dskip, L)
    x2 = x.copy()
    x2[:, 2 * L:] += 1.0                 # every token after block 1
    y2, _ = oracle.train_scan(x2, dt, B, C, A, Dskip, L)
    assert np.array_equal(y0[:, :2 * L], y2[:, :2 * L])
    assert not np.array_equal(y0[:, 2 * L:], y2[:, 2 * L:])
    s = L + 5                            # inside block 1
    x3 = x.copy()
    x3[:, s] += 1.0
    y3, _ = oracle.train_scan(x3, dt, B, C, A, Dskip, L)
    assert np.array_equal(y0[:, :L], y3[:, :L])
    assert np.all(y0[:, L:s] != y3[:, L:s])          # reverse mixes within the block


def test_full_sequence_reverse_is_not_prefix_only():
    """Negative control: with the reverse over the whole sequence, perturbing
    the last token changes the first token's output."""
    rng = np.random.default_rng(11)
    x, dt, B, C, A, Dskip = rand_inputs(rng, 1, 32, 3, 4, a_kind="long")
    y0 = oracle.full_scan(x, dt, B, C, A, Dskip)
    x2 = x.copy()
    x2[:, -1] += 1.0
    y2 = oracle.full_scan(x2, dt, B, C, A, Dskip)
    assert np.all(y0[:, 0] != y2[:, 0])
    yt, _ = oracle.train_scan(x, dt, B, C, A, Dskip, 32)
    assert np.array_equal(y0, yt)


def test_rejects_bad_arguments():
    rng = np.random.default_rng(12)
    x, dt, B, C, A, Dskip = rand_inputs(rng, 1, 12, 3, 4)
    with pytest.raises(ValueError):
        oracle.scan(x, dt, B, C, A, Dskip, 8)      # 12 % 8 != 0


def test_empty_sequence():
    x = np.zeros((1, 0, 3), np.float32)
    B = np.zeros((1, 0, 4), np.float32)
    A = -np.ones((3, 4), np.float32)
    h0 = np.arange(12, dtype=np.float64).reshape(1, 3, 4)
    r = oracle.scan(x, x, B, B, A, np.zeros(3, np.float32), 8, h0=h0)
    assert r["y"].shape == (1, 0, 3)
    assert np.array_equal(r["hT"], h0)


# ---------------------------------------------------- two-stream training form

def test_train_blocks_with_own_bounds_is_continuous_scan():
    """Starting every block from the stream's own boundary states reproduces
    the continuous forward scan, bit for bit."""
    for kind in ("random", "long"):
        rng = np.random.default_rng(30)
        x, dt, B, C, A, Dskip = rand_inputs(rng, 2, 48, 3, 5, a_kind=kind)
        h0 = rng.standard_normal((2, 3, 5))
        for L in (1, 4, 8, 16):
            r = oracle.scan(x, dt, B, C, A, Dskip, L, h0=h0, want_bounds=True)
            yb = oracle.train_blocks(x, dt, B, C, A, Dskip, L, r["bounds"])
            assert np.array_equal(yb, r["y"])


def test_train_blocks_independent_blocks_brute_force():
    """With arbitrary block start states every block is its own problem: the
    materialised form of each block from its own start state."""
    rng = np.random.default_rng(31)
    L = 8
    x, dt, B, C, A, Dskip = rand_inputs(rng, 2, 24, 3, 5)
    h0b = rng.standard_normal((2, 24 // L + 1, 3, 5))
    yb = oracle.train_blocks(x, dt, B, C, A, Dskip, L, h0b)
    for k in range(24 // L):
        seg = lambda a: a[:, k * L:(k + 1) * L]
        want, _ = brute_force(seg(x), seg(dt), seg(B), seg(C), A, Dskip, L, h0b[:, k])
        assert rel(yb[:, k * L:(k + 1) * L], want) < 1e-12


def test_train_blocks_zero_starts_is_block_step_from_zero():
    rng = np.random.default_rng(32)
    L = 8
    x, dt, B, C, A, Dskip = rand_inputs(rng, 1, 32, 3, 4)
    yb = oracle.train_blocks(x, dt, B, C, A, Dskip, L, np.zeros((1, 32 // L + 1, 3, 4)))
    for k in range(32 // L):
        seg = lambda a: np.ascontiguousarray(a[:, k * L:(k + 1) * L])
        ys = oracle.block_step(np.zeros((1, 3, 4)), seg(x), seg(dt), seg(B), seg(C), A, Dskip)
        assert np.array_equal(yb[:, k * L:(k + 1) * L], ys)
