"""Pins for the oracle's reverse-mode gradients (oracle_scan_bwd), checked
against the forward oracle (itself pinned in test_oracle.py), never against
the backward's own formulas:

* central differences of J = <dy, y> (+ <dbounds, h_bounds>) in fp64, for every
  input element, in the continuous form (gradient of train_scan) and in the
  two-stream form (gradient of train_blocks);
* exact Jacobians where y is affine in an input (x and B with a zero start
  state, C and the start state always, dt when A = 0): the gradient element
  is J(unit input) - J(zero input), with no truncation error;
* the all-block chain: the noisy stream's block-start gradients fed back as
  the clean stream's dbounds reproduce the central differences of the
  composed two-stream objective.
"""
import numpy as np
import pytest

import oracle

FD_STEP = 1e-6
FD_TOL = 2e-6        # relative to max(|g|, rms(g)); fp64 central differences
EXACT_TOL = 1e-10


def rand64(rng, batch, T, D, N, a_kind="random"):
    x = rng.standard_normal((batch, T, D))
    dt = np.log1p(np.exp(rng.normal(-1.0, 0.5, (batch, T, D))))
    B = rng.standard_normal((batch, T, N))
    C = rng.standard_normal((batch, T, N))
    if a_kind == "random":
        A = -np.exp(rng.uniform(np.log(0.05), np.log(4.0), (D, N)))
    else:
        A = np.zeros((D, N))
    Dskip = rng.standard_normal(D)
    return dict(x=x, dt=dt, B=B, C=C, A=A, Dskip=Dskip)


def rel(g, r):
    g, r = np.asarray(g, np.float64), np.asarray(r, np.float64)
    if r.size == 0:
        return 0.0
    floor = np.sqrt(np.mean(r * r)) + 1e-300
    return float(np.max(np.abs(g - r) / np.maximum(np.abs(r), floor)))


def objective_continuous(p, L, dy, dbounds):
    r = oracle.scan(p["x"], p["dt"], p["B"], p["C"], p["A"], p["Dskip"], L, h0=p["h0"],
                    want_y=True, want_bounds=dbounds is not None)
    J = float(np.sum(dy * r["y"]))
    if dbounds is not None:
        J += float(np.sum(dbounds * r["bounds"]))
    return J


def objective_blocks(p, L, dy):
    y = oracle.train_blocks(p["x"], p["dt"], p["B"], p["C"], p["A"], p["Dskip"], L, p["h0_blocks"])
    return float(np.sum(dy * y))


def central_differences(p, names, J):
    out = {}
    for name in names:
        g = np.zeros_like(p[name])
        flat = p[name].reshape(-1)
        for i in range(flat.size):
            v = flat[i]
            flat[i] = v + FD_STEP
            jp = J(p)
            flat[i] = v - FD_STEP
            jm = J(p)
            flat[i] = v
            g.reshape(-1)[i] = (jp - jm) / (2 * FD_STEP)
        out[name] = g
    return out


@pytest.mark.parametrize("L,with_bounds", [(1, False), (4, True), (4, False), (12, True)])
def test_continuous_gradient_matches_central_differences(L, with_bounds):
    rng = np.random.default_rng(100 + L)
    batch, T, D, N = 2, 12, 3, 4
    p = rand64(rng, batch, T, D, N)
    p["h0"] = rng.standard_normal((batch, D, N))
    dy = rng.standard_normal((batch, T, D))
    db = rng.standard_normal((batch, T // L + 1, D, N)) if with_bounds else None
    g = oracle.scan_bwd(p["x"], p["dt"], p["B"], p["C"], p["A"], p["Dskip"], L, dy, h0=p["h0"],
                        dbounds=db)
    fd = central_differences(p, ["x", "dt", "B", "C", "A", "Dskip", "h0"],
                             lambda q: objective_continuous(q, L, dy, db))
    for gname, pname in (("dx", "x"), ("ddt", "dt"), ("dB", "B"), ("dC", "C"), ("dA", "A"),
                         ("dDskip", "Dskip"), ("dh0", "h0")):
        assert rel(g[gname], fd[pname]) < FD_TOL, (gname, rel(g[gname], fd[pname]))


@pytest.mark.parametrize("L", [2, 4])
def test_two_stream_gradient_matches_central_differences(L):
    rng = np.random.default_rng(200 + L)
    batch, T, D, N = 2, 8, 3, 4
    p = rand64(rng, batch, T, D, N)
    p["h0_blocks"] = rng.standard_normal((batch, T // L + 1, D, N))
    dy = rng.standard_normal((batch, T, D))
    g = oracle.scan_bwd(p["x"], p["dt"], p["B"], p["C"], p["A"], p["Dskip"], L, dy,
                        h0_blocks=p["h0_blocks"])
    fd = central_differences(p, ["x", "dt", "B", "C", "A", "Dskip", "h0_blocks"],
                             lambda q: objective_blocks(q, L, dy))
    for gname, pname in (("dx", "x"), ("ddt", "dt"), ("dB", "B"), ("dC", "C"), ("dA", "A"),
                         ("dDskip", "Dskip"), ("dh0_blocks", "h0_blocks")):
        assert rel(g[gname], fd[pname]) < FD_TOL, (gname, rel(g[gname], fd[pname]))
    # the last block-start entry is never read by the forward
    assert np.all(g["dh0_blocks"][:, -1] == 0.0)


def unit_jacobian(p, name, J):
    """J(input = e_i) - J(input = 0) for every element i: exact for an input in
    which J is affine."""
    saved = p[name].copy()
    p[name][...] = 0.0
    j0 = J(p)
    g = np.zeros_like(saved)
    flat = p[name].reshape(-1)
    for i in range(flat.size):
        flat[i] = 1.0
        g.reshape(-1)[i] = J(p) - j0
        flat[i] = 0.0
    p[name][...] = saved
    return g


def test_exact_jacobians_of_affine_inputs():
    rng = np.random.default_rng(300)
    batch, T, D, N, L = 2, 8, 3, 4, 4
    dy = rng.standard_normal((batch, T, D))
    # zero start: y is linear in x and affine in B, C
    p = rand64(rng, batch, T, D, N)
    p["h0"] = np.zeros((batch, D, N))
    J = lambda q: objective_continuous(q, L, dy, None)
    g = oracle.scan_bwd(p["x"], p["dt"], p["B"], p["C"], p["A"], p["Dskip"], L, dy, h0=p["h0"])
    for gname, pname in (("dx", "x"), ("dB", "B"), ("dC", "C"), ("dh0", "h0")):
        assert rel(g[gname], unit_jacobian(p, pname, J)) < EXACT_TOL, gname
    # nonzero start: still affine in C and in the start state
    p["h0"] = rng.standard_normal((batch, D, N))
    g = oracle.scan_bwd(p["x"], p["dt"], p["B"], p["C"], p["A"], p["Dskip"], L, dy, h0=p["h0"])
    for gname, pname in (("dC", "C"), ("dh0", "h0")):
        assert rel(g[gname], unit_jacobian(p, pname, J)) < EXACT_TOL, gname
    # Dskip enters as Dskip * x: its gradient is sum over batch and tokens of dy * x
    assert rel(g["dDskip"], np.einsum("btd,btd->d", dy, p["x"])) < EXACT_TOL
    # A = 0 and a zero start: every decay is 1 and y is affine in dt
    p = rand64(rng, batch, T, D, N, a_kind="zero")
    p["h0"] = np.zeros((batch, D, N))
    g = oracle.scan_bwd(p["x"], p["dt"], p["B"], p["C"], p["A"], p["Dskip"], L, dy, h0=p["h0"])
    assert rel(g["ddt"], unit_jacobian(p, "dt", J)) < EXACT_TOL


def test_all_block_chain_matches_central_differences():
    """Clean stream: train_scan over T tokens, its block bounds feed the noisy
    stream's blocks (train_blocks).  J = <dy_c, y_c> + <dy_n, y_n>.  The
    gradient of the clean inputs is the continuous backward with dbounds set
    to the noisy backward's block-start gradients."""
    rng = np.random.default_rng(400)
    batch, T, D, N, L = 1, 8, 2, 3, 4
    c = rand64(rng, batch, T, D, N)
    n = rand64(rng, batch, T, D, N)
    n["A"], n["Dskip"] = c["A"], c["Dskip"]
    c["h0"] = rng.standard_normal((batch, D, N))
    dyc = rng.standard_normal((batch, T, D))
    dyn = rng.standard_normal((batch, T, D))

    def J(q):
        r = oracle.scan(q["x"], q["dt"], q["B"], q["C"], q["A"], q["Dskip"], L, h0=q["h0"],
                        want_y=True, want_bounds=True)
        yn = oracle.train_blocks(n["x"], n["dt"], n["B"], n["C"], q["A"], q["Dskip"], L, r["bounds"])
        return float(np.sum(dyc * r["y"]) + np.sum(dyn * yn))

    r = oracle.scan(c["x"], c["dt"], c["B"], c["C"], c["A"], c["Dskip"], L, h0=c["h0"],
                    want_y=True, want_bounds=True)
    gn = oracle.scan_bwd(n["x"], n["dt"], n["B"], n["C"], n["A"], n["Dskip"], L, dyn,
                         h0_blocks=r["bounds"])
    gc = oracle.scan_bwd(c["x"], c["dt"], c["B"], c["C"], c["A"], c["Dskip"], L, dyc, h0=c["h0"],
                         dbounds=gn["dh0_blocks"])
    fd = central_differences(c, ["x", "dt", "B", "C", "h0", "A", "Dskip"], J)
    for gname, pname in (("dx", "x"), ("ddt", "dt"), ("dB", "B"), ("dC", "C"), ("dh0", "h0")):
        assert rel(gc[gname], fd[pname]) < FD_TOL, gname
    # A and Dskip are shared by both streams: their gradients add
    assert rel(gc["dA"] + gn["dA"], fd["A"]) < FD_TOL
    assert rel(gc["dDskip"] + gn["dDskip"], fd["Dskip"]) < FD_TOL


def test_bwd_of_bf16_inputs_equals_bwd_of_their_fp64_values():
    """bf16 inputs are widened exactly: the gradients equal those of the same
    values passed as fp64."""
    rng = np.random.default_rng(500)
    batch, T, D, N, L = 1, 16, 4, 16, 16

    def bf16(a):
        bits = (np.ascontiguousarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)
        return bits, (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)

    (x, xw), (B, Bw), (C, Cw) = (bf16(rng.standard_normal(s)) for s in
                                 ((batch, T, D), (batch, T, N), (batch, T, N)))
    dt, dtw = bf16(np.abs(rng.standard_normal((batch, T, D))))
    A = -np.exp(rng.uniform(-2, 1, (D, N)))
    Dskip = rng.standard_normal(D)
    dy = rng.standard_normal((batch, T, D))
    g16 = oracle.scan_bwd(x, dt, B, C, A, Dskip, L, dy)
    g64 = oracle.scan_bwd(xw, dtw, Bw, Cw, A, Dskip, L, dy)
    for k in g16:
        assert np.array_equal(g16[k], g64[k]), k


def test_bwd_rejects_bad_arguments():
    rng = np.random.default_rng(600)
    p = rand64(rng, 1, 8, 2, 4)
    dy = np.zeros((1, 8, 2))
    with pytest.raises(ValueError):     # T not a multiple of L
        oracle.scan_bwd(p["x"], p["dt"], p["B"], p["C"], p["A"], p["Dskip"], 3, dy)
    with pytest.raises(ValueError):     # both start-state forms at once
        oracle.scan_bwd(p["x"], p["dt"], p["B"], p["C"], p["A"], p["Dskip"], 4, dy,
                        h0=np.zeros((1, 2, 4)), h0_blocks=np.zeros((1, 3, 2, 4)))


def test_bwd_empty_sequence():
    p = rand64(np.random.default_rng(0), 2, 0, 3, 4)
    g = oracle.scan_bwd(p["x"], p["dt"], p["B"], p["C"], p["A"], p["Dskip"], 4,
                        np.zeros((2, 0, 3)), h0=np.ones((2, 3, 4)))
    assert g["dx"].shape == (2, 0, 3) and np.all(g["dA"] == 0) and np.all(g["dh0"] == 0)


# ---- gradients of the fusions (dt = softplus(dt_raw + bias) or dt_raw + bias,
# output times silu(z)), pinned by central differences of the fused forward

def fused_objective_continuous(p, L, dy, dbounds, softplus):
    r = oracle.scan(p["x"], p["dt"], p["B"], p["C"], p["A"], p["Dskip"], L, h0=p["h0"],
                    want_y=True, want_bounds=dbounds is not None, dt_bias=p.get("bias"),
                    dt_softplus=softplus, z=p.get("z"))
    J = float(np.sum(dy * r["y"]))
    if dbounds is not None:
        J += float(np.sum(dbounds * r["bounds"]))
    return J


def fused_objective_blocks(p, L, dy, softplus):
    y = oracle.train_blocks(p["x"], p["dt"], p["B"], p["C"], p["A"], p["Dskip"], L, p["h0_blocks"],
                            dt_bias=p.get("bias"), dt_softplus=softplus, z=p.get("z"))
    return float(np.sum(dy * y))


FUSED_MODES = [("softplus_bias_gate", True, True, True), ("softplus_gate", True, False, True),
               ("softplus_bias", True, True, False), ("bias_gate", False, True, True),
               ("gate_only", False, False, True)]


def fused_inputs(rng, batch, T, D, N, softplus, with_bias, with_gate):
    p = rand64(rng, batch, T, D, N)
    if softplus:
        p["dt"] = rng.normal(-1.0, 0.8, (batch, T, D))       # raw pre-activation, either sign
    if with_bias:
        p["bias"] = rng.normal(0.0, 0.3 if softplus else 0.05, D)
    if with_gate:
        p["z"] = rng.normal(0.0, 1.5, (batch, T, D))
    return p


@pytest.mark.parametrize("mode,softplus,with_bias,with_gate", FUSED_MODES)
def test_fused_continuous_gradient_matches_central_differences(mode, softplus, with_bias, with_gate):
    rng = np.random.default_rng(300 + len(mode))
    batch, T, D, N, L = 2, 8, 3, 4, 4
    p = fused_inputs(rng, batch, T, D, N, softplus, with_bias, with_gate)
    p["h0"] = rng.standard_normal((batch, D, N))
    dy = rng.standard_normal((batch, T, D))
    db = rng.standard_normal((batch, T // L + 1, D, N))
    g = oracle.scan_bwd(p["x"], p["dt"], p["B"], p["C"], p["A"], p["Dskip"], L, dy, h0=p["h0"],
                        dbounds=db, dt_bias=p.get("bias"), dt_softplus=softplus, z=p.get("z"))
    names = ["x", "dt", "B", "C", "A", "Dskip", "h0"] + (["bias"] if with_bias else []) + \
        (["z"] if with_gate else [])
    fd = central_differences(p, names, lambda q: fused_objective_continuous(q, L, dy, db, softplus))
    pairs = [("dx", "x"), ("ddt", "dt"), ("dB", "B"), ("dC", "C"), ("dA", "A"), ("dDskip", "Dskip"),
             ("dh0", "h0")]
    if with_bias:
        pairs.append(("d_dt_bias", "bias"))
    if with_gate:
        pairs.append(("dz", "z"))
    for gname, pname in pairs:
        assert rel(g[gname], fd[pname]) < FD_TOL, (mode, gname, rel(g[gname], fd[pname]))


@pytest.mark.parametrize("mode,softplus,with_bias,with_gate", FUSED_MODES[:2] + FUSED_MODES[3:4])
def test_fused_two_stream_gradient_matches_central_differences(mode, softplus, with_bias, with_gate):
    rng = np.random.default_rng(400 + len(mode))
    batch, T, D, N, L = 2, 8, 3, 4, 2
    p = fused_inputs(rng, batch, T, D, N, softplus, with_bias, with_gate)
    p["h0_blocks"] = rng.standard_normal((batch, T // L + 1, D, N))
    dy = rng.standard_normal((batch, T, D))
    g = oracle.scan_bwd(p["x"], p["dt"], p["B"], p["C"], p["A"], p["Dskip"], L, dy,
                        h0_blocks=p["h0_blocks"], dt_bias=p.get("bias"), dt_softplus=softplus,
                        z=p.get("z"))
    names = ["x", "dt", "B", "C", "A", "Dskip", "h0_blocks"] + (["bias"] if with_bias else []) + \
        (["z"] if with_gate else [])
    fd = central_differences(p, names, lambda q: fused_objective_blocks(q, L, dy, softplus))
    pairs = [("dx", "x"), ("ddt", "dt"), ("dB", "B"), ("dC", "C"), ("dA", "A"), ("dDskip", "Dskip"),
             ("dh0_blocks", "h0_blocks")]
    if with_bias:
        pairs.append(("d_dt_bias", "bias"))
    if with_gate:
        pairs.append(("dz", "z"))
    for gname, pname in pairs:
        assert rel(g[gname], fd[pname]) < FD_TOL, (mode, gname, rel(g[gname], fd[pname]))


def test_fused_gradients_without_fusion_arguments_are_the_plain_ones():
    rng = np.random.default_rng(500)
    batch, T, D, N, L = 2, 16, 3, 4, 4
    p = rand64(rng, batch, T, D, N)
    dy = rng.standard_normal((batch, T, D))
    a = oracle.scan_bwd(p["x"], p["dt"], p["B"], p["C"], p["A"], p["Dskip"], L, dy)
    b = oracle.scan_bwd(p["x"], p["dt"], p["B"], p["C"], p["A"], p["Dskip"], L, dy, dt_bias=None,
                        dt_softplus=False, z=None)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


# ---- gradients with separate reverse-direction operands (dt_r, B_r, C_r, A_r and
# the reverse bias), pinned by central differences of the forward that uses them

def sep_inputs(rng, batch, T, D, N, softplus, fused):
    p = fused_inputs(rng, batch, T, D, N, softplus, fused, fused)
    q = rand64(rng, batch, T, D, N)
    p["dt_r"] = rng.normal(-1.0, 0.8, (batch, T, D)) if softplus else q["dt"]
    p["B_r"], p["C_r"], p["A_r"] = q["B"], q["C"], q["A"]
    if fused:
        p["bias_r"] = rng.normal(0.0, 0.3 if softplus else 0.05, D)
    return p


def sep_rev(p):
    return dict(dt=p["dt_r"], B=p["B_r"], C=p["C_r"], A=p["A_r"], dt_bias=p.get("bias_r"))


SEP_MODES = [("plain", False, False), ("softplus_bias_gate", True, True)]
SEP_PAIRS = [("dx", "x"), ("ddt", "dt"), ("dB", "B"), ("dC", "C"), ("dA", "A"), ("dDskip", "Dskip"),
             ("ddt_rev", "dt_r"), ("dB_rev", "B_r"), ("dC_rev", "C_r"), ("dA_rev", "A_r")]


@pytest.mark.parametrize("mode,softplus,fused", SEP_MODES)
def test_separate_reverse_operands_continuous_gradient(mode, softplus, fused):
    rng = np.random.default_rng(700 + len(mode))
    batch, T, D, N, L = 2, 8, 3, 4, 4
    p = sep_inputs(rng, batch, T, D, N, softplus, fused)
    p["h0"] = rng.standard_normal((batch, D, N))
    dy = rng.standard_normal((batch, T, D))
    db = rng.standard_normal((batch, T // L + 1, D, N))

    def J(q):
        r = oracle.scan(q["x"], q["dt"], q["B"], q["C"], q["A"], q["Dskip"], L, h0=q["h0"], want_y=True,
                        want_bounds=True, dt_bias=q.get("bias"), dt_softplus=softplus, z=q.get("z"),
                        rev=sep_rev(q))
        return float(np.sum(dy * r["y"]) + np.sum(db * r["bounds"]))

    g = oracle.scan_bwd(p["x"], p["dt"], p["B"], p["C"], p["A"], p["Dskip"], L, dy, h0=p["h0"],
                        dbounds=db, dt_bias=p.get("bias"), dt_softplus=softplus, z=p.get("z"),
                        rev=sep_rev(p))
    pairs = SEP_PAIRS + [("dh0", "h0")]
    if fused:
        pairs += [("d_dt_bias", "bias"), ("d_dt_bias_rev", "bias_r"), ("dz", "z")]
    fd = central_differences(p, [pn for _, pn in pairs], J)
    for gname, pname in pairs:
        assert rel(g[gname], fd[pname]) < FD_TOL, (mode, gname, rel(g[gname], fd[pname]))


@pytest.mark.parametrize("mode,softplus,fused", SEP_MODES)
def test_separate_reverse_operands_two_stream_gradient(mode, softplus, fused):
    rng = np.random.default_rng(800 + len(mode))
    batch, T, D, N, L = 2, 8, 3, 4, 2
    p = sep_inputs(rng, batch, T, D, N, softplus, fused)
    p["h0_blocks"] = rng.standard_normal((batch, T // L + 1, D, N))
    dy = rng.standard_normal((batch, T, D))

    def J(q):
        y = oracle.train_blocks(q["x"], q["dt"], q["B"], q["C"], q["A"], q["Dskip"], L, q["h0_blocks"],
                                dt_bias=q.get("bias"), dt_softplus=softplus, z=q.get("z"), rev=sep_rev(q))
        return float(np.sum(dy * y))

    g = oracle.scan_bwd(p["x"], p["dt"], p["B"], p["C"], p["A"], p["Dskip"], L, dy,
                        h0_blocks=p["h0_blocks"], dt_bias=p.get("bias"), dt_softplus=softplus,
                        z=p.get("z"), rev=sep_rev(p))
    pairs = SEP_PAIRS + [("dh0_blocks", "h0_blocks")]
    if fused:
        pairs += [("d_dt_bias", "bias"), ("d_dt_bias_rev", "bias_r"), ("dz", "z")]
    fd = central_differences(p, [pn for _, pn in pairs], J)
    for gname, pname in pairs:
        assert rel(g[gname], fd[pname]) < FD_TOL, (mode, gname, rel(g[gname], fd[pname]))


def test_separate_operands_equal_to_the_forwards_split_the_shared_gradients():
    """With the reverse given the forward's own operands, each shared operand's
    gradient is the sum of its two direction's parts (the shared routine's
    result), and the gradients of the rest agree."""
    rng = np.random.default_rng(900)
    batch, T, D, N, L = 2, 16, 3, 4, 4
    p = rand64(rng, batch, T, D, N)
    dy = rng.standard_normal((batch, T, D))
    bias = rng.normal(0.0, 0.3, D)
    dtr = rng.normal(-1.0, 0.8, (batch, T, D))
    shared = oracle.scan_bwd(p["x"], dtr, p["B"], p["C"], p["A"], p["Dskip"], L, dy, dt_bias=bias,
                             dt_softplus=True)
    sep = oracle.scan_bwd(p["x"], dtr, p["B"], p["C"], p["A"], p["Dskip"], L, dy, dt_bias=bias,
                          dt_softplus=True, rev=dict(dt=dtr, B=p["B"], C=p["C"], A=p["A"], dt_bias=bias))
    for k, kr in (("ddt", "ddt_rev"), ("dB", "dB_rev"), ("dC", "dC_rev"), ("dA", "dA_rev"),
                  ("d_dt_bias", "d_dt_bias_rev")):
        assert rel(sep[k] + sep[kr], shared[k]) < 1e-12, k
    for k in ("dx", "dDskip", "dh0"):
        assert rel(sep[k], shared[k]) < 1e-12, k
