"""Pins for the oracle's optional Mamba-1 fusions around the scan (the step
size dt = softplus(dt_raw + bias) and the output gate y * silu(z)), checked
against the unfused oracle (pinned in test_oracle.py) fed with the transform
computed by library routines: numpy.logaddexp for softplus, scipy's expit for
the sigmoid.
"""
import numpy as np
import pytest
from scipy.special import expit

import oracle


def inputs(rng, batch, T, D, N, raw_mean=-1.0, raw_std=0.5):
    x = rng.standard_normal((batch, T, D))
    raw = rng.normal(raw_mean, raw_std, (batch, T, D))
    B = rng.standard_normal((batch, T, N))
    C = rng.standard_normal((batch, T, N))
    A = -np.exp(rng.uniform(np.log(0.05), np.log(4.0), (D, N)))
    Dskip = rng.standard_normal(D)
    bias = rng.normal(0.0, 0.5, D)
    z = rng.standard_normal((batch, T, D)) * 2.0
    return x, raw, B, C, A, Dskip, bias, z


def rel(g, r):
    floor = np.sqrt(np.mean(r * r)) + 1e-300
    return float(np.max(np.abs(g - r) / np.maximum(np.abs(r), floor)))


@pytest.mark.parametrize("L", [1, 4, 16])
def test_softplus_step_equals_library_softplus(L):
    rng = np.random.default_rng(700 + L)
    x, raw, B, C, A, Ds, bias, _ = inputs(rng, 2, 32, 3, 4)
    h0 = rng.standard_normal((2, 3, 4))
    fused = oracle.scan(x, raw, B, C, A, Ds, L, h0=h0, want_bounds=True, dt_bias=bias, dt_softplus=True)
    dt = np.logaddexp(0.0, raw + bias)
    plain = oracle.scan(x, dt, B, C, A, Ds, L, h0=h0, want_bounds=True)
    for k in ("y", "hT", "bounds"):
        assert rel(fused[k], plain[k]) < 1e-12, k


def test_softplus_extreme_arguments():
    """Large positive and negative arguments: softplus(v) -> v and -> e^v
    without overflow or loss of the small values."""
    rng = np.random.default_rng(710)
    x, _, B, C, A, Ds, _, _ = inputs(rng, 1, 64, 2, 4)
    raw = np.linspace(-40.0, 40.0, 64 * 2).reshape(1, 64, 2)
    fused = oracle.scan(x, raw, B, C, A, Ds, 16, dt_softplus=True)
    plain = oracle.scan(x, np.logaddexp(0.0, raw), B, C, A, Ds, 16)
    assert np.all(np.isfinite(fused["y"]))
    assert rel(fused["y"], plain["y"]) < 1e-12


def test_bias_without_softplus_is_a_plain_shift():
    rng = np.random.default_rng(720)
    x, raw, B, C, A, Ds, bias, _ = inputs(rng, 2, 16, 3, 4, raw_mean=0.5, raw_std=0.1)
    fused = oracle.scan(x, raw, B, C, A, Ds, 8, dt_bias=bias)
    plain = oracle.scan(x, raw + bias, B, C, A, Ds, 8)
    assert np.array_equal(fused["y"], plain["y"]) and np.array_equal(fused["hT"], plain["hT"])


@pytest.mark.parametrize("L", [2, 16])
def test_gate_is_silu(L):
    rng = np.random.default_rng(730 + L)
    x, raw, B, C, A, Ds, bias, z = inputs(rng, 2, 32, 3, 4)
    dt = np.logaddexp(0.0, raw)
    gated = oracle.scan(x, dt, B, C, A, Ds, L, z=z)
    plain = oracle.scan(x, dt, B, C, A, Ds, L)
    assert rel(gated["y"], plain["y"] * z * expit(z)) < 1e-12
    # the gate acts on the output only: states are unchanged
    assert np.array_equal(gated["hT"], plain["hT"])


def test_two_stream_form_fusions():
    rng = np.random.default_rng(740)
    L = 4
    x, raw, B, C, A, Ds, bias, z = inputs(rng, 2, 16, 3, 4)
    h0b = rng.standard_normal((2, 16 // L + 1, 3, 4))
    fused = oracle.train_blocks(x, raw, B, C, A, Ds, L, h0b, dt_bias=bias, dt_softplus=True, z=z)
    plain = oracle.train_blocks(x, np.logaddexp(0.0, raw + bias), B, C, A, Ds, L, h0b)
    assert rel(fused, plain * z * expit(z)) < 1e-12


def test_fusions_of_bf16_inputs_widen_exactly():
    rng = np.random.default_rng(750)
    x, raw, B, C, A, Ds, bias, z = inputs(rng, 1, 16, 4, 4)

    def bf16(a):
        bits = (np.ascontiguousarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)
        return bits, (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)

    (xb, xw), (rb, rw), (Bb, Bw), (Cb, Cw), (zb, zw) = (bf16(a) for a in (x, raw, B, C, z))
    a = oracle.scan(xb, rb, Bb, Cb, A, Ds, 16, dt_bias=bias, dt_softplus=True, z=zb)
    b = oracle.scan(xw, rw, Bw, Cw, A, Ds, 16, dt_bias=bias, dt_softplus=True, z=zw)
    assert np.array_equal(a["y"], b["y"])


# ---- separate reverse-direction operands

def rev_operands(rng, batch, T, D, N):
    return dict(dt=np.log1p(np.exp(rng.normal(-0.5, 0.5, (batch, T, D)))),
                B=rng.standard_normal((batch, T, N)), C=rng.standard_normal((batch, T, N)),
                A=-np.exp(rng.uniform(np.log(0.05), np.log(4.0), (D, N))))


def test_reverse_operands_equal_to_forward_are_the_shared_scan():
    rng = np.random.default_rng(760)
    x, raw, B, C, A, Ds, bias, z = inputs(rng, 2, 32, 3, 4)
    dt = np.log1p(np.exp(raw))
    shared = oracle.scan(x, dt, B, C, A, Ds, 8, want_parts=True)
    same = oracle.scan(x, dt, B, C, A, Ds, 8, want_parts=True, rev=dict(dt=dt, B=B, C=C, A=A))
    for k in ("y", "yf", "yr", "hT"):
        assert np.array_equal(shared[k], same[k]), k


def test_reverse_operands_leave_the_forward_and_the_cache_alone():
    rng = np.random.default_rng(770)
    x, raw, B, C, A, Ds, bias, z = inputs(rng, 2, 32, 3, 4)
    dt = np.log1p(np.exp(raw))
    rev = rev_operands(rng, 2, 32, 3, 4)
    a = oracle.scan(x, dt, B, C, A, Ds, 8, want_parts=True, want_bounds=True)
    b = oracle.scan(x, dt, B, C, A, Ds, 8, want_parts=True, want_bounds=True, rev=rev)
    for k in ("yf", "hT", "bounds"):
        assert np.array_equal(a[k], b[k]), k
    assert not np.allclose(a["yr"], b["yr"])


@pytest.mark.parametrize("softplus", [False, True])
def test_reverse_with_own_operands_is_the_flipped_forward_of_them(softplus):
    """With one block covering the row, the reverse part equals the forward
    scan (from zero) of the time-flipped inputs taken with the reverse
    operands, flipped back."""
    rng = np.random.default_rng(780 + softplus)
    T = 24
    x, raw, B, C, A, Ds, bias, z = inputs(rng, 2, T, 3, 4)
    rev = rev_operands(rng, 2, T, 3, 4)
    rev["dt_bias"] = rng.normal(0.0, 0.3, 3)
    dt = raw if softplus else np.log1p(np.exp(raw))
    got = oracle.scan(x, dt, B, C, A, Ds, T, want_parts=True, rev=rev, dt_softplus=softplus,
                      dt_bias=bias)["yr"]
    f = lambda a: np.ascontiguousarray(a[:, ::-1])
    ref = oracle.scan(f(x), f(rev["dt"]), f(rev["B"]), f(rev["C"]), rev["A"], Ds, T, want_parts=True,
                      dt_softplus=softplus, dt_bias=rev["dt_bias"])["yf"]
    assert rel(got, f(ref)) < 1e-12


def test_two_stream_form_with_reverse_operands():
    rng = np.random.default_rng(790)
    L, T = 4, 16
    x, raw, B, C, A, Ds, bias, z = inputs(rng, 2, T, 3, 4)
    dt = np.log1p(np.exp(raw))
    rev = rev_operands(rng, 2, T, 3, 4)
    r = oracle.scan(x, dt, B, C, A, Ds, L, want_bounds=True, rev=rev, z=z)
    yb = oracle.train_blocks(x, dt, B, C, A, Ds, L, r["bounds"], rev=rev, z=z)
    assert rel(yb, r["y"]) < 1e-13
