"""The oracle's pins must be strong enough to notice a plausible slip.

Each case copies the oracle's C source to a temporary directory, plants one
mistake in that copy, builds it, points the oracle wrapper at the mutant and
runs every pin of tests/test_oracle.py (forward mutants) or of
tests/test_oracle_bwd.py (mutants of the gradient routine).  At least one pin
must fail for every mutant.  Nothing here touches the real oracle library or
any GPU code.
"""
import ctypes
import inspect
import os
import subprocess

import pytest

import oracle
from oracle import oracle as _oracle_mod
import test_oracle as pins
import test_oracle_bwd as bwd_pins
import test_oracle_fused as fused_pins

SRC = os.path.join(os.path.dirname(_oracle_mod.__file__), "bdssm_oracle.c")

MUTANTS = {
    "drop_skip_term": ("if (y) y[ix] = (fwd[t] + acc + Dskip[d] * xv) *", "if (y) y[ix] = (fwd[t] + acc) *"),
    "decay_sign": ("const double decay = exp(dtv * A[d * N + n]);\n                    const double inject",
                   "const double decay = exp(-dtv * A[d * N + n]);\n                    const double inject"),
    "reverse_exclusive": ("r[n] = decay * r[n] + inject;\n                            acc += ld(rv.Cm, ib + n, dtype) * r[n];",
                          "acc += ld(rv.Cm, ib + n, dtype) * r[n];\n                            r[n] = decay * r[n] + inject;"),
    "B_C_swapped": ("const double inject = dtv * ld(Bm, ib + n, dtype) * xv;\n                    h[n]",
                    "const double inject = dtv * ld(Cm, ib + n, dtype) * xv;\n                    h[n]"),
    "A_transposed": ("const double decay = exp(dtv * A[d * N + n]);\n                    const double inject",
                     "const double decay = exp(dtv * A[n * D + d]);\n                    const double inject"),
    "ignore_initial_state": ("h[n] = h0 ? h0[(b * D + d) * N + n] : 0.0;", "h[n] = 0.0;"),
    "reverse_not_reset": ("for (int64_t n = 0; n < N; ++n) r[n] = 0.0;\n", ""),
    "no_reverse": ("if (y) y[ix] = (fwd[t] + acc +", "if (y) y[ix] = (fwd[t] + 0.0 * acc +"),
    "forward_reset_per_block": ("if (bounds && (t + 1) % L == 0)",
                                "if ((t + 1) % L == 0) for (int64_t n = 0; n < N; ++n) h[n] = 0.0;\n"
                                "                if (bounds && (t + 1) % L == 0)"),
    "reverse_blocks_shifted": ("for (int64_t t = k * L + L - 1; t >= k * L; --t) {",
                               "for (int64_t t = (k * L + L) % T; t > k * L; --t) {"),
    "inject_missing_dt": ("const double inject = dtv * ld(Bm, ib + n, dtype) * xv;\n                    h[n]",
                          "const double inject = ld(Bm, ib + n, dtype) * xv;\n                    h[n]"),
}

MUTANTS_BWD = {
    "bwd_reverse_adjoint_no_decay": ("q[n] = a[t * N + n] * g;", "q[n] = g;"),
    "bwd_da_missing_reverse_term": ("const double da = gf * hp[t * N + n] + gr[t * N + n] * rn[t * N + n];",
                                    "const double da = gf * hp[t * N + n];"),
    "bwd_dbounds_ignored": ("if (!blocks && block_end && dbounds)", "if (0)"),
    "bwd_ddt_missing_decay_term": ("sdt += du * bv * xv + da * at * A[d * N + n];",
                                   "sdt += du * bv * xv;"),
    "bwd_dC_forward_only": ("const double hsum = (at * hp[t * N + n] + u) + (at * rn[t * N + n] + u);",
                            "const double hsum = (at * hp[t * N + n] + u);"),
    "bwd_two_stream_adjoint_crosses_blocks": ("if (blocks && block_end)\n                        for (int64_t n = 0; n < N; ++n) q[n] = 0.0;",
                                              ""),
    "bwd_forward_adjoint_no_decay": ("q[n] = at * gf;", "q[n] = gf;"),
    "bwd_dx_missing_skip": ("dx[ix] = sx + gy * Dskip[d];", "dx[ix] = sx;"),
    "bwd_dB_missing_dt": ("my_dB[ib + n] += du * dtv * xv;", "my_dB[ib + n] += du * xv;"),
    "bwd_dA_missing_dt": ("my_dA[d * N + n] += da * at * dtv;", "my_dA[d * N + n] += da * at;"),
    # gradients of the fusions
    "bwd_softplus_derivative_missing": ("const double draw = dt_softplus ? sdt * sigmoid(vraw) : sdt;",
                                        "const double draw = sdt;"),
    "bwd_gate_not_applied_to_dy": ("const double gy = z ? dy[ix] * silu(zv) : dy[ix];",
                                   "const double gy = dy[ix];"),
    "bwd_dz_missing_derivative_term": ("dz[ix] = dy[ix] * ypre * s * (1.0 + zv * (1.0 - s));",
                                       "dz[ix] = dy[ix] * ypre * s;"),
    "bwd_ypre_missing_skip": ("double sdt = 0.0, sx = 0.0, ypre = Dskip[d] * xv;",
                              "double sdt = 0.0, sx = 0.0, ypre = 0.0;"),
    "bwd_dbias_before_softplus": ("my_dbias[d] += draw;", "my_dbias[d] += sdt;"),
    # gradients with separate reverse operands
    "sep_reverse_adjoint_uses_forward_C": ("const double g = gy * ld(C_r, ib + n, dtype) + q[n];",
                                           "const double g = gy * ld(Cm, ib + n, dtype) + q[n];"),
    "sep_dBr_uses_forward_dt": ("my_dBr[ib + n] += g_r * dtr * xv;", "my_dBr[ib + n] += g_r * dtv * xv;"),
    "sep_dx_missing_reverse_term": ("sx += gf * dtv * bv + g_r * dtr * bvr;", "sx += gf * dtv * bv;"),
    "sep_reverse_decay_uses_forward_A": ("const double at = exp(dtr * A_r[d * N + n]);",
                                         "const double at = exp(dtr * A[d * N + n]);"),
    "sep_dAr_missing_decay": ("my_dAr[d * N + n] += da_r * atr * dtr;", "my_dAr[d * N + n] += da_r * dtr;"),
}

MUTANTS_FUSED = {
    "softplus_wrong_branch": ("return v > 0.0 ? v + log1p(exp(-v)) : log1p(exp(v));",
                              "return v > 0.0 ? v + log1p(exp(v)) : log1p(exp(v));"),
    "bias_ignored": ("const double v = raw + bias;", "const double v = raw;"),
    "gate_is_sigmoid": ("static double silu(double z) { return z / (1.0 + exp(-z)); }",
                        "static double silu(double z) { return 1.0 / (1.0 + exp(-z)); }"),
    "reverse_uses_forward_A": ("const double decay = exp(dtv * rv.A[d * N + n]);\n                            const double inject = dtv * ld(rv.Bm",
                               "const double decay = exp(dtv * A[d * N + n]);\n                            const double inject = dtv * ld(rv.Bm"),
    "reverse_uses_forward_C": ("acc += ld(rv.Cm, ib + n, dtype) * r[n];\n                        }\n                        if (yf)",
                               "acc += ld(Cm, ib + n, dtype) * r[n];\n                        }\n                        if (yf)"),
    "reverse_uses_forward_bias": ("const double dtv = step_size(ld(rv.dt, ix, dtype), rv.dt_bias ? rv.dt_bias[d] : 0.0, dt_softplus);\n                        const double xv",
                                  "const double dtv = step_size(ld(rv.dt, ix, dtype), dt_bias ? dt_bias[d] : 0.0, dt_softplus);\n                        const double xv"),
    "gate_missing": ("if (y) y[ix] = (fwd[t] + acc + Dskip[d] * xv) * (z ? silu(ld(z, ix, dtype)) : 1.0);",
                     "if (y) y[ix] = (fwd[t] + acc + Dskip[d] * xv);"),
}


def _pin_functions(module=pins):
    out = []
    for name, fn in inspect.getmembers(module, inspect.isfunction):
        if not name.startswith("test_") or name in ("test_rejects_bad_arguments",
                                                     "test_bwd_rejects_bad_arguments"):
            continue
        params = getattr(fn, "pytestmark", [])
        cases = [()]
        for m in params:
            if m.name == "parametrize":
                multi = "," in m.args[0]
                cases = [tuple(v) if multi else (v,) for v in m.args[1]]
        for c in cases:
            out.append((name, fn, c))
    return out


def _run_mutant(old, new, tmp_path, module):
    src = open(SRC).read()
    assert src.count(old) >= 1, "mutation anchor not found"
    mutated = src.replace(old, new, 1)
    cpath = tmp_path / "mut.c"
    cpath.write_text(mutated)
    so = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-o", str(so), str(cpath), "-lm"],
                   check=True)
    lib = _oracle_mod.bind(ctypes.CDLL(str(so)))
    saved = _oracle_mod._lib
    _oracle_mod._lib = lib
    caught = []
    try:
        for name, fn, case in _pin_functions(module):
            try:
                fn(*case)
            except (AssertionError, ValueError, IndexError):
                caught.append(name)
    finally:
        _oracle_mod._lib = saved
    return caught


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_some_pin_catches_mutant(mutant, tmp_path):
    old, new = MUTANTS[mutant]
    assert _run_mutant(old, new, tmp_path, pins), "no pin noticed mutant %s" % mutant


@pytest.mark.parametrize("mutant", sorted(MUTANTS_BWD))
def test_some_gradient_pin_catches_mutant(mutant, tmp_path):
    old, new = MUTANTS_BWD[mutant]
    assert _run_mutant(old, new, tmp_path, bwd_pins), "no gradient pin noticed mutant %s" % mutant


@pytest.mark.parametrize("mutant", sorted(MUTANTS_FUSED))
def test_some_fusion_pin_catches_mutant(mutant, tmp_path):
    old, new = MUTANTS_FUSED[mutant]
    assert _run_mutant(old, new, tmp_path, fused_pins), "no fusion pin noticed mutant %s" % mutant
