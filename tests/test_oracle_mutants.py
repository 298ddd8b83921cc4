"""The oracle's pins must be strong enough to notice a plausible slip.

Each case copies the oracle's C source to a temporary directory, plants one
mistake in that copy, builds it, points the oracle wrapper at the mutant and
runs every pin of tests/test_oracle.py.  At least one pin must fail for every
mutant.  Nothing here touches the real oracle library or any GPU code.
"""
import ctypes
import inspect
import os
import subprocess

import pytest

import oracle
from oracle import oracle as _oracle_mod
import test_oracle as pins

SRC = os.path.join(os.path.dirname(_oracle_mod.__file__), "bdssm_oracle.c")

MUTANTS = {
    "drop_skip_term": ("y[ix] = fwd[t] + acc + (double)Dskip[d] * xv;", "y[ix] = fwd[t] + acc;"),
    "decay_sign": ("const double decay = exp(dtv * (double)A[d * N + n]);\n                    const double inject",
                   "const double decay = exp(-dtv * (double)A[d * N + n]);\n                    const double inject"),
    "reverse_exclusive": ("r[n] = decay * r[n] + inject;\n                            acc += ld(Cm, ib + n, dtype) * r[n];",
                          "acc += ld(Cm, ib + n, dtype) * r[n];\n                            r[n] = decay * r[n] + inject;"),
    "B_C_swapped": ("const double inject = dtv * ld(Bm, ib + n, dtype) * xv;\n                    h[n]",
                    "const double inject = dtv * ld(Cm, ib + n, dtype) * xv;\n                    h[n]"),
    "A_transposed": ("const double decay = exp(dtv * (double)A[d * N + n]);\n                    const double inject",
                     "const double decay = exp(dtv * (double)A[n * D + d]);\n                    const double inject"),
    "ignore_initial_state": ("h[n] = h0 ? h0[(b * D + d) * N + n] : 0.0;", "h[n] = 0.0;"),
    "reverse_not_reset": ("for (int64_t n = 0; n < N; ++n) r[n] = 0.0;\n", ""),
    "no_reverse": ("if (y) y[ix] = fwd[t] + acc +", "if (y) y[ix] = fwd[t] + 0.0 * acc +"),
    "forward_reset_per_block": ("if (bounds && (t + 1) % L == 0)",
                                "if ((t + 1) % L == 0) for (int64_t n = 0; n < N; ++n) h[n] = 0.0;\n"
                                "                if (bounds && (t + 1) % L == 0)"),
    "reverse_blocks_shifted": ("for (int64_t t = k * L + L - 1; t >= k * L; --t) {",
                               "for (int64_t t = (k * L + L) % T; t > k * L; --t) {"),
    "inject_missing_dt": ("const double inject = dtv * ld(Bm, ib + n, dtype) * xv;\n                    h[n]",
                          "const double inject = ld(Bm, ib + n, dtype) * xv;\n                    h[n]"),
}


def _pin_functions():
    out = []
    for name, fn in inspect.getmembers(pins, inspect.isfunction):
        if not name.startswith("test_") or name == "test_rejects_bad_arguments":
            continue
        params = getattr(fn, "pytestmark", [])
        cases = [()]
        for m in params:
            if m.name == "parametrize":
                cases = [(v,) for v in m.args[1]]
        for c in cases:
            out.append((name, fn, c))
    return out


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_some_pin_catches_mutant(mutant, tmp_path):
    old, new = MUTANTS[mutant]
    src = open(SRC).read()
    assert src.count(old) >= 1, "mutation anchor not found: %s" % mutant
    mutated = src.replace(old, new, 1)
    cpath = tmp_path / "mut.c"
    cpath.write_text(mutated)
    so = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-o", str(so), str(cpath), "-lm"],
                   check=True)
    lib = ctypes.CDLL(str(so))
    P = ctypes.c_void_p
    I = ctypes.c_int64
    lib.oracle_scan.argtypes = [I, I, I, I, I, ctypes.c_int] + [P] * 12
    lib.oracle_scan.restype = ctypes.c_int
    saved = _oracle_mod._lib
    _oracle_mod._lib = lib
    caught = []
    try:
        for name, fn, case in _pin_functions():
            try:
                fn(*case)
            except (AssertionError, ValueError, IndexError):
                caught.append(name)
    finally:
        _oracle_mod._lib = saved
    assert caught, "no pin noticed mutant %s" % mutant
