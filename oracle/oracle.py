"""ctypes marshalling for the fp64 oracle (TEST INFRASTRUCTURE ONLY).

Stream inputs (x, dt, B, C) are numpy arrays: float32, float64, or bfloat16
passed as their raw uint16 bit patterns (``dtype=np.uint16``).  A and Dskip
are passed to the C code as float64 (float32 values convert exactly).  States
and every output are float64.  Shapes follow the library: x, dt, y: [batch, T, D];
B, C: [batch, T, N]; A: [D, N]; Dskip: [D]; states: [batch, D, N].
"""
import ctypes
import os
import subprocess

import numpy as np

F32 = 0
BF16 = 1
F64 = 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bdssm_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


# the sanitizer build (address + undefined behaviour, host code only): a
# process that loads it needs the ASan runtime preloaded (LD_PRELOAD)
SANITIZE_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                  "-fno-sanitize-recover=all"]


def build(force=True, sanitize=False, out=None):
    """Compile the C oracle into oracle/liboracle.so (or `out`) with gcc +
    OpenMP; sanitize=True builds with AddressSanitizer and UBSan."""
    lib = out or _LIB
    if not force and os.path.exists(lib) and os.path.getmtime(lib) >= os.path.getmtime(_SRC):
        return lib
    tmp = lib + ".tmp%d" % os.getpid()
    opt = SANITIZE_FLAGS if sanitize else ["-O2"]
    cmd = ["gcc"] + opt + ["-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
                           "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


def bind(lib):
    """Declare the C signatures on a loaded oracle library."""
    P = ctypes.c_void_p
    I = ctypes.c_int64
    lib.oracle_scan.argtypes = [I, I, I, I, I, ctypes.c_int] + [P] * 12
    lib.oracle_scan.restype = ctypes.c_int
    lib.oracle_scan_ex.argtypes = ([I, I, I, I, I, ctypes.c_int] + [P] * 8 + [ctypes.c_int]
                                   + [P] * 11)
    lib.oracle_scan_ex.restype = ctypes.c_int
    lib.oracle_train_blocks_ex.argtypes = ([I, I, I, I, I, ctypes.c_int] + [P] * 8 + [ctypes.c_int]
                                           + [P] * 7)
    lib.oracle_train_blocks_ex.restype = ctypes.c_int
    lib.oracle_version.restype = ctypes.c_int
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_train_blocks.argtypes = [I, I, I, I, I, ctypes.c_int] + [P] * 8
    lib.oracle_train_blocks.restype = ctypes.c_int
    lib.oracle_scan_bwd.argtypes = ([I, I, I, I, I, ctypes.c_int] + [P] * 6 + [ctypes.c_int]
                                    + [P] * 12)
    lib.oracle_scan_bwd.restype = ctypes.c_int
    lib.oracle_scan_bwd_ex.argtypes = ([I, I, I, I, I, ctypes.c_int] + [P] * 6 + [ctypes.c_int]
                                       + [P] * 5 + [ctypes.c_int] + [P] * 11)
    lib.oracle_scan_bwd_ex.restype = ctypes.c_int
    lib.oracle_scan_bwd_sep.argtypes = ([I, I, I, I, I, ctypes.c_int] + [P] * 6 + [ctypes.c_int]
                                        + [P] * 5 + [ctypes.c_int] + [P] * 6 + [P] * 15)
    lib.oracle_scan_bwd_sep.restype = ctypes.c_int
    return lib


def load():
    """The oracle library: oracle/liboracle.so (built if missing or stale), or
    the build named by BDSSM_ORACLE_LIB (e.g. the sanitizer build)."""
    global _lib
    if _lib is None:
        path = os.environ.get("BDSSM_ORACLE_LIB")
        if not path:
            path = _LIB
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build()
        _lib = bind(ctypes.CDLL(path))
    return _lib


def num_threads():
    """Threads the oracle's row loop uses."""
    return load().oracle_num_threads()


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(a):
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float64:
        return F64
    raise TypeError("oracle inputs must be float32, float64 or bf16 bits (uint16), got %s" % a.dtype)


def _c(a, dt=None):
    if a is None:
        return None
    a = np.asarray(a)
    if dt is not None:
        a = a.astype(dt, copy=False)
    return np.ascontiguousarray(a)


def _reverse(x, B, A, rev):
    """Marshal separate reverse-direction operands: dict with dt, B, C, A and
    optionally dt_bias, or None (the reverse shares the forward's)."""
    if rev is None:
        return (None,) * 5
    dt_r, B_r, C_r = _c(rev["dt"]), _c(rev["B"]), _c(rev["C"])
    A_r = _c(rev["A"], np.float64)
    bias_r = _c(rev.get("dt_bias"), np.float64)
    for a in (dt_r, B_r, C_r):
        if a.dtype != x.dtype:
            raise TypeError("reverse operands must share x's dtype")
    assert dt_r.shape == x.shape and B_r.shape == B.shape and C_r.shape == B.shape
    assert A_r.shape == A.shape
    return dt_r, B_r, C_r, A_r, bias_r


def _fusion(x, D, dt_bias, z):
    """Marshal the optional fusions: dt_bias [D] (float64), z (x's dtype)."""
    bias = _c(dt_bias, np.float64)
    if bias is not None:
        assert bias.shape == (D,)
    zz = _c(z)
    if zz is not None:
        if zz.dtype != x.dtype or zz.shape != x.shape:
            raise TypeError("z must match x in dtype and shape")
    return bias, zz


def scan(x, dt, B, C, A, Dskip, L, h0=None, want_y=True, want_parts=False, want_bounds=False,
         dt_bias=None, dt_softplus=False, z=None, rev=None):
    """Core oracle: continuous forward from h0, reverse segmented into L-token
    blocks.  Returns a dict with 'y' (and 'yf', 'yr' if want_parts), 'hT',
    and 'bounds' ([batch, T/L+1, D, N]) if want_bounds.  Optional fusions:
    dt <- dt + dt_bias, then softplus if dt_softplus; y <- y * silu(z).
    rev: separate reverse-direction operands {dt, B, C, A[, dt_bias]}."""
    x, dt, B = _c(x), _c(dt), _c(B)
    C = _c(C)
    A = _c(A, np.float64)
    Dskip = _c(Dskip, np.float64)
    h0 = _c(h0, np.float64)
    code = _dtype_code(x)
    for a in (dt, B) + ((C,) if C is not None else ()):
        if a.dtype != x.dtype:
            raise TypeError("x, dt, B, C must share one dtype")
    batch, T, D = x.shape
    N = A.shape[1]
    assert dt.shape == (batch, T, D) and B.shape == (batch, T, N) and A.shape == (D, N)
    if C is not None:
        assert C.shape == (batch, T, N)
    if h0 is not None:
        assert h0.shape == (batch, D, N)
    out = {"hT": np.empty((batch, D, N), np.float64)}
    y = yf = yr = bounds = None
    if want_y:
        y = out["y"] = np.empty((batch, T, D), np.float64)
        if want_parts:
            yf = out["yf"] = np.empty((batch, T, D), np.float64)
            yr = out["yr"] = np.empty((batch, T, D), np.float64)
    if want_bounds:
        bounds = out["bounds"] = np.empty((batch, T // L + 1, D, N), np.float64)
    bias, zz = _fusion(x, D, dt_bias, z)
    rv = _reverse(x, B, A, rev)
    rc = load().oracle_scan_ex(batch, T, D, N, L, code, _ptr(x), _ptr(dt), _ptr(B), _ptr(C),
                               _ptr(A), _ptr(Dskip), _ptr(h0), _ptr(bias), int(bool(dt_softplus)),
                               _ptr(zz), *[_ptr(a) for a in rv], _ptr(y), _ptr(yf), _ptr(yr),
                               _ptr(out["hT"]), _ptr(bounds))
    if rc != 0:
        raise ValueError("oracle_scan rejected its arguments (rc=%d)" % rc)
    return out


def prefill(x, dt, B, C, A, Dskip, L, h_init=None, want_y=False, **fusion):
    """Clean-context prefill -> (h_cache, y or None)."""
    r = scan(x, dt, B, C, A, Dskip, L, h0=h_init, want_y=want_y, **fusion)
    return r["hT"], r.get("y")


def block_step(h_cache, x, dt, B, C, A, Dskip, **fusion):
    """One denoising step on an L-token block (L = x.shape[1]) -> y."""
    L = x.shape[1]
    return scan(x, dt, B, C, A, Dskip, L, h0=h_cache, want_y=True, **fusion)["y"]


def commit(h_cache, x, dt, B, C, A, Dskip, want_y=False, **fusion):
    """Finalise an L-token block -> (new h_cache, y or None)."""
    L = x.shape[1]
    r = scan(x, dt, B, C, A, Dskip, L, h0=h_cache, want_y=want_y, **fusion)
    return r["hT"], r.get("y")


def train_scan(x, dt, B, C, A, Dskip, L, h_init=None, want_bounds=False, **fusion):
    """All-block training form -> (y, h_bounds or None)."""
    r = scan(x, dt, B, C, A, Dskip, L, h0=h_init, want_y=True, want_bounds=want_bounds, **fusion)
    return r["y"], r.get("bounds")


def full_scan(x, dt, B, C, A, Dskip, **fusion):
    """Full-sequence bidirectional baseline (reverse over the whole row) -> y."""
    T = x.shape[1]
    return scan(x, dt, B, C, A, Dskip, max(T, 1), h0=None, want_y=True, **fusion)["y"]


def train_blocks(x, dt, B, C, A, Dskip, L, h0_blocks, dt_bias=None, dt_softplus=False, z=None,
                 rev=None):
    """Two-stream training form, noisy stream: every L-block k scanned from
    h0_blocks[:, k] ([batch, T/L + 1, D, N]) plus the in-block reverse -> y."""
    x, dt, B, C = _c(x), _c(dt), _c(B), _c(C)
    A = _c(A, np.float64)
    Dskip = _c(Dskip, np.float64)
    h0 = _c(h0_blocks, np.float64)
    code = _dtype_code(x)
    batch, T, D = x.shape
    N = A.shape[1]
    assert h0.shape == (batch, T // L + 1, D, N)
    y = np.empty((batch, T, D), np.float64)
    bias, zz = _fusion(x, D, dt_bias, z)
    rv = _reverse(x, B, A, rev)
    rc = load().oracle_train_blocks_ex(batch, T, D, N, L, code, _ptr(x), _ptr(dt), _ptr(B), _ptr(C),
                                       _ptr(A), _ptr(Dskip), _ptr(h0), _ptr(bias),
                                       int(bool(dt_softplus)), _ptr(zz), *[_ptr(a) for a in rv],
                                       _ptr(y))
    if rc != 0:
        raise ValueError("oracle_train_blocks rejected its arguments (rc=%d)" % rc)
    return y


def scan_bwd(x, dt, B, C, A, Dskip, L, dy, h0=None, h0_blocks=None, dbounds=None, dt_bias=None,
             dt_softplus=False, z=None, rev=None):
    """Reverse-mode gradients of the training forms.  Continuous form (the
    gradient of train_scan): forward from h0, optional dbounds = dJ/dh_bounds
    ([batch, T/L+1, D, N]).  Two-stream form (the gradient of train_blocks):
    pass h0_blocks.  dy = dJ/dy [batch, T, D].  Returns a dict of float64
    arrays: dx, ddt [batch, T, D]; dB, dC [batch, T, N]; dA [D, N];
    dDskip [D]; and dh0 [batch, D, N] or dh0_blocks [batch, T/L+1, D, N].
    With the forward's fusions (dt_bias, dt_softplus, z as in scan) ddt is the
    gradient of the dt stream (before bias and softplus), and the dict also
    holds d_dt_bias [D] (when dt_bias is given) and dz [batch, T, D] (when z
    is given).  rev: separate reverse-direction operands {dt, B, C, A[, dt_bias]}
    as in scan; their gradients come back as ddt_rev, dB_rev, dC_rev, dA_rev
    (and d_dt_bias_rev when rev has a dt_bias)."""
    x, dt, B, C = _c(x), _c(dt), _c(B), _c(C)
    A = _c(A, np.float64)
    Dskip = _c(Dskip, np.float64)
    h0 = _c(h0, np.float64)
    h0b = _c(h0_blocks, np.float64)
    dy = _c(dy, np.float64)
    dbounds = _c(dbounds, np.float64)
    code = _dtype_code(x)
    for a in (dt, B, C):
        if a.dtype != x.dtype:
            raise TypeError("x, dt, B, C must share one dtype")
    batch, T, D = x.shape
    N = A.shape[1]
    nb = T // L
    assert dy.shape == (batch, T, D)
    blocks = h0b is not None
    if blocks:
        assert h0b.shape == (batch, nb + 1, D, N)
    if dbounds is not None:
        assert dbounds.shape == (batch, nb + 1, D, N)
    out = {"dx": np.empty((batch, T, D)), "ddt": np.empty((batch, T, D)),
           "dB": np.empty((batch, T, N)), "dC": np.empty((batch, T, N)),
           "dA": np.empty((D, N)), "dDskip": np.empty(D)}
    if blocks:
        out["dh0_blocks"] = np.empty((batch, nb + 1, D, N))
    else:
        out["dh0"] = np.empty((batch, D, N))
    bias, zz = _fusion(x, D, dt_bias, z)
    if bias is not None:
        out["d_dt_bias"] = np.empty(D)
    if zz is not None:
        out["dz"] = np.empty((batch, T, D))
    if rev is not None:
        rv = _reverse(x, B, A, rev)
        out.update(ddt_rev=np.empty((batch, T, D)), dB_rev=np.empty((batch, T, N)),
                   dC_rev=np.empty((batch, T, N)), dA_rev=np.empty((D, N)))
        if rv[4] is not None:
            out["d_dt_bias_rev"] = np.empty(D)
        rc = load().oracle_scan_bwd_sep(
            batch, T, D, N, L, code, _ptr(x), _ptr(dt), _ptr(B), _ptr(C), _ptr(A), _ptr(Dskip),
            int(blocks), _ptr(h0), _ptr(h0b), _ptr(dy), _ptr(dbounds), _ptr(bias),
            int(bool(dt_softplus)), _ptr(zz), _ptr(rv[0]), _ptr(rv[1]), _ptr(rv[2]), _ptr(rv[3]),
            _ptr(rv[4]), _ptr(out["dx"]), _ptr(out["ddt"]), _ptr(out["dB"]), _ptr(out["dC"]),
            _ptr(out["dA"]), _ptr(out["dDskip"]), _ptr(out.get("dh0")), _ptr(out.get("dh0_blocks")),
            _ptr(out.get("dz")), _ptr(out.get("d_dt_bias")), _ptr(out["ddt_rev"]), _ptr(out["dB_rev"]),
            _ptr(out["dC_rev"]), _ptr(out["dA_rev"]), _ptr(out.get("d_dt_bias_rev")))
        if rc != 0:
            raise ValueError("oracle_scan_bwd_sep rejected its arguments (rc=%d)" % rc)
        return out
    rc = load().oracle_scan_bwd_ex(batch, T, D, N, L, code, _ptr(x), _ptr(dt), _ptr(B), _ptr(C),
                                   _ptr(A), _ptr(Dskip), int(blocks), _ptr(h0), _ptr(h0b), _ptr(dy),
                                   _ptr(dbounds), _ptr(bias), int(bool(dt_softplus)), _ptr(zz),
                                   _ptr(out["dx"]), _ptr(out["ddt"]), _ptr(out["dB"]),
                                   _ptr(out["dC"]), _ptr(out["dA"]), _ptr(out["dDskip"]),
                                   _ptr(out.get("dh0")), _ptr(out.get("dh0_blocks")),
                                   _ptr(out.get("dz")), _ptr(out.get("d_dt_bias")))
    if rc != 0:
        raise ValueError("oracle_scan_bwd rejected its arguments (rc=%d)" % rc)
    return out
