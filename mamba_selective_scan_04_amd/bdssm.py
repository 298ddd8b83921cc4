"""ctypes binding of libbdssm.so.  Argument marshalling only.

Names and semantics follow include/bdssm.h:
  prefill(x, dt, B, C, A, Dskip, block_len, h_init=None, h_cache=None, y=None, want_y=False)
  prefill_noalloc(x, dt, B, C, A, Dskip, block_len, h_init=None, h_cache=None, y=None, want_y=False)
  block_step(h_cache, x, dt, B, C, A, Dskip, y=None)
  commit(h_cache, x, dt, B, C, A, Dskip, want_y=False, y=None)
  train_scan(x, dt, B, C, A, Dskip, block_len, h_init=None, want_bounds=False, y=None, h_bounds=None)
  train_scan_blocks(x, dt, B, C, A, Dskip, block_len, h0_blocks, y=None)
  full_scan(x, dt, B, C, A, Dskip, y=None)
  train_scan_bwd(x, dt, B, C, A, Dskip, block_len, h_bounds, dy, d_bounds=None, want_dh_init=False)
  train_scan_blocks_bwd(x, dt, B, C, A, Dskip, block_len, h0_blocks, dy, want_dh0_blocks=False)
  bind_block_step(...), bind_commit(...): the call checked and marshalled once, for
      repeated eager launches (BoundCall)
The six forward functions also take the optional layer features as keyword
arguments: dt_bias ([D] fp32), dt_softplus (bool), z (gate, like y), and rev
(separate reverse-direction operands: dict with dt, B, C, A, optional dt_bias).
Shapes: x, dt, y [batch, T, D]; B, C [batch, T, 16]; A [D, 16] fp32;
Dskip [D] fp32; states [batch, D, 16] fp32.  x/dt/B/C/y share fp32 or bf16.
All tensors must be contiguous, on the current CUDA (HIP) device.  Work is
enqueued on torch's current stream; nothing synchronises.
"""
import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# BDSSM_LIBRARY: load another build of the library (comparisons of builds)
LIB_PATH = os.environ.get("BDSSM_LIBRARY") or os.path.join(HERE, "libbdssm.so")

F32 = 0
BF16 = 1
OP_PREFILL, OP_TRAIN, OP_FULL, OP_TRAIN_BWD, OP_BLOCKS_BWD = 0, 1, 2, 3, 4
OP_TRAIN_BWD_REV, OP_BLOCKS_BWD_REV = 5, 6      # the backward with separate reverse operands
SCRATCH_BYTES = 72 << 20    # BDSSM_SCRATCH_BYTES: the scratch array of bdssm_prefill_noalloc
# the five entry points of the scan, each also in an _ex form that takes the
# fusions (the binding calls the plain form when no fusion is asked for)
PLAIN = ("bdssm_prefill", "bdssm_block_step", "bdssm_commit", "bdssm_train_scan", "bdssm_full_scan")
EXPORTS = PLAIN + tuple(f + "_ex" for f in PLAIN) + (
    "bdssm_prefill_noalloc", "bdssm_train_scan_blocks", "bdssm_train_scan_bwd",
    "bdssm_train_scan_blocks_bwd", "bdssm_workspace_bytes", "bdssm_workspace_bytes_op",
    "bdssm_status_str", "bdssm_version")


class BdssmError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__("%s failed: %s (status %d)" % (fn, msg, status))
        self.status = status


class Shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("d_inner", ctypes.c_int64),
                ("d_state", ctypes.c_int64), ("block_len", ctypes.c_int64),
                ("dtype", ctypes.c_int32)]


class Fusion(ctypes.Structure):
    _fields_ = [("dt_bias", ctypes.c_void_p), ("dt_softplus", ctypes.c_int32),
                ("z", ctypes.c_void_p), ("dt_rev", ctypes.c_void_p), ("B_rev", ctypes.c_void_p),
                ("C_rev", ctypes.c_void_p), ("A_rev", ctypes.c_void_p),
                ("dt_bias_rev", ctypes.c_void_p)]


class FusionGrads(ctypes.Structure):
    _fields_ = [("dz", ctypes.c_void_p), ("d_dt_bias", ctypes.c_void_p), ("ddt_rev", ctypes.c_void_p),
                ("dB_rev", ctypes.c_void_p), ("dC_rev", ctypes.c_void_p), ("dA_rev", ctypes.c_void_p),
                ("d_dt_bias_rev", ctypes.c_void_p)]


_lib = None


def load():
    """Load libbdssm.so (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError("libbdssm.so not built: run `python -m mamba_selective_scan_04_amd.build` "
                          "(or __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, S = ctypes.c_void_p, ctypes.c_int64, ctypes.POINTER(Shape)
    Z = ctypes.c_size_t
    F = ctypes.POINTER(Fusion)
    lib.bdssm_prefill.argtypes = [S, I, P, P, P, P, P, P, P, P, P, P, Z, P]
    lib.bdssm_block_step.argtypes = [S, P, P, P, P, P, P, P, P, P]
    lib.bdssm_commit.argtypes = [S, P, P, P, P, P, P, P, P, P]
    lib.bdssm_train_scan.argtypes = [S, I, P, P, P, P, P, P, P, P, P, P, Z, P]
    lib.bdssm_full_scan.argtypes = [S, I, P, P, P, P, P, P, P, P, Z, P]
    for f in PLAIN:   # the _ex forms: the fusion before the stream
        getattr(lib, f + "_ex").argtypes = getattr(lib, f).argtypes[:-1] + [F, P]
    lib.bdssm_prefill_noalloc.argtypes = [S, I, P, P, P, P, P, P, P, P, P, F, P]
    lib.bdssm_train_scan_blocks.argtypes = [S, I, P, P, P, P, P, P, P, P, F, P]
    G = ctypes.POINTER(FusionGrads)
    lib.bdssm_train_scan_bwd.argtypes = [S, I] + [P] * 17 + [Z, F, G, P]
    lib.bdssm_train_scan_blocks_bwd.argtypes = [S, I] + [P] * 16 + [Z, F, G, P]
    for f in EXPORTS:
        getattr(lib, f).restype = ctypes.c_int
    lib.bdssm_workspace_bytes.argtypes = [S, I]
    lib.bdssm_workspace_bytes.restype = ctypes.c_size_t
    lib.bdssm_workspace_bytes_op.argtypes = [S, I, ctypes.c_int]
    lib.bdssm_workspace_bytes_op.restype = ctypes.c_size_t
    lib.bdssm_status_str.argtypes = [ctypes.c_int]
    lib.bdssm_status_str.restype = ctypes.c_char_p
    _lib = lib
    return lib


def version():
    return load().bdssm_version()


def status_str(status):
    return load().bdssm_status_str(int(status)).decode()


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError("x/dt/B/C must be float32 or bfloat16, got %s" % t.dtype)


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t, name, dtype=None, shape=None):
    # the cheapest torch accessors: this runs for every tensor of every call
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if not t.is_cuda:
        raise ValueError("%s must be on the GPU (got %s)" % (name, t.device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype is not dtype:
        raise TypeError("%s must be %s (got %s)" % (name, dtype, t.dtype))
    if shape is not None and t.shape != shape:
        raise ValueError("%s must have shape %s (got %s)" % (name, tuple(shape), tuple(t.shape)))


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _shape(batch, D, N, L, code):
    return Shape(batch, D, N, L, code)


def _raise(fn, rc):
    if rc != 0:
        raise BdssmError(fn, rc, status_str(rc))


def _form(name, fz, args):
    """(function, its name, full arguments) of one of the five scan entry
    points: the plain form without a fusion, the _ex form with one."""
    if fz is None:
        return getattr(load(), name), name, tuple(args) + (_stream(),)
    return getattr(load(), name + "_ex"), name + "_ex", tuple(args) + (fz, _stream())


def _call(name, fz, *args):
    fn, fname, full = _form(name, fz, args)
    rc = fn(*full)
    _raise(fname, rc)
    return rc


def _streams(x, dt, B, C, A, Dskip, need_c=True):
    if x.dim() != 3:
        raise ValueError("x must be [batch, T, D]")
    batch, T, D = x.shape
    _check(x, "x")
    code = _dtype_code(x)
    _check(dt, "dt", x.dtype, (batch, T, D))
    _check(B, "B", x.dtype)
    if B.dim() != 3 or B.shape[0] != batch or B.shape[1] != T:
        raise ValueError("B must be [batch, T, d_state]")
    N = B.shape[2]
    if need_c or C is not None:
        _check(C, "C", x.dtype, (batch, T, N))
    _check(A, "A", torch.float32, (D, N))
    if Dskip is not None:
        _check(Dskip, "Dskip", torch.float32, (D,))
    return batch, T, D, N, code


def _fusion(x, D, dt_bias=None, dt_softplus=False, z=None, rev=None):
    """Marshal the optional layer features -> ctypes pointer to a Fusion, or
    None.  rev: separate reverse-direction operands, a dict with dt, B, C
    (stream dtype), A ([D, 16] fp32) and optionally dt_bias ([D] fp32)."""
    if dt_bias is None and not dt_softplus and z is None and rev is None:
        return None
    _check(dt_bias, "dt_bias", torch.float32, (D,))
    _check(z, "z", x.dtype, tuple(x.shape))
    ptr = lambda t: None if t is None else t.data_ptr()
    r = {} if rev is None else rev
    if rev is not None:
        batch, T = x.shape[0], x.shape[1]
        _check(r["dt"], "rev['dt']", x.dtype, tuple(x.shape))
        _check(r["B"], "rev['B']", x.dtype)
        _check(r["C"], "rev['C']", x.dtype, tuple(r["B"].shape))
        if r["B"].dim() != 3 or tuple(r["B"].shape[:2]) != (batch, T):
            raise ValueError("rev['B'] must be [batch, T, d_state]")
        _check(r["A"], "rev['A']", torch.float32, (D, r["B"].shape[2]))
        _check(r.get("dt_bias"), "rev['dt_bias']", torch.float32, (D,))
    f = Fusion(ptr(dt_bias), 1 if dt_softplus else 0, ptr(z), ptr(r.get("dt")), ptr(r.get("B")),
               ptr(r.get("C")), ptr(r.get("A")), ptr(r.get("dt_bias")))
    return ctypes.pointer(f)


def workspace_bytes(batch, d_inner, T, op=None, block_len=16, d_state=16, dtype=torch.bfloat16):
    """Workspace bytes of the entry point op (OP_*) at length T; op None: a
    workspace that serves prefill, train_scan and full_scan."""
    s = _shape(batch, d_inner, d_state, block_len, BF16 if dtype == torch.bfloat16 else F32)
    if op is None:
        n = load().bdssm_workspace_bytes(ctypes.byref(s), T)
    else:
        n = load().bdssm_workspace_bytes_op(ctypes.byref(s), T, op)
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("invalid shape for workspace query")
    return n


def _workspace(nbytes, device):
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def prefill(x, dt, B, C, A, Dskip, block_len, h_init=None, h_cache=None, y=None, want_y=False,
            ws=None, **fusion):
    """Build the prefix cache over a clean context -> (h_cache, y or None)."""
    batch, T, D, N, code = _streams(x, dt, B, C, A, Dskip, need_c=want_y or y is not None)
    want_y = want_y or y is not None
    _check(h_init, "h_init", torch.float32, (batch, D, N))
    if h_cache is None:
        h_cache = torch.empty(batch, D, N, dtype=torch.float32, device=x.device)
    _check(h_cache, "h_cache", torch.float32, (batch, D, N))
    if want_y and y is None:
        y = torch.empty_like(x)
    _check(y, "y", x.dtype, (batch, T, D))
    s = _shape(batch, D, N, block_len, code)
    if ws is None:
        ws = _workspace(workspace_bytes(batch, D, T, OP_PREFILL, block_len, N, x.dtype), x.device)
    fz = _fusion(x, D, **fusion)
    _call("bdssm_prefill", fz, ctypes.byref(s), T, _p(x), _p(dt), _p(B), _p(C), _p(A), _p(Dskip),
               _p(h_init), _p(h_cache), _p(y), _p(ws), 0 if ws is None else ws.numel())
    return h_cache, y


def prefill_noalloc(x, dt, B, C, A, Dskip, block_len, h_init=None, h_cache=None, y=None,
                    want_y=False, **fusion):
    """prefill without a workspace argument: the library's own scratch array
    serves as the workspace (calls on one device must not overlap in time).
    Allocates nothing itself when h_cache (and y, if wanted) are passed in.
    -> (h_cache, y or None)."""
    batch, T, D, N, code = _streams(x, dt, B, C, A, Dskip, need_c=want_y or y is not None)
    want_y = want_y or y is not None
    _check(h_init, "h_init", torch.float32, (batch, D, N))
    if h_cache is None:
        h_cache = torch.empty(batch, D, N, dtype=torch.float32, device=x.device)
    _check(h_cache, "h_cache", torch.float32, (batch, D, N))
    if want_y and y is None:
        y = torch.empty_like(x)
    _check(y, "y", x.dtype, (batch, T, D))
    s = _shape(batch, D, N, block_len, code)
    fz = _fusion(x, D, **fusion)
    rc = load().bdssm_prefill_noalloc(ctypes.byref(s), T, _p(x), _p(dt), _p(B), _p(C), _p(A), _p(Dskip),
                                      _p(h_init), _p(h_cache), _p(y), fz, _stream())
    _raise("bdssm_prefill_noalloc", rc)
    return h_cache, y


def block_step(h_cache, x, dt, B, C, A, Dskip, y=None, **fusion):
    """One denoising step on the active block (T == block_len) -> y."""
    batch, T, D, N, code = _streams(x, dt, B, C, A, Dskip)
    _check(h_cache, "h_cache", torch.float32, (batch, D, N))
    if y is None:
        y = torch.empty_like(x)
    _check(y, "y", x.dtype, (batch, T, D))
    s = _shape(batch, D, N, T, code)
    fz = _fusion(x, D, **fusion)
    _call("bdssm_block_step", fz, ctypes.byref(s), _p(h_cache), _p(x), _p(dt), _p(B), _p(C), _p(A),
          _p(Dskip), _p(y))
    return y


def commit(h_cache, x, dt, B, C, A, Dskip, want_y=False, y=None, **fusion):
    """Advance the cache over a finished block, in place -> (h_cache, y or None)."""
    want_y = want_y or y is not None
    batch, T, D, N, code = _streams(x, dt, B, C, A, Dskip, need_c=want_y)
    _check(h_cache, "h_cache", torch.float32, (batch, D, N))
    if want_y and y is None:
        y = torch.empty_like(x)
    _check(y, "y", x.dtype, (batch, T, D))
    s = _shape(batch, D, N, T, code)
    fz = _fusion(x, D, **fusion)
    _call("bdssm_commit", fz, ctypes.byref(s), _p(h_cache), _p(x), _p(dt), _p(B), _p(C), _p(A),
          _p(Dskip), _p(y))
    return h_cache, y


def train_scan(x, dt, B, C, A, Dskip, block_len, h_init=None, want_bounds=False, y=None,
               h_bounds=None, ws=None, **fusion):
    """All-block training form -> (y, h_bounds or None)."""
    batch, T, D, N, code = _streams(x, dt, B, C, A, Dskip)
    _check(h_init, "h_init", torch.float32, (batch, D, N))
    if y is None:
        y = torch.empty_like(x)
    _check(y, "y", x.dtype, (batch, T, D))
    if want_bounds and h_bounds is None:
        h_bounds = torch.empty(batch, T // block_len + 1, D, N, dtype=torch.float32, device=x.device)
    if h_bounds is not None:
        _check(h_bounds, "h_bounds", torch.float32, (batch, T // block_len + 1, D, N))
    s = _shape(batch, D, N, block_len, code)
    if ws is None:
        ws = _workspace(workspace_bytes(batch, D, T, OP_TRAIN, block_len, N, x.dtype), x.device)
    fz = _fusion(x, D, **fusion)
    _call("bdssm_train_scan", fz, ctypes.byref(s), T, _p(x), _p(dt), _p(B), _p(C), _p(A),
          _p(Dskip), _p(h_init), _p(y), _p(h_bounds), _p(ws), 0 if ws is None else ws.numel())
    return y, h_bounds


def train_scan_blocks(x, dt, B, C, A, Dskip, block_len, h0_blocks, y=None, **fusion):
    """Two-stream training form, noisy stream: every block k starts from
    h0_blocks[:, k] ([batch, T/L + 1, D, 16], the h_bounds layout) -> y."""
    batch, T, D, N, code = _streams(x, dt, B, C, A, Dskip)
    _check(h0_blocks, "h0_blocks", torch.float32, (batch, T // block_len + 1, D, N))
    if y is None:
        y = torch.empty_like(x)
    _check(y, "y", x.dtype, (batch, T, D))
    s = _shape(batch, D, N, block_len, code)
    fz = _fusion(x, D, **fusion)
    rc = load().bdssm_train_scan_blocks(ctypes.byref(s), T, _p(x), _p(dt), _p(B), _p(C), _p(A),
                                        _p(Dskip), _p(h0_blocks), _p(y), fz, _stream())
    _raise("bdssm_train_scan_blocks", rc)
    return y


def full_scan(x, dt, B, C, A, Dskip, y=None, ws=None, **fusion):
    """Full-sequence bidirectional baseline (reverse over the whole sequence) -> y."""
    batch, T, D, N, code = _streams(x, dt, B, C, A, Dskip)
    if y is None:
        y = torch.empty_like(x)
    _check(y, "y", x.dtype, (batch, T, D))
    s = _shape(batch, D, N, 1, code)
    if ws is None:
        ws = _workspace(workspace_bytes(batch, D, T, OP_FULL, 1, N, x.dtype), x.device)
    fz = _fusion(x, D, **fusion)
    _call("bdssm_full_scan", fz, ctypes.byref(s), T, _p(x), _p(dt), _p(B), _p(C), _p(A), _p(Dskip),
          _p(y), _p(ws), 0 if ws is None else ws.numel())
    return y


class BoundCall:
    """One library call with its arguments checked and marshalled once.
    Calling the object enqueues the same call again, on the stream that was
    current when it was bound, with the same tensors (which it keeps alive):
    the per-call host cost is the ctypes call and the launch alone.  The
    tensors' contents may change between calls; their storage must not."""
    __slots__ = ("_fn", "_args", "_name", "_keep")

    def __init__(self, fn, name, args, keep):
        self._fn, self._name, self._args, self._keep = fn, name, tuple(args), keep

    def __call__(self):
        rc = self._fn(*self._args)
        if rc != 0:
            _raise(self._name, rc)


def bind_block_step(h_cache, x, dt, B, C, A, Dskip, y, **fusion):
    """block_step(h_cache, x, dt, B, C, A, Dskip, y=y, **fusion) as a BoundCall."""
    batch, T, D, N, code = _streams(x, dt, B, C, A, Dskip)
    _check(h_cache, "h_cache", torch.float32, (batch, D, N))
    _check(y, "y", x.dtype, (batch, T, D))
    s = _shape(batch, D, N, T, code)
    fz = _fusion(x, D, **fusion)
    args = (ctypes.byref(s), _p(h_cache), _p(x), _p(dt), _p(B), _p(C), _p(A), _p(Dskip), _p(y))
    fn, name, args = _form("bdssm_block_step", fz, args)
    return BoundCall(fn, name, args, (s, fz, h_cache, x, dt, B, C, A, Dskip, y, fusion))


def bind_commit(h_cache, x, dt, B, C, A, Dskip, y=None, **fusion):
    """commit(h_cache, x, dt, B, C, A, Dskip, y=y, **fusion) as a BoundCall."""
    batch, T, D, N, code = _streams(x, dt, B, C, A, Dskip, need_c=y is not None)
    _check(h_cache, "h_cache", torch.float32, (batch, D, N))
    _check(y, "y", x.dtype, (batch, T, D))
    s = _shape(batch, D, N, T, code)
    fz = _fusion(x, D, **fusion)
    args = (ctypes.byref(s), _p(h_cache), _p(x), _p(dt), _p(B), _p(C), _p(A), _p(Dskip), _p(y))
    fn, name, args = _form("bdssm_commit", fz, args)
    return BoundCall(fn, name, args, (s, fz, h_cache, x, dt, B, C, A, Dskip, y, fusion))


def _grad_outputs(x, D, N):
    batch, T = x.shape[0], x.shape[1]
    dev = x.device
    return (torch.empty_like(x), torch.empty_like(x),
            torch.empty(batch, T, N, dtype=x.dtype, device=dev),
            torch.empty(batch, T, N, dtype=x.dtype, device=dev),
            torch.empty(D, N, dtype=torch.float32, device=dev),
            torch.empty(D, dtype=torch.float32, device=dev))


def _fusion_grads(x, D, fusion):
    """Outputs of the fused forward's gradients: dz when z is given, d_dt_bias
    when dt_bias is, and with separate reverse operands (rev) ddt_rev, dB_rev,
    dC_rev, dA_rev (and d_dt_bias_rev when rev has a dt_bias)
    -> (ctypes pointer or None, dict of the tensors)."""
    out = {}
    if fusion.get("z") is not None:
        out["dz"] = torch.empty_like(x)
    if fusion.get("dt_bias") is not None:
        out["d_dt_bias"] = torch.empty(D, dtype=torch.float32, device=x.device)
    rev = fusion.get("rev")
    if rev is not None:
        out["ddt_rev"] = torch.empty_like(x)
        out["dB_rev"] = torch.empty_like(rev["B"])
        out["dC_rev"] = torch.empty_like(rev["C"])
        out["dA_rev"] = torch.empty_like(rev["A"])
        if rev.get("dt_bias") is not None:
            out["d_dt_bias_rev"] = torch.empty(D, dtype=torch.float32, device=x.device)
    if not out:
        return None, out
    ptr = lambda t: None if t is None else t.data_ptr()
    g = FusionGrads(*[ptr(out.get(k)) for k in ("dz", "d_dt_bias", "ddt_rev", "dB_rev", "dC_rev",
                                                 "dA_rev", "d_dt_bias_rev")])
    return ctypes.pointer(g), out


def train_scan_bwd(x, dt, B, C, A, Dskip, block_len, h_bounds, dy, d_bounds=None,
                   want_dh_init=False, ws=None, **fusion):
    """Gradients of train_scan given dy (and dJ/dh_bounds) -> dict with dx, ddt,
    dB, dC (stream dtype), dA, dDskip (fp32) and dh_init (fp32 or None).
    h_bounds: the block states train_scan returned for the same inputs.
    fusion: the forward's dt_bias / dt_softplus / z / rev; ddt is then the
    gradient of the raw dt stream, and the dict gains d_dt_bias (fp32 [D], with
    a bias), dz (with a gate) and, with separate reverse operands, ddt_rev,
    dB_rev, dC_rev, dA_rev (and d_dt_bias_rev)."""
    batch, T, D, N, code = _streams(x, dt, B, C, A, Dskip)
    nb = T // block_len + 1
    _check(h_bounds, "h_bounds", torch.float32, (batch, nb, D, N))
    _check(dy, "dy", x.dtype, (batch, T, D))
    _check(d_bounds, "d_bounds", torch.float32, (batch, nb, D, N))
    dx, ddt, dB, dC, dA, dDs = _grad_outputs(x, D, N)
    dh = torch.empty(batch, D, N, dtype=torch.float32, device=x.device) if want_dh_init else None
    s = _shape(batch, D, N, block_len, code)
    if ws is None:
        op = OP_TRAIN_BWD_REV if fusion.get("rev") is not None else OP_TRAIN_BWD
        ws = _workspace(workspace_bytes(batch, D, T, op, block_len, N, x.dtype), x.device)
    fz = _fusion(x, D, **fusion)
    gz, extra = _fusion_grads(x, D, fusion)
    rc = load().bdssm_train_scan_bwd(ctypes.byref(s), T, _p(x), _p(dt), _p(B), _p(C), _p(A),
                                     _p(Dskip), _p(h_bounds), _p(dy), _p(d_bounds), _p(dx),
                                     _p(ddt), _p(dB), _p(dC), _p(dA), _p(dDs), _p(dh), _p(ws),
                                     0 if ws is None else ws.numel(), fz, gz, _stream())
    _raise("bdssm_train_scan_bwd", rc)
    return dict({"dx": dx, "ddt": ddt, "dB": dB, "dC": dC, "dA": dA, "dDskip": dDs, "dh_init": dh},
                **extra)


def train_scan_blocks_bwd(x, dt, B, C, A, Dskip, block_len, h0_blocks, dy, want_dh0_blocks=False,
                          ws=None, **fusion):
    """Gradients of train_scan_blocks -> dict with dx, ddt, dB, dC, dA, dDskip
    and dh0_blocks ([batch, T/L+1, D, 16] fp32, or None); with the fusions as
    in train_scan_bwd, also d_dt_bias and dz."""
    batch, T, D, N, code = _streams(x, dt, B, C, A, Dskip)
    nb = T // block_len + 1
    _check(h0_blocks, "h0_blocks", torch.float32, (batch, nb, D, N))
    _check(dy, "dy", x.dtype, (batch, T, D))
    dx, ddt, dB, dC, dA, dDs = _grad_outputs(x, D, N)
    dh = (torch.empty(batch, nb, D, N, dtype=torch.float32, device=x.device)
          if want_dh0_blocks else None)
    s = _shape(batch, D, N, block_len, code)
    if ws is None:
        op = OP_BLOCKS_BWD_REV if fusion.get("rev") is not None else OP_BLOCKS_BWD
        ws = _workspace(workspace_bytes(batch, D, T, op, block_len, N, x.dtype), x.device)
    fz = _fusion(x, D, **fusion)
    gz, extra = _fusion_grads(x, D, fusion)
    rc = load().bdssm_train_scan_blocks_bwd(ctypes.byref(s), T, _p(x), _p(dt), _p(B), _p(C), _p(A),
                                            _p(Dskip), _p(h0_blocks), _p(dy), _p(dx), _p(ddt),
                                            _p(dB), _p(dC), _p(dA), _p(dDs), _p(dh), _p(ws),
                                            0 if ws is None else ws.numel(), fz, gz, _stream())
    _raise("bdssm_train_scan_blocks_bwd", rc)
    return dict({"dx": dx, "ddt": ddt, "dB": dB, "dC": dC, "dA": dA, "dDskip": dDs,
                 "dh0_blocks": dh}, **extra)
