"""Host-side checks of the C ABI, no GPU needed: the library loads, exports
every symbol include/bdssm.h declares, sizes workspaces, and rejects bad
arguments before any HIP call (so rejected calls are safe without a device).
"""
import ctypes
import os
import re

import pytest

import mamba_selective_scan_04_amd as m
from mamba_selective_scan_04_amd import bdssm as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    txt = open(os.path.join(ROOT, "include", "bdssm.h")).read()
    return sorted(set(re.findall(r"\b(bdssm_[a-z_]+)\s*\(", txt)))


def test_exports_match_header():
    lib = m.load()
    names = header_functions()
    assert set(names) == set(m.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings():
    assert m.version() == 10700
    for code in range(-7, 1):
        assert m.status_str(code) not in ("", "unknown status")
    assert m.status_str(-99) == "unknown status"


FAKE = 0x10000            # 16-byte aligned, never dereferenced: rejected calls return first
MIS = 0x10002             # misaligned


def shape(batch=1, D=64, N=16, L=16, dtype=B.BF16):
    return B.Shape(batch, D, N, L, dtype)


def lib():
    return m.load()


def P(v):
    return ctypes.c_void_p(v)


def prefill(s, T, x=FAKE, dt=FAKE + 0x1000, Bm=FAKE + 0x2000, C=FAKE + 0x3000, A=FAKE + 0x4000,
            Ds=FAKE + 0x5000, h_init=None, h_cache=FAKE + 0x6000, y=None, ws=None, ws_bytes=0):
    return lib().bdssm_prefill(ctypes.byref(s), T, P(x), P(dt), P(Bm), P(C), P(A), P(Ds),
                               P(h_init), P(h_cache), P(y), P(ws), ws_bytes, None)


def test_shape_errors():
    assert prefill(shape(N=6), 16) == -2           # state counts: 4, 8, 16, 32
    assert prefill(shape(N=64), 16) == -2
    assert prefill(shape(L=0), 16) == -2
    assert prefill(shape(L=-4), 16) == -2
    assert prefill(shape(L=3), 16) == -2         # T % L != 0 for a block length off the wave set
    assert prefill(shape(L=257), 257) == -2      # beyond the LDS-staged block kernel
    assert prefill(shape(), 24) == -2            # T % L != 0
    assert prefill(shape(), -16) == -2
    assert prefill(shape(batch=-1), 16) == -2


def test_dtype_error():
    assert prefill(shape(dtype=7), 16) == -3


def test_null_errors():
    assert lib().bdssm_prefill(None, 16, *([None] * 10), 0, None) == -1
    assert lib().bdssm_prefill_ex(None, 16, *([None] * 10), 0, None, None) == -1
    assert prefill(shape(), 16, x=None) == -1
    assert prefill(shape(), 16, h_cache=None) == -1
    # y requested without C
    assert prefill(shape(), 16, C=None, y=FAKE + 0x7000) == -1


def test_alignment_error():
    assert prefill(shape(), 16, x=MIS) == -4
    assert prefill(shape(), 16, h_cache=MIS) == -4


def test_workspace_error():
    s = shape(batch=1, D=1536)
    need = m.workspace_bytes(1, 1536, 65536, m.OP_PREFILL)
    assert need > 0
    big = 0x100000000
    # no workspace / too small
    assert prefill(s, 65536, x=big, dt=big * 2, Bm=big * 3, C=big * 4, A=big * 5, Ds=big * 6,
                   h_cache=big * 7) == -5
    assert prefill(s, 65536, x=big, dt=big * 2, Bm=big * 3, C=big * 4, A=big * 5, Ds=big * 6,
                   h_cache=big * 7, ws=big * 8, ws_bytes=need - 1) == -5


def test_alias_error():
    # y overlapping x
    assert prefill(shape(), 16, y=FAKE) == -7
    # block step output on top of the cache
    s = shape()
    rc = lib().bdssm_block_step(ctypes.byref(s), P(FAKE), P(FAKE + 0x1000), P(FAKE + 0x2000),
                                P(FAKE + 0x3000), P(FAKE + 0x4000), P(FAKE + 0x5000),
                                P(FAKE + 0x6000), P(FAKE), None)
    assert rc == -7


def test_empty_calls_are_noops():
    # batch 0 / D 0: nothing to do, no pointer needed, no HIP call
    assert prefill(shape(batch=0), 16, x=None, dt=None, Bm=None, C=None, h_cache=None) == 0
    assert prefill(shape(D=0), 16, x=None, dt=None, Bm=None, C=None, h_cache=None) == 0
    s = shape(batch=0)
    assert lib().bdssm_full_scan(ctypes.byref(s), 0, *([None] * 8), 0, None) == 0
    assert lib().bdssm_full_scan_ex(ctypes.byref(s), 0, *([None] * 8), 0, None, None) == 0


def test_workspace_sizes():
    assert m.workspace_bytes(1, 64, 0, m.OP_TRAIN) == 0
    # short sequences need no chunking and therefore no workspace
    assert m.workspace_bytes(1, 64, 16, m.OP_PREFILL) == 0
    # the baseline always needs its fp32 output staging buffer
    assert m.workspace_bytes(1, 64, 16, m.OP_FULL) >= 64 * 16 * 4
    with pytest.raises(ValueError):
        m.workspace_bytes(1, 64, 24, m.OP_TRAIN, block_len=16)
    # other block lengths chunk by whole blocks; short sequences need none
    assert m.workspace_bytes(1, 64, 32, m.OP_TRAIN, block_len=32) == 0
    assert m.workspace_bytes(8, 1536, 4800, m.OP_TRAIN, block_len=48) > 0
    with pytest.raises(ValueError):
        m.workspace_bytes(1, 64, 512, m.OP_TRAIN, block_len=512)
    # other state counts size their chunk states by N
    assert m.workspace_bytes(8, 1536, 4096, m.OP_TRAIN, d_state=32) > m.workspace_bytes(8, 1536, 4096, m.OP_TRAIN, d_state=8)
    with pytest.raises(ValueError):
        m.workspace_bytes(1, 64, 512, m.OP_TRAIN, d_state=6)
    # the backward's general path takes the other state counts and block lengths
    assert m.workspace_bytes(1, 64, 512, m.OP_TRAIN_BWD, d_state=8) > 0
    assert m.workspace_bytes(1, 64, 512, m.OP_TRAIN_BWD, block_len=32) > 0
    assert m.workspace_bytes(2, 64, 512, m.OP_BLOCKS_BWD, block_len=256, d_state=32) > 0
    # separate reverse operands: their own partials on top
    assert m.workspace_bytes(8, 1536, 4096, m.OP_TRAIN_BWD_REV) > m.workspace_bytes(8, 1536, 4096, m.OP_TRAIN_BWD)
    assert m.workspace_bytes(2, 64, 512, m.OP_BLOCKS_BWD_REV, block_len=32) > 0
    with pytest.raises(ValueError):
        m.workspace_bytes(1, 64, 512, 7)
    with pytest.raises(ValueError):
        m.workspace_bytes(1, 64, 512, m.OP_TRAIN_BWD, block_len=512)
    with pytest.raises(ValueError):
        m.workspace_bytes(1, 64, 512, m.OP_BLOCKS_BWD, d_state=6)
    # monotone in T
    a = m.workspace_bytes(8, 1536, 4096, m.OP_TRAIN)
    b = m.workspace_bytes(8, 1536, 8192, m.OP_TRAIN)
    assert 0 < a <= b


def test_timestep_free_prefix_operators():
    """The prefix operator takes no diffusion timestep: prefill and commit
    have no timestep parameter at the ABI."""
    txt = open(os.path.join(ROOT, "include", "bdssm.h")).read()
    for fn in ("bdssm_prefill", "bdssm_commit"):
        decl = txt[txt.index("int " + fn + "("):]
        decl = decl[:decl.index(");")]
        assert "timestep" not in decl and "int64_t t," not in decl


def test_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros(1, 16, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        m.block_step(torch.zeros(1, 64, 16), x, x, torch.zeros(1, 16, 16, dtype=torch.bfloat16),
                     torch.zeros(1, 16, 16, dtype=torch.bfloat16), torch.zeros(64, 16), torch.zeros(64))


def train_bwd(s, T, x=FAKE, dt=FAKE + 0x1000, Bm=FAKE + 0x2000, C=FAKE + 0x3000, A=FAKE + 0x4000,
              Ds=FAKE + 0x5000, hb=FAKE + 0x6000, dy=FAKE + 0x7000, dbnd=None, dx=FAKE + 0x8000,
              ddt=FAKE + 0x9000, dB=FAKE + 0xA000, dC=FAKE + 0xB000, dA=FAKE + 0xC000,
              dD=FAKE + 0xD000, dh=None, ws=None, ws_bytes=0, fusion=None, grads=None):
    return lib().bdssm_train_scan_bwd(ctypes.byref(s), T, P(x), P(dt), P(Bm), P(C), P(A), P(Ds),
                                      P(hb), P(dy), P(dbnd), P(dx), P(ddt), P(dB), P(dC), P(dA),
                                      P(dD), P(dh), P(ws), ws_bytes,
                                      None if fusion is None else ctypes.byref(fusion),
                                      None if grads is None else ctypes.byref(grads), None)


def test_backward_argument_errors():
    s = shape(D=8)
    assert train_bwd(shape(N=6), 16) == -2             # unsupported state count
    assert train_bwd(s, 24) == -2                      # T % L != 0
    assert train_bwd(shape(D=8, L=257), 257) == -2     # blocks above 256 tokens
    # other state counts and block lengths pass the checks (general path) and
    # stop at the missing workspace
    assert train_bwd(shape(D=8, N=8), 16) == -5
    assert train_bwd(shape(D=8, L=32), 32) == -5
    assert train_bwd(shape(D=8, L=3), 12) == -5
    assert train_bwd(s, 16, hb=None) == -1             # saved block states required
    assert train_bwd(s, 16, dy=None) == -1
    assert train_bwd(s, 16, dA=None) == -1
    assert train_bwd(s, 16, dx=MIS) == -4
    assert train_bwd(s, 16, dx=FAKE) == -7             # dx on top of x
    assert train_bwd(s, 16, dB=FAKE + 0x8000) == -7    # two outputs overlap
    assert train_bwd(s, 16, dC=FAKE + 0x7000) == -7    # output on top of dy
    # with a valid argument set the missing workspace is reported
    need = m.workspace_bytes(1, 8, 16, m.OP_TRAIN_BWD)
    assert need > 0
    assert train_bwd(s, 16) == -5
    assert train_bwd(s, 16, ws=FAKE + 0x100000, ws_bytes=need - 1) == -5
    rc = lib().bdssm_train_scan_blocks_bwd(ctypes.byref(s), 16, *[P(FAKE + k * 0x1000) for k in range(6)],
                                           P(None), P(FAKE + 0x7000), *[P(FAKE + k * 0x1000) for k in range(8, 14)],
                                           P(None), P(None), 0, None, None, None)
    assert rc == -1                                    # h0_blocks required


def test_fused_backward_argument_errors():
    s = shape(D=8)
    Fz, G = B.Fusion, B.FusionGrads
    bias, z = FAKE + 0x20000, FAKE + 0x21000
    # separate reverse operands need B_rev, C_rev, A_rev and their gradient outputs
    assert train_bwd(s, 16, fusion=Fz(None, 0, None, FAKE + 0x22000)) == -1
    rv = Fz(None, 0, None, FAKE + 0x22000, FAKE + 0x25000, FAKE + 0x26000, FAKE + 0x27000)
    assert train_bwd(s, 16, fusion=rv) == -1
    assert train_bwd(s, 16, fusion=rv, grads=G(None, None, FAKE + 0x28000, FAKE + 0x29000)) == -1
    full = G(None, None, FAKE + 0x28000, FAKE + 0x29000, FAKE + 0x2A000, FAKE + 0x2B000)
    assert train_bwd(s, 16, fusion=rv, grads=full) == -5                     # reaches the workspace
    assert train_bwd(s, 16, fusion=rv, grads=G(None, None, FAKE + 0x28000, FAKE + 0x29000, FAKE + 0x2A000,
                                               FAKE + 0x25000)) == -7        # dA_rev on top of B_rev
    assert train_bwd(s, 16, fusion=rv, grads=G(None, None, FAKE, FAKE + 0x29000, FAKE + 0x2A000,
                                               FAKE + 0x2B000)) == -7        # ddt_rev on top of x
    assert train_bwd(s, 16, fusion=Fz(None, 0, z)) == -1                      # gate without dz
    assert train_bwd(s, 16, fusion=Fz(None, 0, z), grads=G(None, None)) == -1
    assert train_bwd(s, 16, fusion=Fz(None, 0, z), grads=G(MIS, None)) == -4
    assert train_bwd(s, 16, fusion=Fz(MIS, 1, None)) == -4                    # misaligned bias
    assert train_bwd(s, 16, fusion=Fz(None, 0, z), grads=G(z, None)) == -7    # dz on top of z
    assert train_bwd(s, 16, fusion=Fz(None, 0, z), grads=G(FAKE, None)) == -7  # dz on top of x
    assert train_bwd(s, 16, fusion=Fz(None, 0, z),
                     grads=G(FAKE + 0x8000, None)) == -7                     # dz on top of dx
    assert train_bwd(s, 16, fusion=Fz(bias, 1, None),
                     grads=G(None, FAKE + 0xC000)) == -7                     # d_dt_bias on dA
    assert train_bwd(s, 16, fusion=Fz(bias, 1, None), grads=G(None, bias)) == -7
    assert train_bwd(s, 16, fusion=Fz(None, 0, z), grads=G(FAKE + 0x23000, None),
                     dx=z) == -7                                             # dx on top of z
    # valid fused arguments reach the workspace check
    assert train_bwd(s, 16, fusion=Fz(bias, 1, z), grads=G(FAKE + 0x23000, FAKE + 0x24000)) == -5


def test_backward_workspace_sizes():
    # the dB / dC channel partials dominate: batch * ceil(D/64) * T * 32 fp32
    n = m.workspace_bytes(8, 1536, 4096, m.OP_TRAIN_BWD)
    assert n >= 8 * 24 * 4096 * 32 * 4
    n2 = m.workspace_bytes(8, 1536, 4096, m.OP_BLOCKS_BWD)
    assert 8 * 24 * 4096 * 32 * 4 <= n2 <= n
    assert m.workspace_bytes(1, 64, 0, m.OP_TRAIN_BWD) == 0


@pytest.mark.parametrize("op", ["OP_TRAIN_BWD", "OP_BLOCKS_BWD"])
def test_long_block_backward_workspace(op, monkeypatch):
    """Block lengths that are multiples of 16 above 16 (16 states) add the
    group states [batch, T/16, 2, D, 16] fp32 to the backward's workspace; the
    query reserves them also when BDSSM_BWD_KERNEL=general routes these
    lengths to the general kernel (whose other arrays differ in size: a call
    under another setting than the query's is refused when its workspace is
    too small)."""
    batch, D, T = 2, 256, 1024
    gstate = batch * (T // 16) * 2 * D * 16 * 4
    op = getattr(m, op)
    n32 = m.workspace_bytes(batch, D, T, op, block_len=32)
    assert n32 >= gstate
    monkeypatch.setenv("BDSSM_BWD_KERNEL", "general")
    assert m.workspace_bytes(batch, D, T, op, block_len=32) >= gstate
    assert m.workspace_bytes(batch, D, T, op, block_len=64) >= gstate


def test_fusion_argument_errors():
    f = B.Fusion(MIS, 1, None)                         # misaligned bias
    s = shape()
    rc = lib().bdssm_block_step_ex(ctypes.byref(s), P(FAKE), P(FAKE + 0x1000), P(FAKE + 0x2000),
                                   P(FAKE + 0x3000), P(FAKE + 0x4000), P(FAKE + 0x5000),
                                   P(FAKE + 0x6000), P(FAKE + 0x7000), ctypes.byref(f), None)
    assert rc == -4
    f = B.Fusion(None, 1, FAKE + 0x7000)               # gate on top of y
    rc = lib().bdssm_block_step_ex(ctypes.byref(s), P(FAKE), P(FAKE + 0x1000), P(FAKE + 0x2000),
                                   P(FAKE + 0x3000), P(FAKE + 0x4000), P(FAKE + 0x5000),
                                   P(FAKE + 0x6000), P(FAKE + 0x7000), ctypes.byref(f), None)
    assert rc == -7


def test_single_block_rows_beyond_32bit_offsets():
    """block_step and commit address one block's rows with 32-bit buffer
    offsets: L x d_inner x 4 bytes at or above 2^31 is rejected (here 256 x
    2^21 x 4 = 2^31) before any HIP call.  With one channel fewer the call
    passes that check and stops at the next host check (a NULL cache or
    output), so nothing is ever launched."""
    far = [(k + 1) << 33 for k in range(8)]
    for D, want in ((1 << 21, -2), ((1 << 21) - 1, -1)):
        s = shape(batch=1, D=D, L=256, dtype=B.F32)
        rc = lib().bdssm_block_step(ctypes.byref(s), None, P(far[1]), P(far[2]), P(far[3]), P(far[4]),
                                    P(far[5]), P(far[6]), None, None)
        assert rc == want, (D, rc)
        rc = lib().bdssm_commit(ctypes.byref(s), None, P(far[1]), P(far[2]), P(far[3]), P(far[4]),
                                P(far[5]), P(far[6]), None, None)
        assert rc == want, (D, rc)
