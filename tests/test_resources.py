"""The compiler's resource report of the hot kernels (written by the build
into _build/*.resources.tsv): no register spills, and the waves per SIMD
their design assumes (three for the two-state bidirectional and backward
kernels).  A change that pushes one of them over its register budget shows
here, on the CPU, before any timing."""
import csv
import glob
import os
import re

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
BUILD = os.path.join(os.path.dirname(HERE), "mamba_selective_scan_04_amd", "_build")


def rows():
    out = []
    for path in glob.glob(os.path.join(BUILD, "*.resources.tsv")):
        with open(path) as f:
            out += list(csv.DictReader(f, delimiter="\t"))
    return out


ROWS = rows()
pytestmark = pytest.mark.skipif(not ROWS, reason="no resource report (run the build first)")

BIDIR = re.compile(r"17bidir_pair_kernelI([tf])Li(\d+)ELi(\d+)ELb([01])ELi([01])E")
BWD = re.compile(r"15bwd_pair_kernelI([tf])Li(\d+)ELi(\d+)ELb([01])ELb([01])E")
CHUNK = re.compile(r"18chunk_state_kernelItLb([01])ELb([01])ELi(\d)ELi16E")


def matching(rx, keep):
    got = []
    for r in ROWS:
        m = rx.search(r["kernel"])
        if m and keep(m.groups()):
            got.append((m.groups(), int(r["vgpr_spill"] or 0), int(r["waves"] or 0), int(r["vgprs"] or 0)))
    return got


def test_bidirectional_pair_kernel_fits_three_waves():
    # every state count, blocks of 8 and 16 tokens and the long-block form
    # (L = 0), both stream types, both block-start forms, with and without
    # the fusions
    got = matching(BIDIR, lambda g: g[2] in ("0", "8", "16"))
    assert len(got) == 2 * 4 * 3 * 2 * 2
    bad = [(g, s, w, v) for g, s, w, v in got if s != 0 or w < 3]
    assert not bad, bad


def test_backward_pair_kernel_fits_three_waves():
    # 16 and 32 states at 16-token blocks and the long-block form (16 states)
    want = lambda g: (g[1] in ("16", "32") and g[2] == "16") or (g[1] == "16" and g[2] == "0")
    got = matching(BWD, want)
    assert len(got) == 2 * 3 * 2 * 2
    bad = [(g, s, w, v) for g, s, w, v in got if s != 0 or w < 3]
    assert not bad, bad


def test_prefill_chunk_scan_does_not_spill():
    # the bf16 chunk scan at 16 states with a plain or biased step size, at
    # the seven waves per SIMD it is built for (with the softplus formed
    # inside, a few registers spill at seven waves: not checked)
    got = matching(CHUNK, lambda g: g[2] in ("0", "1"))
    assert len(got) == 3 * 2
    bad = [(g, s, w, v) for g, s, w, v in got if s != 0 or w < 7]
    assert not bad, bad


BOTH = re.compile(r"17chunk_both_kernelI([tf])Li(\d)ELi(\d+)E")
TREE = re.compile(r"17carry_tree_kernelILb([01])E")


def test_baseline_aggregate_pass_does_not_spill():
    # both directions' chunk aggregates in one pass: every stream type, step
    # size form and state count without spills, four waves per SIMD at 16
    # states (five spilled)
    got = matching(BOTH, lambda g: True)
    assert len(got) == 2 * 3 * 4
    bad = [(g, s, w, v) for g, s, w, v in got if s != 0 or (g[2] == "16" and w < 4)]
    assert not bad, bad


def test_segmented_carry_does_not_spill():
    got = matching(TREE, lambda g: True)
    assert len(got) == 2
    assert all(s == 0 for _, s, _, _ in got), got
