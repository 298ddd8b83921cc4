"""Shared helpers of the GPU parity tests: seeded inputs (from the synthetic
input module), marshalling to the oracle, and the error metric.

Error metric (relative per element, with the reference RMS as the floor):
    err = max_i |g_i - r_i| / max(|r_i|, rms(r))
Elements at or above the RMS are judged relative to themselves, smaller ones
relative to the RMS.  The floor is the scale at which fp32 arithmetic works:
a state or output that is a long sum of terms of either sign carries
rounding error proportional to the size of those terms, not to the (possibly
cancelled) result, so a near-zero element can not be held to 1e-4 of itself
by any fp32 implementation.
Bars: 1e-4 for fp32 streams and for the fp32 states, 2e-2 for bf16 outputs.
"""
import numpy as np
import torch

from mamba_selective_scan_04_amd import synth

N = 16
TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}
STATE_TOL = 1e-4


def rel_err(got, ref):
    g = np.asarray(got, np.float64)
    r = np.asarray(ref, np.float64)
    if r.size == 0:
        return 0.0
    rms = np.sqrt(np.mean(r * r))
    den = np.maximum(np.abs(r), rms + 1e-300)
    return float(np.max(np.abs(g - r) / den))


def to_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


class Case:
    """Seeded inputs for one (batch, T, D) problem, on the host and the GPU."""

    def __init__(self, batch, T, D, dtype, sid=7, a_kind="default", k0=0, device="cuda",
                 gen_device="cpu", n=N):
        self.batch, self.T, self.D, self.dtype, self.n = batch, T, D, dtype, n
        x, dt, B, C = synth.stream(batch, T, D, n, sid, k0, dtype, gen_device)
        A, Dskip = synth.params(D, n, sid, a_kind, gen_device)
        self.host = None
        if gen_device == "cpu":
            self.host = dict(x=x, dt=dt, B=B, C=C, A=A, Dskip=Dskip)
        self.dev = {k: v.to(device).contiguous() for k, v in
                    dict(x=x, dt=dt, B=B, C=C, A=A, Dskip=Dskip).items()}

    def args(self):
        d = self.dev
        return d["x"], d["dt"], d["B"], d["C"], d["A"], d["Dskip"]

    def oracle_args(self, t0=0, t1=None, chans=None):
        """Oracle inputs for tokens [t0, t1) and (optionally) a subset of
        channels; read back from the GPU tensors so both sides see the same
        values."""
        t1 = self.T if t1 is None else t1
        d = self.dev
        if chans is None:
            xs, dts = d["x"][:, t0:t1], d["dt"][:, t0:t1]
            A, Ds = d["A"], d["Dskip"]
        else:
            idx = torch.as_tensor(chans, device=d["x"].device)
            xs = d["x"][:, t0:t1].index_select(2, idx)
            dts = d["dt"][:, t0:t1].index_select(2, idx)
            A, Ds = d["A"].index_select(0, idx), d["Dskip"].index_select(0, idx)
        return (synth.to_oracle(xs), synth.to_oracle(dts), synth.to_oracle(d["B"][:, t0:t1]),
                synth.to_oracle(d["C"][:, t0:t1]), synth.to_oracle(A), synth.to_oracle(Ds))

    def segment(self, t0, t1):
        """Tokens [t0, t1) as fresh contiguous copies (at batch 1 the slice is
        already contiguous, and a view would start at an offset that need not
        meet the library's 16-byte base alignment)."""
        d = self.dev
        return tuple(d[k][:, t0:t1].clone(memory_format=torch.contiguous_format) for k in ("x", "dt", "B", "C")) + (
            d["A"], d["Dskip"])


def worst(got, ref):
    """Where rel_err peaks: (index, got, ref, floor) -- printed by failing tests."""
    g = np.asarray(got, np.float64)
    r = np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(r * r))
    den = np.maximum(np.abs(r), rms + 1e-300)
    e = np.abs(g - r) / den
    i = np.unravel_index(int(np.argmax(e)), e.shape)
    return dict(index=tuple(int(v) for v in i), got=float(g[i]), ref=float(r[i]),
                floor=float(rms), err=float(e[i]), normwise=float(np.max(np.abs(g - r)) / np.max(np.abs(r))),
                q13=rel_err_q13(g, r))


def rel_err_q13(got, ref):
    """The same metric with the floor at 0.01 rms(r) (reported beside the
    bars in failure messages; the bars apply to rel_err)."""
    g = np.asarray(got, np.float64)
    r = np.asarray(ref, np.float64)
    if r.size == 0:
        return 0.0
    rms = np.sqrt(np.mean(r * r))
    return float(np.max(np.abs(g - r) / np.maximum(np.abs(r), 0.01 * rms + 1e-300)))


def bf16_within_ulp(got, ref):
    """Fraction of bf16 outputs within one bf16 rounding of the oracle's value:
    |g - bf16(r)| <= |bf16(r)| 2^-7 (bf16(r): the fp64 value rounded to fp32,
    then to bf16 by torch's round-to-nearest-even)."""
    r = torch.from_numpy(np.ascontiguousarray(np.asarray(ref, np.float64))).float().to(torch.bfloat16).float()
    r = r.numpy().astype(np.float64)
    g = np.asarray(got, np.float64)
    if r.size == 0:
        return 1.0
    return float(np.mean(np.abs(g - r) <= np.abs(r) * 2.0 ** -7 + 1e-30))
