"""Helpers for the GPU parity tests: host<->device copies and the tolerance rule.

Tolerance (both forms): an element passes iff |g - r| <= rtol * max(|r|, rms(r)),
rms over the compared tensor; rtol = 1e-4 for fp32 I/O and 2e-2 for bf16 I/O
with fp32 state.  The rms floor keeps the rule well-posed where the silu gate
drives outputs to ~0.
"""
from __future__ import annotations

import sys

import numpy as np

from workloads import bf16_bits_to_f32

RTOL = {"f32": 1e-4, "bf16": 2e-2}


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def dev(a):
    import torch
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def host64(t) -> np.ndarray:
    import torch
    if t.dtype == torch.bfloat16:
        return bf16_bits_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    return t.detach().cpu().numpy().astype(np.float64)


def check(got: np.ndarray, ref: np.ndarray, rtol: float, what: str) -> dict:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} vs {ref.shape}"
    assert np.all(np.isfinite(got)), f"{what}: non-finite GPU values"
    if ref.size == 0:
        return {"max_rel": 0.0, "normwise": 0.0}
    rms = float(np.sqrt(np.mean(ref * ref)))
    scale = np.maximum(np.abs(ref), rms)
    err = np.abs(got - ref)
    bad = err > rtol * scale
    rel = float(np.max(err / np.where(scale > 0, scale, 1.0)))
    nw = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    if bad.any():
        i = np.unravel_index(np.argmax(err / np.where(scale > 0, scale, 1.0)), ref.shape)
        raise AssertionError(f"{what}: {int(bad.sum())}/{ref.size} elements out of tolerance {rtol}; "
                             f"worst at {i}: got {got[i]!r} ref {ref[i]!r}; max rel {rel:.3e}, normwise {nw:.3e}")
    return {"max_rel": rel, "normwise": nw}


class StreamCheck:
    """The same rule as check(), applied to a tensor compared block by block (when neither side fits in
    memory at once as fp64).  An element fails iff err > rtol*|r| and err > rtol*rms(r) with rms over the
    whole tensor, so per block it is enough to keep sum(r^2), the element count, and the largest error
    among elements that already exceed rtol*|r|; finish() then compares that with rtol*rms."""

    def __init__(self, rtol: float, what: str):
        self.rtol, self.what = rtol, what
        self.sq, self.n, self.worst, self.where = 0.0, 0, 0.0, None
        self.err2, self.max_rel_abs = 0.0, 0.0

    def add(self, got: np.ndarray, ref: np.ndarray, tag) -> None:
        got = np.asarray(got, np.float64)
        ref = np.asarray(ref, np.float64)
        assert got.shape == ref.shape, f"{self.what} {tag}: shape {got.shape} vs {ref.shape}"
        assert np.all(np.isfinite(got)), f"{self.what} {tag}: non-finite GPU values"
        self.sq += float(np.sum(ref * ref))
        self.n += ref.size
        err = np.abs(got - ref)
        self.err2 += float(np.sum(err * err))
        over = err > self.rtol * np.abs(ref)
        if over.any():
            e = float(err[over].max())
            if e > self.worst:
                self.worst = e
                i = np.unravel_index(np.argmax(np.where(over, err, -1.0)), ref.shape)
                self.where = (tag, i, float(got[i]), float(ref[i]))

    def finish(self) -> dict:
        rms = float(np.sqrt(self.sq / max(self.n, 1)))
        if self.worst > self.rtol * rms:
            raise AssertionError(f"{self.what}: worst error {self.worst!r} above rtol*rms = {self.rtol * rms!r} "
                                 f"(and above rtol*|ref|) at {self.where}")
        return {"rms": rms, "worst_over_rtol_ref": self.worst, "normwise": float(np.sqrt(self.err2 / max(self.sq, 1e-300)))}
