"""CPU oracle for the selective scan (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  The product library never uses it.

``scan_fwd``  -- Mamba-1 selective scan, plain sequential fp64 recurrence
                 (mssm_oracle.c: oracle_scan_fwd).  Pinned by the tests in
                 tests/test_oracle_pins.py: LTI == convolution, delta -> 0 keeps
                 the state, geometric closed form, brute-force unrolled sum,
                 chaining, reset at large delta, linearity/causality, gate and
                 skip special cases.
``ssd_fwd``   -- Mamba-2 scalar-A multi-head form, its own sequential loop
                 (mssm_oracle.c: oracle_ssd_fwd).  Pinned by: equality with the
                 Mamba-1 oracle under head broadcast, the geometric closed form
                 with scalar A, a brute-force unrolled sum, chaining.
``ssd3_fwd``  -- Mamba-3 SISO recurrence (exponential-trapezoidal input rule) in
                 the scalar-A multi-head form, its own sequential loop
                 (mssm_oracle.c: oracle_ssd3_fwd).  Pinned by: equality with
                 ``ssd_fwd`` at lam = 1, second-order convergence to the closed-form
                 solution of the continuous-time system at lam = 1/2 (first order
                 at lam = 1), and a brute-force sum over the implicit width-2
                 convolution weights.
``ssdc_fwd``  -- the same with a complex-valued state: each state pair is a
                 complex number and the head's transition a + i*omega per pair,
                 in C99 complex arithmetic (mssm_oracle.c: oracle_ssdc_fwd).
                 Pinned by: equality with ``ssd3_fwd`` at omega = 0, the
                 rotated-B/C real form (RoPE) as a brute-force sum, the complex
                 geometric closed form, and the previous-token inputs.
``ssdm_fwd``  -- Mamba-3 MIMO: R inputs and R outputs per channel of a head on the
                 head's one state (B and C widened by the rank), with the
                 exponential-trapezoidal rule or, without lam, the Mamba-2 rule
                 (mssm_oracle.c: oracle_ssdm_fwd).  Pinned by: equality with
                 ``ssd3_fwd`` / ``ssd_fwd`` at R = 1, the superposition of R x R
                 SISO runs (one per input rank and output rank), a brute-force
                 unrolled sum, and resuming through the previous token's inputs.
``conv_silu``, ``conv_scan_fwd``
              -- the short causal convolution + SiLU in front of the scan, and
                 the scan on its output (mssm_oracle.c: oracle_conv_silu,
                 oracle_conv_scan_fwd).  Pinned by numpy.convolve, the impulse
                 response, chaining through the initial inputs, and equality
                 with scan_fwd on the convolved x.
``scan_bwd``  -- gradients of ``scan_fwd`` by reverse mode through the same
                 sequential loop, fp64 (mssm_oracle.c: oracle_scan_bwd).  Pinned
                 by central finite differences of ``scan_fwd`` itself
                 (tests/pins.py: pin_scan_bwd_finite_differences).
Both take the already-rounded inputs the GPU receives (bf16 bit patterns are
decoded by the C code's own codec) and return fp64 results.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mssm_oracle.c")
_LIB = os.path.join(_HERE, "libmssm_oracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (IEEE fp64, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-std=c99", "-o", tmp, _SRC, "-lm", "-lpthread"])
        os.replace(tmp, _LIB)
    return _LIB


def load_library(path: Optional[str] = None):
    """Load (and bind) an oracle shared library; the default one is built on demand."""
    lib = ctypes.CDLL(path or build())
    p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.oracle_scan_fwd.restype = i32
    lib.oracle_scan_fwd.argtypes = [i64, i64, i64, i64, i32, p, p, p, p, p, p, p, p, i64, i64, p, p, i32]
    lib.oracle_ssd_fwd.restype = i32
    lib.oracle_ssd_fwd.argtypes = [i64, i64, i64, i64, i64, i64, i32, p, p, p, p, p, p, p, p, i64, i64, p, p, i32]
    lib.oracle_ssd3_fwd.restype = i32
    lib.oracle_ssd3_fwd.argtypes = [i64, i64, i64, i64, i64, i64, i32] + [p] * 9 + [p, p, i32]
    lib.oracle_ssdc_fwd.restype = i32
    lib.oracle_ssdc_fwd.argtypes = [i64, i64, i64, i64, i64, i64, i32] + [p] * 12 + [p, p, i32]
    lib.oracle_ssdm_fwd.restype = i32
    lib.oracle_ssdm_fwd.argtypes = [i64] * 7 + [i32] + [p] * 11 + [p, p, i32]
    lib.oracle_conv_silu.restype = i32
    lib.oracle_conv_silu.argtypes = [i64, i64, i64, i64, i32, p, p, p, p, p]
    lib.oracle_conv_scan_fwd.restype = i32
    lib.oracle_conv_scan_fwd.argtypes = [i64, i64, i64, i64, i64, i32] + [p] * 4 + [p] * 7 + [i64, i64, p, p, i32]
    lib.oracle_scan_bwd.restype = i32
    lib.oracle_scan_bwd.argtypes = [i64, i64, i64, i64, i32] + [p] * 10 + [p] * 8 + [i32]
    return lib


def _get():
    global _lib
    if _lib is None:
        _lib = load_library()
    return _lib


def _io_code(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return 1
    if a.dtype == np.float32:
        return 0
    raise TypeError(f"io arrays must be float32 or uint16 (bf16 bits), got {a.dtype}")


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _c(a: Optional[np.ndarray], dtype=None) -> Optional[np.ndarray]:
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=dtype) if dtype is not None else np.ascontiguousarray(a)


def default_threads() -> int:
    return max(1, len(os.sched_getaffinity(0)))


def scan_fwd(x, delta, A, B, C, D=None, z=None, h0=None, c0: int = 0, c1: Optional[int] = None,
             nthreads: Optional[int] = None, lib=None):
    """Mamba-1 selective scan. x/delta/z [Bsz, L, Dm]; B/C [Bsz, L, N]; A [Dm, N]; D [Dm]; h0 [Bsz, Dm, N].

    Returns (out [Bsz, L, c1-c0] fp64, final_state [Bsz, c1-c0, N] fp64) for channels [c0, c1).
    """
    x, delta, B, C, z = _c(x), _c(delta), _c(B), _c(C), _c(z)
    io = _io_code(x)
    for t in (delta, B, C) + ((z,) if z is not None else ()):
        if _io_code(t) != io:
            raise TypeError("x, delta, B, C, z must share one dtype")
    A, D, h0 = _c(A, np.float32), _c(D, np.float32), _c(h0, np.float32)
    bsz, L, dm = x.shape
    N = A.shape[1]
    c1 = dm if c1 is None else c1
    nc = c1 - c0
    out = np.empty((bsz, L, nc), dtype=np.float64)
    fin = np.empty((bsz, nc, N), dtype=np.float64)
    rc = (lib or _get()).oracle_scan_fwd(bsz, L, dm, N, io, _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C),
                                         _ptr(D), _ptr(z), _ptr(h0), c0, c1, _ptr(out), _ptr(fin),
                                         nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_scan_fwd rejected its arguments")
    return out, fin


def ssd_fwd(x, delta, A, B, C, D=None, z=None, h0=None, hd0: int = 0, hd1: Optional[int] = None,
            nthreads: Optional[int] = None, lib=None):
    """Mamba-2 scalar-A form. x/z [Bsz, L, H, P]; delta [Bsz, L, H]; B/C [Bsz, L, G, N]; A/D [H].

    Returns (out [Bsz, L, hd1-hd0, P] fp64, final_state [Bsz, hd1-hd0, P, N] fp64) for heads [hd0, hd1).
    """
    x, delta, B, C, z = _c(x), _c(delta), _c(B), _c(C), _c(z)
    io = _io_code(x)
    A, D, h0 = _c(A, np.float32), _c(D, np.float32), _c(h0, np.float32)
    bsz, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    hd1 = H if hd1 is None else hd1
    nh = hd1 - hd0
    out = np.empty((bsz, L, nh, P), dtype=np.float64)
    fin = np.empty((bsz, nh, P, N), dtype=np.float64)
    rc = (lib or _get()).oracle_ssd_fwd(bsz, L, H, P, N, G, io, _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C),
                                        _ptr(D), _ptr(z), _ptr(h0), hd0, hd1, _ptr(out), _ptr(fin),
                                        nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_ssd_fwd rejected its arguments")
    return out, fin


def ssd3_fwd(x, delta, lam, A, B, C, D=None, z=None, h0=None, nthreads: Optional[int] = None, lib=None):
    """Mamba-3 SISO recurrence in the scalar-A multi-head form: the exponential-trapezoidal rule
    h_t = a_t h_{t-1} + (1 - lam_t) d_t a_t B_{t-1} x_{t-1} + lam_t d_t B_t x_t, a_t = exp(d_t A).

    Shapes as in ``ssd_fwd``; ``lam`` [Bsz, L, H] in the io dtype.  Returns (out [Bsz, L, H, P] fp64,
    final_state [Bsz, H, P, N] fp64).
    """
    x, delta, lam, B, C, z = _c(x), _c(delta), _c(lam), _c(B), _c(C), _c(z)
    io = _io_code(x)
    for t in (delta, lam, B, C) + ((z,) if z is not None else ()):
        if _io_code(t) != io:
            raise TypeError("x, delta, lam, B, C, z must share one dtype")
    A, D, h0 = _c(A, np.float32), _c(D, np.float32), _c(h0, np.float32)
    bsz, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    out = np.empty((bsz, L, H, P), dtype=np.float64)
    fin = np.empty((bsz, H, P, N), dtype=np.float64)
    rc = (lib or _get()).oracle_ssd3_fwd(bsz, L, H, P, N, G, io, _ptr(x), _ptr(delta), _ptr(lam), _ptr(A),
                                         _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0), _ptr(out), _ptr(fin),
                                         nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_ssd3_fwd rejected its arguments")
    return out, fin


def ssdm_fwd(x, delta, lam, A, B, C, D=None, z=None, h0=None, x_prev=None, B_prev=None,
             nthreads: Optional[int] = None, lib=None):
    """Mamba-3 MIMO: R inputs and R outputs per channel of a head on its one state,
    S_t = a_t S_{t-1} + (1 - lam_t) d_t a_t U_{t-1} + lam_t d_t U_t with U_t = sum_r x[t,h,r,:] (x) B[t,g,r,:],
    y[t,h,r,p] = C[t,g,r,:] . S_t[p,:] (+ D x) (* silu(z)).

    x, z [Bsz, L, H, R, P]; delta, lam [Bsz, L, H] (lam None: lam = 1, the Mamba-2 rule); B, C
    [Bsz, L, G, R, N]; x_prev [Bsz, H, R, P], B_prev [Bsz, G, R, N] (None: no previous token).
    Returns (out [Bsz, L, H, R, P] fp64, final_state [Bsz, H, P, N] fp64)."""
    x, delta, lam, B, C, z = _c(x), _c(delta), _c(lam), _c(B), _c(C), _c(z)
    x_prev, B_prev = _c(x_prev), _c(B_prev)
    io = _io_code(x)
    for t in (delta, B, C) + tuple(v for v in (lam, z, x_prev, B_prev) if v is not None):
        if _io_code(t) != io:
            raise TypeError("x, delta, lam, B, C, z, x_prev, B_prev must share one dtype")
    A, D, h0 = _c(A, np.float32), _c(D, np.float32), _c(h0, np.float32)
    bsz, L, H, R, P = x.shape
    G, N = B.shape[2], B.shape[4]
    if B.shape[3] != R:
        raise ValueError("B must be [Bsz, L, G, R, N] with x's R")
    out = np.empty((bsz, L, H, R, P), dtype=np.float64)
    fin = np.empty((bsz, H, P, N), dtype=np.float64)
    rc = (lib or _get()).oracle_ssdm_fwd(bsz, L, H, P, N, G, R, io, _ptr(x), _ptr(delta), _ptr(lam), _ptr(A),
                                         _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0), _ptr(x_prev),
                                         _ptr(B_prev), _ptr(out), _ptr(fin), nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_ssdm_fwd rejected its arguments")
    return out, fin


def ssdc_fwd(x, delta, lam, A, omega, B, C, D=None, z=None, h0=None, x_prev=None, B_prev=None,
             nthreads: Optional[int] = None, lib=None):
    """Mamba-3 SISO recurrence with a complex-valued state: as ``ssd3_fwd`` with the head's transition
    a + i*omega[h, k] on state pair k (omega [H, N/2] fp32), and the token before step 0 given by
    x_prev [Bsz, H, P] and B_prev [Bsz, G, N] (io dtype; None: no previous token).
    Returns (out [Bsz, L, H, P] fp64, final_state [Bsz, H, P, N] fp64)."""
    x, delta, lam, B, C, z = _c(x), _c(delta), _c(lam), _c(B), _c(C), _c(z)
    x_prev, B_prev = _c(x_prev), _c(B_prev)
    io = _io_code(x)
    for t in (delta, lam, B, C) + tuple(v for v in (z, x_prev, B_prev) if v is not None):
        if _io_code(t) != io:
            raise TypeError("x, delta, lam, B, C, z, x_prev, B_prev must share one dtype")
    A, omega, D, h0 = _c(A, np.float32), _c(omega, np.float32), _c(D, np.float32), _c(h0, np.float32)
    bsz, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    if omega.shape != (H, N // 2):
        raise ValueError("omega must be [H, N/2]")
    out = np.empty((bsz, L, H, P), dtype=np.float64)
    fin = np.empty((bsz, H, P, N), dtype=np.float64)
    rc = (lib or _get()).oracle_ssdc_fwd(bsz, L, H, P, N, G, io, _ptr(x), _ptr(delta), _ptr(lam), _ptr(A),
                                         _ptr(omega), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0), _ptr(x_prev),
                                         _ptr(B_prev), _ptr(out), _ptr(fin), nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_ssdc_fwd rejected its arguments")
    return out, fin


def scan_bwd(x, delta, A, B, C, D=None, z=None, h0=None, dout=None, dfinal=None,
             nthreads: Optional[int] = None, lib=None):
    """Gradients of the Mamba-1 selective scan for the loss sum(out * dout) + sum(final_state * dfinal).

    Shapes as in ``scan_fwd``; ``dout`` [Bsz, L, Dm] in the io dtype, ``dfinal`` [Bsz, Dm, N] fp32 (either
    may be None: zero).  Returns a dict of fp64 arrays: dx, ddelta, dA, dB, dC, dD (None without D),
    dz (None without z), dh0 [Bsz, Dm, N].
    """
    x, delta, B, C, z = _c(x), _c(delta), _c(B), _c(C), _c(z)
    io = _io_code(x)
    for t in (delta, B, C) + ((z,) if z is not None else ()):
        if _io_code(t) != io:
            raise TypeError("x, delta, B, C, z must share one dtype")
    A, D, h0, dfinal = _c(A, np.float32), _c(D, np.float32), _c(h0, np.float32), _c(dfinal, np.float32)
    bsz, L, dm = x.shape
    N = A.shape[1]
    if dout is None:
        dout = np.zeros_like(x)
    dout = _c(dout)
    if _io_code(dout) != io:
        raise TypeError("dout must share the io dtype")
    g = {
        "dx": np.empty((bsz, L, dm)), "ddelta": np.empty((bsz, L, dm)), "dA": np.empty((dm, N)),
        "dB": np.empty((bsz, L, N)), "dC": np.empty((bsz, L, N)),
        "dD": np.empty(dm) if D is not None else None, "dz": np.empty((bsz, L, dm)) if z is not None else None,
        "dh0": np.empty((bsz, dm, N)),
    }
    rc = (lib or _get()).oracle_scan_bwd(
        bsz, L, dm, N, io, _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0),
        _ptr(dout), _ptr(dfinal), _ptr(g["dx"]), _ptr(g["ddelta"]), _ptr(g["dA"]), _ptr(g["dB"]), _ptr(g["dC"]),
        _ptr(g["dD"]), _ptr(g["dz"]), _ptr(g["dh0"]), nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_scan_bwd rejected its arguments")
    return g


def conv_silu(xin, w, bias=None, init=None, lib=None):
    """Short causal convolution + SiLU. xin [Bsz, L, Dm] (io dtype); w [Dm, W] fp32; bias [Dm] fp32;
    init [Bsz, W-1, Dm] (io dtype, the inputs before t = 0). Returns x [Bsz, L, Dm] fp64."""
    xin, init = _c(xin), _c(init)
    io = _io_code(xin)
    if init is not None and _io_code(init) != io:
        raise TypeError("init must share the io dtype")
    w, bias = _c(w, np.float32), _c(bias, np.float32)
    bsz, L, dm = xin.shape
    W = w.shape[1]
    x = np.empty((bsz, L, dm), dtype=np.float64)
    rc = (lib or _get()).oracle_conv_silu(bsz, L, dm, W, io, _ptr(xin), _ptr(w), _ptr(bias), _ptr(init), _ptr(x))
    if rc != 0:
        raise ValueError("oracle_conv_silu rejected its arguments")
    return x


def conv_scan_fwd(xin, w, bias, init, delta, A, B, C, D=None, z=None, h0=None, c0: int = 0,
                  c1: Optional[int] = None, nthreads: Optional[int] = None, lib=None):
    """scan_fwd with x = conv_silu(xin, w, bias, init) (kept in fp64). Returns (out, final_state) fp64."""
    xin, init, delta, B, C, z = _c(xin), _c(init), _c(delta), _c(B), _c(C), _c(z)
    io = _io_code(xin)
    for t in (delta, B, C) + tuple(a for a in (z, init) if a is not None):
        if _io_code(t) != io:
            raise TypeError("xin, delta, B, C, z, init must share one dtype")
    w, bias = _c(w, np.float32), _c(bias, np.float32)
    A, D, h0 = _c(A, np.float32), _c(D, np.float32), _c(h0, np.float32)
    bsz, L, dm = xin.shape
    N, W = A.shape[1], w.shape[1]
    c1 = dm if c1 is None else c1
    nc = c1 - c0
    out = np.empty((bsz, L, nc), dtype=np.float64)
    fin = np.empty((bsz, nc, N), dtype=np.float64)
    rc = (lib or _get()).oracle_conv_scan_fwd(bsz, L, dm, N, W, io, _ptr(xin), _ptr(w), _ptr(bias), _ptr(init),
                                              _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0),
                                              c0, c1, _ptr(out), _ptr(fin), nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_conv_scan_fwd rejected its arguments")
    return out, fin
