"""Pins for the CPU oracle: results the pages and the mathematics fix, computed
without the recurrence (closed forms, convolution, explicit products).

Each pin takes an oracle library handle (``lib``) so the mutation tests can
run the same pins against deliberately broken builds of the oracle.  A pin
raises AssertionError when the oracle disagrees.

Passages (page title, section):
  LTI == convolution   "P20 - Mamba" 5 (fixed A, B, C: a convolution with a
                       long kernel); "Mamba-2 y state-space models" 4.1
                       (parallelisable via a convolution).
  delta -> 0           "03 - Modelos de espacio de estados", "El mecanismo
                       selectivo": a closed gate keeps the state.
  large delta          same section: an open gate lets the state absorb the
                       new input (the old state is forgotten).
  geometric form       scalar A ("Mamba-3" introduction) with constant inputs.
  unrolled sum         "Parallel scan": the recurrence h_t = Abar_t h_{t-1} +
                       Bbar_t x_t unrolled into a sum of products.
  chaining             the fixed-size state is the whole memory
                       ("Mamba-2 y state-space models" 4.3 notes).
  short convolution    the causal convolution in front of the scan ("Mamba-3"
                       blog, "Arquitectura") against numpy.convolve, its impulse
                       response, chaining through the initial inputs, and the
                       scan of its output.
  gradients            the reverse-mode derivative of the scan must equal
                       central finite differences of the (separately pinned)
                       forward oracle, for every input and both outputs.
"""
from __future__ import annotations

import numpy as np

import oracle
from workloads import bf16_bits_to_f32, f32_to_bf16_bits


def _silu(v):
    return v / (1.0 + np.exp(-v))


def _close(got, want, rtol, what):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    scale = max(float(np.max(np.abs(want))) if want.size else 0.0, 1e-300)
    err = float(np.max(np.abs(got - want))) if want.size else 0.0
    assert err <= rtol * scale, f"{what}: max abs err {err:.3e} > {rtol:.1e} * {scale:.3e}"


def _rng(seed):
    return np.random.default_rng(seed)


def _neg_A(rng, d, n):
    # distinct, channel-dependent negative values (so an index mix-up shows)
    return -(rng.uniform(0.2, 2.5, size=(d, n))).astype(np.float32)


# ---------------------------------------------------------------------------
# Mamba-1 pins
# ---------------------------------------------------------------------------
def pin_lti_convolution(lib, seed=1):
    """Constant delta per channel and constant B, C: y = conv(x, K), K_k = sum_n C_n (e^{d A})^k d B_n."""
    rng = _rng(seed)
    bsz, L, d, n = 2, 96, 3, 5
    A = _neg_A(rng, d, n)
    dc = rng.uniform(0.05, 0.6, size=d).astype(np.float32)
    beta = rng.standard_normal(n).astype(np.float32)
    gamma = rng.standard_normal(n).astype(np.float32)
    x = rng.standard_normal((bsz, L, d)).astype(np.float32)
    delta = np.broadcast_to(dc, (bsz, L, d)).copy()
    B = np.broadcast_to(beta, (bsz, L, n)).copy()
    C = np.broadcast_to(gamma, (bsz, L, n)).copy()
    out, _ = oracle.scan_fwd(x, delta, A, B, C, lib=lib)
    k = np.arange(L, dtype=np.float64)[:, None, None]                       # [L, 1, 1]
    dc64, beta64, gamma64 = dc.astype(np.float64), beta.astype(np.float64), gamma.astype(np.float64)
    decay = np.exp(dc64[:, None] * A.astype(np.float64))                   # [d, n]
    K = np.sum(gamma64[None, None, :] * decay[None] ** k * (dc64[:, None] * beta64[None, :])[None], axis=-1)  # [L, d]
    want = np.empty((bsz, L, d))
    for b in range(bsz):
        for c in range(d):
            want[b, :, c] = np.convolve(x[b, :, c].astype(np.float64), K[:, c])[:L]
    _close(out, want, 1e-12, "LTI convolution")


def pin_delta_zero(lib, seed=2):
    """delta == 0: the state is untouched (bitwise) and y_t = C_t . h0 + D x_t, gated."""
    rng = _rng(seed)
    bsz, L, d, n = 2, 33, 4, 3
    A = _neg_A(rng, d, n)
    x = rng.standard_normal((bsz, L, d)).astype(np.float32)
    z = rng.standard_normal((bsz, L, d)).astype(np.float32)
    B = rng.standard_normal((bsz, L, n)).astype(np.float32)
    C = rng.standard_normal((bsz, L, n)).astype(np.float32)
    D = rng.standard_normal(d).astype(np.float32)
    h0 = rng.standard_normal((bsz, d, n)).astype(np.float32)
    delta = np.zeros((bsz, L, d), np.float32)
    out, fin = oracle.scan_fwd(x, delta, A, B, C, D, z, h0, lib=lib)
    assert np.array_equal(fin, h0.astype(np.float64)), "delta=0 must leave the state unchanged"
    y = np.einsum("bln,bdn->bld", C.astype(np.float64), h0.astype(np.float64)) + D.astype(np.float64) * x.astype(np.float64)
    _close(out, y * _silu(z.astype(np.float64)), 1e-13, "delta=0 readout")


def pin_geometric(lib, seed=3):
    """Scalar A, constant delta/x/B/C: h_t = a^{t+1} h0 + d B u (1 - a^{t+1}) / (1 - a)."""
    rng = _rng(seed)
    bsz, L, d, n = 1, 57, 3, 4
    alpha, dl, u = np.float32(-0.7), np.float32(0.3), np.float32(1.3)
    A = np.full((d, n), alpha, np.float32)
    beta = rng.standard_normal(n).astype(np.float32)
    gamma = rng.standard_normal(n).astype(np.float32)
    D = rng.standard_normal(d).astype(np.float32)
    z = rng.standard_normal((bsz, L, d)).astype(np.float32)
    h0 = rng.standard_normal((bsz, d, n)).astype(np.float32)
    x = np.full((bsz, L, d), u, np.float32)
    delta = np.full((bsz, L, d), dl, np.float32)
    B = np.broadcast_to(beta, (bsz, L, n)).copy()
    C = np.broadcast_to(gamma, (bsz, L, n)).copy()
    out, fin = oracle.scan_fwd(x, delta, A, B, C, D, z, h0, lib=lib)
    a = np.exp(np.float64(dl) * np.float64(alpha))
    p = a ** np.arange(1, L + 1, dtype=np.float64)                           # a^{t+1}
    h = p[None, :, None, None] * h0[:, None].astype(np.float64) + \
        (np.float64(dl) * beta.astype(np.float64) * np.float64(u))[None, None, None, :] * \
        ((1 - p) / (1 - a))[None, :, None, None]                              # [b, L, d, n]
    y = np.einsum("bldn,n->bld", h, gamma.astype(np.float64)) + D.astype(np.float64) * np.float64(u)
    _close(out, y * _silu(z.astype(np.float64)), 1e-12, "geometric closed form")
    _close(fin, h[:, -1], 1e-12, "geometric final state")


def bruteforce_scan(x, delta, A, B, C, D=None, z=None, h0=None):
    """y_t = sum_n C_t[n] (prod_{r<=t} e^{d_r A}) h0[n] + sum_{s<=t} sum_n C_t[n] (prod_{s<r<=t} e^{d_r A}) d_s B_s[n] x_s."""
    x, delta, A, B, C = (np.asarray(v, np.float64) for v in (x, delta, A, B, C))
    bsz, L, d = x.shape
    n = A.shape[1]
    out = np.zeros((bsz, L, d))
    for b in range(bsz):
        for c in range(d):
            for t in range(L):
                tot = 0.0
                for m in range(n):
                    if h0 is not None:
                        prod = 1.0
                        for r in range(0, t + 1):
                            prod *= np.exp(delta[b, r, c] * A[c, m])
                        tot += C[b, t, m] * prod * float(h0[b, c, m])
                    for s in range(t + 1):
                        prod = 1.0
                        for r in range(s + 1, t + 1):
                            prod *= np.exp(delta[b, r, c] * A[c, m])
                        tot += C[b, t, m] * prod * delta[b, s, c] * B[b, s, m] * x[b, s, c]
                if D is not None:
                    tot += float(D[c]) * x[b, t, c]
                if z is not None:
                    tot *= _silu(float(z[b, t, c]))
                out[b, t, c] = tot
    return out


def pin_bruteforce(lib, seed=4):
    rng = _rng(seed)
    bsz, L, d, n = 2, 24, 3, 4
    A = _neg_A(rng, d, n)
    x = rng.standard_normal((bsz, L, d)).astype(np.float32)
    delta = rng.uniform(0.01, 0.8, size=(bsz, L, d)).astype(np.float32)
    B = rng.standard_normal((bsz, L, n)).astype(np.float32)
    C = rng.standard_normal((bsz, L, n)).astype(np.float32)
    D = rng.standard_normal(d).astype(np.float32)
    z = rng.standard_normal((bsz, L, d)).astype(np.float32)
    h0 = rng.standard_normal((bsz, d, n)).astype(np.float32)
    out, _ = oracle.scan_fwd(x, delta, A, B, C, D, z, h0, lib=lib)
    _close(out, bruteforce_scan(x, delta, A, B, C, D, z, h0), 1e-12, "brute-force unrolled sum")


def pin_chaining(lib, seed=5):
    """scan(x)[L1:] == scan(x[L1:], h0 = final(scan(x[:L1]))), and the finals agree."""
    rng = _rng(seed)
    bsz, L, d, n, L1 = 2, 70, 3, 4, 29
    A = _neg_A(rng, d, n)
    x = rng.standard_normal((bsz, L, d)).astype(np.float32)
    delta = rng.uniform(0.01, 0.5, size=(bsz, L, d)).astype(np.float32)
    B = rng.standard_normal((bsz, L, n)).astype(np.float32)
    C = rng.standard_normal((bsz, L, n)).astype(np.float32)
    D = rng.standard_normal(d).astype(np.float32)
    z = rng.standard_normal((bsz, L, d)).astype(np.float32)
    full, fin = oracle.scan_fwd(x, delta, A, B, C, D, z, lib=lib)
    _, mid = oracle.scan_fwd(x[:, :L1], delta[:, :L1], A, B[:, :L1], C[:, :L1], D, z[:, :L1], lib=lib)
    # the state is handed over in fp32 (the carrier type); compare with a matching tolerance
    tail, fin2 = oracle.scan_fwd(x[:, L1:], delta[:, L1:], A, B[:, L1:], C[:, L1:], D, z[:, L1:],
                                 mid.astype(np.float32), lib=lib)
    _close(tail, full[:, L1:], 1e-6, "chaining output")
    _close(fin2, fin, 1e-6, "chaining final state")


def pin_reset(lib, seed=6):
    """delta = 200, A <= -1: the old state is wiped (e^{-200}), h_t = d B_t x_t."""
    rng = _rng(seed)
    bsz, L, d, n = 1, 20, 3, 4
    A = -(1.0 + rng.uniform(0, 3, size=(d, n))).astype(np.float32)
    x = rng.standard_normal((bsz, L, d)).astype(np.float32)
    delta = np.full((bsz, L, d), 200.0, np.float32)
    B = rng.standard_normal((bsz, L, n)).astype(np.float32)
    C = rng.standard_normal((bsz, L, n)).astype(np.float32)
    D = rng.standard_normal(d).astype(np.float32)
    h0 = rng.standard_normal((bsz, d, n)).astype(np.float32)
    out, _ = oracle.scan_fwd(x, delta, A, B, C, D, None, h0, lib=lib)
    cb = np.sum(C.astype(np.float64) * B.astype(np.float64), axis=-1)        # [b, L]
    want = 200.0 * x.astype(np.float64) * cb[:, :, None] + D.astype(np.float64) * x.astype(np.float64)
    _close(out, want, 1e-13, "reset at large delta")


def pin_linearity_causality(lib, seed=7):
    rng = _rng(seed)
    bsz, L, d, n = 2, 40, 3, 4
    A = _neg_A(rng, d, n)
    x1 = rng.standard_normal((bsz, L, d)).astype(np.float32)
    x2 = rng.standard_normal((bsz, L, d)).astype(np.float32)
    delta = rng.uniform(0.01, 0.5, size=(bsz, L, d)).astype(np.float32)
    B = rng.standard_normal((bsz, L, n)).astype(np.float32)
    C = rng.standard_normal((bsz, L, n)).astype(np.float32)
    D = rng.standard_normal(d).astype(np.float32)
    a, b = 0.75, -1.5
    y1, _ = oracle.scan_fwd(x1, delta, A, B, C, D, lib=lib)
    y2, _ = oracle.scan_fwd(x2, delta, A, B, C, D, lib=lib)
    x12 = (a * x1.astype(np.float64) + b * x2.astype(np.float64))
    # inputs are fp32: a*x1 + b*x2 is computed exactly in fp64 and passed through fp32 -> small rounding
    y12, _ = oracle.scan_fwd(x12.astype(np.float32), delta, A, B, C, D, lib=lib)
    _close(y12, a * y1 + b * y2, 1e-6, "linearity in x")
    t0 = 17
    xp = x1.copy()
    xp[:, t0] += np.float32(3.0)
    yp, _ = oracle.scan_fwd(xp, delta, A, B, C, D, lib=lib)
    assert np.array_equal(yp[:, :t0], y1[:, :t0]), "outputs before t0 must not depend on x[t0]"
    assert not np.array_equal(yp[:, t0], y1[:, t0]), "output at t0 must depend on x[t0]"


def pin_gate_skip(lib, seed=8):
    rng = _rng(seed)
    bsz, L, d, n = 2, 30, 3, 4
    A = _neg_A(rng, d, n)
    x = rng.standard_normal((bsz, L, d)).astype(np.float32)
    delta = rng.uniform(0.01, 0.5, size=(bsz, L, d)).astype(np.float32)
    B = rng.standard_normal((bsz, L, n)).astype(np.float32)
    C = rng.standard_normal((bsz, L, n)).astype(np.float32)
    D = rng.standard_normal(d).astype(np.float32)
    z = rng.standard_normal((bsz, L, d)).astype(np.float32)
    out, _ = oracle.scan_fwd(x, delta, A, B, C, D, np.zeros_like(z), lib=lib)
    assert np.all(out == 0.0), "z == 0 gates the output to exactly 0"
    want = D.astype(np.float64) * x.astype(np.float64) * _silu(z.astype(np.float64))
    out, _ = oracle.scan_fwd(x, delta, A, B, np.zeros_like(C), D, z, lib=lib)
    _close(out, want, 1e-14, "C == 0 leaves D x silu(z)")
    out, _ = oracle.scan_fwd(x, delta, A, np.zeros_like(B), C, D, z, lib=lib)
    _close(out, want, 1e-14, "B == 0, h0 == 0 leaves D x silu(z)")
    out_noD, _ = oracle.scan_fwd(x, delta, A, B, C, None, None, lib=lib)
    out_D, _ = oracle.scan_fwd(x, delta, A, B, C, D, None, lib=lib)
    _close(out_D - out_noD, D.astype(np.float64) * x.astype(np.float64), 1e-12, "skip term D x")


def pin_bf16_codec(lib, seed=9):
    """bf16 inputs are read exactly: oracle(bf16 bits) == oracle(same values as fp32)."""
    rng = _rng(seed)
    bsz, L, d, n = 2, 25, 3, 4
    A = _neg_A(rng, d, n)
    mk = lambda *s: f32_to_bf16_bits(rng.standard_normal(s).astype(np.float32))
    x, z = mk(bsz, L, d), mk(bsz, L, d)
    delta = f32_to_bf16_bits(rng.uniform(0.01, 0.5, size=(bsz, L, d)).astype(np.float32))
    B, C = mk(bsz, L, n), mk(bsz, L, n)
    D = rng.standard_normal(d).astype(np.float32)
    ob, fb = oracle.scan_fwd(x, delta, A, B, C, D, z, lib=lib)
    f = bf16_bits_to_f32
    of, ff = oracle.scan_fwd(f(x), f(delta), A, f(B), f(C), D, f(z), lib=lib)
    assert np.array_equal(ob, of) and np.array_equal(fb, ff), "bf16 decode must be exact"


# ---------------------------------------------------------------------------
# Mamba-2 (scalar A per head) pins
# ---------------------------------------------------------------------------
def _ssd_case(rng, bsz=2, L=37, H=4, P=3, N=5, G=2, with_dz=True, with_h0=True):
    x = rng.standard_normal((bsz, L, H, P)).astype(np.float32)
    delta = rng.uniform(0.01, 0.6, size=(bsz, L, H)).astype(np.float32)
    A = -(rng.uniform(0.3, 3.0, size=H)).astype(np.float32)
    B = rng.standard_normal((bsz, L, G, N)).astype(np.float32)
    C = rng.standard_normal((bsz, L, G, N)).astype(np.float32)
    D = rng.standard_normal(H).astype(np.float32) if with_dz else None
    z = rng.standard_normal((bsz, L, H, P)).astype(np.float32) if with_dz else None
    h0 = rng.standard_normal((bsz, H, P, N)).astype(np.float32) if with_h0 else None
    return x, delta, A, B, C, D, z, h0


def pin_ssd_equals_broadcast_scan(lib, seed=11):
    """The scalar-A head form is the diagonal scan with A and delta broadcast over the head's P channels."""
    rng = _rng(seed)
    x, delta, A, B, C, D, z, h0 = _ssd_case(rng)
    bsz, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    out, fin = oracle.ssd_fwd(x, delta, A, B, C, D, z, h0, lib=lib)
    hpg = H // G
    for g in range(G):
        hs = slice(g * hpg, (g + 1) * hpg)
        xe = x[:, :, hs, :].reshape(bsz, L, hpg * P)
        de = np.repeat(delta[:, :, hs], P, axis=2)
        Ae = np.repeat(np.repeat(A[hs], P)[:, None], N, axis=1)
        De = np.repeat(D[hs], P)
        ze = z[:, :, hs, :].reshape(bsz, L, hpg * P)
        h0e = h0[:, hs].reshape(bsz, hpg * P, N)
        ye, fe = oracle.scan_fwd(xe, de, Ae, B[:, :, g], C[:, :, g], De, ze, h0e, lib=lib)
        _close(out[:, :, hs, :].reshape(bsz, L, hpg * P), ye, 1e-13, f"SSD == broadcast scan (group {g})")
        _close(fin[:, hs].reshape(bsz, hpg * P, N), fe, 1e-13, f"SSD final == broadcast scan (group {g})")


def pin_ssd_geometric(lib, seed=12):
    rng = _rng(seed)
    bsz, L, H, P, N, G = 1, 45, 2, 3, 4, 1
    dl, u = np.float32(0.25), np.float32(-0.8)
    A = np.array([-0.5, -1.7], np.float32)
    beta = rng.standard_normal(N).astype(np.float32)
    gamma = rng.standard_normal(N).astype(np.float32)
    x = np.full((bsz, L, H, P), u, np.float32)
    delta = np.full((bsz, L, H), dl, np.float32)
    B = np.broadcast_to(beta, (bsz, L, G, N)).copy()
    C = np.broadcast_to(gamma, (bsz, L, G, N)).copy()
    h0 = rng.standard_normal((bsz, H, P, N)).astype(np.float32)
    out, fin = oracle.ssd_fwd(x, delta, A, B, C, None, None, h0, lib=lib)
    for h in range(H):
        a = np.exp(np.float64(dl) * np.float64(A[h]))
        p = a ** np.arange(1, L + 1, dtype=np.float64)
        hs = p[:, None, None] * h0[0, h][None].astype(np.float64) + \
            (np.float64(dl) * np.float64(u) * beta.astype(np.float64))[None, None, :] * ((1 - p) / (1 - a))[:, None, None]
        y = np.einsum("lpn,n->lp", hs, gamma.astype(np.float64))
        _close(out[0, :, h, :], y, 1e-12, "SSD geometric closed form")
        _close(fin[0, h], hs[-1], 1e-12, "SSD geometric final")


def pin_ssd_bruteforce(lib, seed=13):
    rng = _rng(seed)
    x, delta, A, B, C, D, z, h0 = _ssd_case(rng, bsz=1, L=16, H=2, P=2, N=3, G=1)
    out, _ = oracle.ssd_fwd(x, delta, A, B, C, D, z, h0, lib=lib)
    x64, d64, B64, C64 = (v.astype(np.float64) for v in (x, delta, B, C))
    bsz, L, H, P = x.shape
    want = np.zeros_like(out)
    for h in range(H):
        ell = d64[0, :, h] * np.float64(A[h])                     # log-decay per step
        for t in range(L):
            for p in range(P):
                tot = np.float64(0.0)
                for s in range(-1, t + 1):
                    w = np.exp(np.sum(ell[s + 1:t + 1]))          # decay from after s up to t
                    if s < 0:
                        tot += w * np.dot(C64[0, t, 0], h0[0, h, p].astype(np.float64))
                    else:
                        tot += w * np.dot(C64[0, t, 0], B64[0, s, 0]) * d64[0, s, h] * x64[0, s, h, p]
                tot += np.float64(D[h]) * x64[0, t, h, p]
                tot *= _silu(np.float64(z[0, t, h, p]))
                want[0, t, h, p] = tot
    _close(out, want, 1e-11, "SSD brute-force unrolled sum")


def pin_ssd_chaining(lib, seed=14):
    rng = _rng(seed)
    x, delta, A, B, C, D, z, _ = _ssd_case(rng, L=50, with_h0=False)
    L1 = 21
    full, fin = oracle.ssd_fwd(x, delta, A, B, C, D, z, lib=lib)
    _, mid = oracle.ssd_fwd(x[:, :L1], delta[:, :L1], A, B[:, :L1], C[:, :L1], D, z[:, :L1], lib=lib)
    tail, fin2 = oracle.ssd_fwd(x[:, L1:], delta[:, L1:], A, B[:, L1:], C[:, L1:], D, z[:, L1:],
                                mid.astype(np.float32), lib=lib)
    _close(tail, full[:, L1:], 1e-6, "SSD chaining output")
    _close(fin2, fin, 1e-6, "SSD chaining final")


# ---------------------------------------------------------------------------
# Mamba-3 SISO recurrence: exponential-trapezoidal input rule
# ---------------------------------------------------------------------------
def _ssd3_case(rng, bsz=2, L=37, H=4, P=3, N=5, G=2, with_dz=True, with_h0=True):
    x, delta, A, B, C, D, z, h0 = _ssd_case(rng, bsz, L, H, P, N, G, with_dz, with_h0)
    lam = rng.uniform(0.0, 1.0, (bsz, L, H)).astype(np.float32)
    return x, delta, lam, A, B, C, D, z, h0


def pin_ssd3_lam_one_is_ssd(lib, seed=15):
    """lam = 1 puts the whole step weight on the right end: the Mamba-2 rule delta * B_t * x_t."""
    rng = _rng(seed)
    x, delta, lam, A, B, C, D, z, h0 = _ssd3_case(rng)
    ones = np.ones_like(lam)
    out, fin = oracle.ssd3_fwd(x, delta, ones, A, B, C, D, z, h0, lib=lib)
    ref, ref_fin = oracle.ssd_fwd(x, delta, A, B, C, D, z, h0, lib=lib)
    _close(out, ref, 1e-13, "lam = 1 output vs Mamba-2 form")
    _close(fin, ref_fin, 1e-13, "lam = 1 final state vs Mamba-2 form")


def pin_ssd3_trapezoid_order(lib, seed=16):
    """The scheme is a quadrature of h' = a h + u(t) over each step.  Against the closed-form solution
    for u = sin(w t), h(0) = 0:  h(T) = (w e^{aT} - a sin wT - w cos wT) / (a^2 + w^2), halving the step
    must cut the worst error about 4x at lam = 1/2 (second order) and about 2x at lam = 1 (first order).
    Step 0 has delta = 0 (no time passes: it only records u(0)); steps k >= 1 span ((k-1)h, kh]."""
    a, w, T = -0.75, 2.0, 4.0
    errs = {}
    for lam_v in (0.5, 1.0):
        for K in (128, 256):
            hstep = T / K                                    # 1/32, 1/64: exact in fp32
            tk = np.arange(K + 1) * hstep
            x = np.sin(w * tk).astype(np.float32).reshape(1, K + 1, 1, 1)
            delta = np.full((1, K + 1, 1), hstep, np.float32)
            delta[0, 0, 0] = 0.0
            lam = np.full((1, K + 1, 1), lam_v, np.float32)
            one = np.ones((1, K + 1, 1, 1), np.float32)
            out, _ = oracle.ssd3_fwd(x, delta, lam, np.array([a], np.float32), one, one, lib=lib)
            xs = x[0, :, 0, 0].astype(np.float64)            # the fp32-rounded input the scheme saw
            exact = (w * np.exp(a * tk) - a * np.sin(w * tk) - w * np.cos(w * tk)) / (a * a + w * w)
            # the rounding of the input samples moves the result by far less than the quadrature error
            assert np.max(np.abs(xs - np.sin(w * tk))) < 1e-7
            errs[(lam_v, K)] = np.max(np.abs(out[0, :, 0, 0] - exact))
    r_trap = errs[(0.5, 128)] / errs[(0.5, 256)]
    r_right = errs[(1.0, 128)] / errs[(1.0, 256)]
    assert 3.6 < r_trap < 4.4, f"trapezoidal rule not second order: error ratio {r_trap:.3f} ({errs})"
    assert 1.8 < r_right < 2.2, f"right-end rule not first order: error ratio {r_right:.3f} ({errs})"
    assert errs[(0.5, 256)] < 1e-4, errs


def pin_ssd3_bruteforce(lib, seed=17):
    """Unrolled, x_s reaches the output at t through two weights that share one decay:
    y_t = sum_{s<=t} (C_t . B_s) exp(sum_{r=s+1..t} d_r A) w(t, s) x_s + exp(sum_{r<=t} d_r A) C_t . h0,
    w(t, s) = lam_s d_s + [s < t] (1 - lam_{s+1}) d_{s+1}  (a width-2 convolution on the state input)."""
    rng = _rng(seed)
    x, delta, lam, A, B, C, D, z, h0 = _ssd3_case(rng, bsz=2, L=14, H=3, P=2, N=3, G=1)
    out, fin = oracle.ssd3_fwd(x, delta, lam, A, B, C, D, z, h0, nthreads=1, lib=lib)
    x64, d64, l64, B64, C64 = (v.astype(np.float64) for v in (x, delta, lam, B, C))
    bsz, L, H, P = x.shape
    want = np.zeros_like(out)
    want_fin = np.zeros_like(fin)
    for b in range(bsz):
        for h in range(H):
            ell = d64[b, :, h] * np.float64(A[h])
            for t in range(L):
                for p in range(P):
                    tot = np.exp(np.sum(ell[:t + 1])) * np.dot(C64[b, t, 0], h0[b, h, p].astype(np.float64))
                    for s in range(t + 1):
                        wts = l64[b, s, h] * d64[b, s, h]
                        if s < t:
                            wts += (1.0 - l64[b, s + 1, h]) * d64[b, s + 1, h]
                        tot += np.exp(np.sum(ell[s + 1:t + 1])) * np.dot(C64[b, t, 0], B64[b, s, 0]) * wts * \
                            x64[b, s, h, p]
                    tot += np.float64(D[h]) * x64[b, t, h, p]
                    want[b, t, h, p] = tot * _silu(np.float64(z[b, t, h, p]))
            for p in range(P):
                st = np.exp(np.sum(ell)) * h0[b, h, p].astype(np.float64)
                for s in range(L):
                    wts = l64[b, s, h] * d64[b, s, h]
                    if s < L - 1:
                        wts += (1.0 - l64[b, s + 1, h]) * d64[b, s + 1, h]
                    st = st + np.exp(np.sum(ell[s + 1:])) * wts * x64[b, s, h, p] * B64[b, s, 0]
                want_fin[b, h, p] = st
    _close(out, want, 1e-11, "Mamba-3 brute-force unrolled sum")
    _close(fin, want_fin, 1e-11, "Mamba-3 brute-force final state")


def ssd3_resume_state(fin, delta, lam, B, x, L1, H, G):
    """The state to resume a Mamba-3 sequence at step L1 from the state after step L1-1: that state plus
    the left-end term of step L1, (1 - lam_{L1}) delta_{L1} x_{L1-1} (x) B_{L1-1} (fp64)."""
    hpg = H // G
    d = delta[:, L1].astype(np.float64)                                   # [b, H]
    w = (1.0 - lam[:, L1].astype(np.float64)) * d                         # [b, H]
    xp = x[:, L1 - 1].astype(np.float64)                                  # [b, H, P]
    Bp = B[:, L1 - 1].astype(np.float64)[:, np.arange(H) // hpg]          # [b, H, N]
    return fin + w[:, :, None, None] * xp[:, :, :, None] * Bp[:, :, None, :]


def pin_ssd3_resume(lib, seed=18):
    """Splitting a sequence at L1 and resuming from the first part's final state plus the boundary's
    left-end term reproduces the whole run (the header's stated way to continue a sequence)."""
    rng = _rng(seed)
    x, delta, lam, A, B, C, D, z, h0 = _ssd3_case(rng, L=45)
    L1 = 17
    H, G = x.shape[2], B.shape[2]
    full, fin = oracle.ssd3_fwd(x, delta, lam, A, B, C, D, z, h0, lib=lib)
    _, mid = oracle.ssd3_fwd(x[:, :L1], delta[:, :L1], lam[:, :L1], A, B[:, :L1], C[:, :L1], D, z[:, :L1], h0,
                             lib=lib)
    h1 = ssd3_resume_state(mid, delta, lam, B, x, L1, H, G)
    tail, fin2 = oracle.ssd3_fwd(x[:, L1:], delta[:, L1:], lam[:, L1:], A, B[:, L1:], C[:, L1:], D, z[:, L1:],
                                 h1.astype(np.float32), lib=lib)
    _close(tail, full[:, L1:], 1e-6, "Mamba-3 resumed output")
    _close(fin2, fin, 1e-6, "Mamba-3 resumed final state")


# ---------------------------------------------------------------------------
# Mamba-3 SISO recurrence with a complex-valued state (rotations per state pair)
# ---------------------------------------------------------------------------
def _ssdc_case(rng, bsz=2, L=23, H=3, P=2, N=6, G=1):
    x, delta, lam, A, B, C, D, z, h0 = _ssd3_case(rng, bsz, L, H, P, N, G)
    omega = rng.uniform(-3.0, 3.0, (H, N // 2)).astype(np.float32)
    return x, delta, lam, A, omega, B, C, D, z, h0


def _rot(u, v, phi):
    """Rotate the pairs (u, v) by the angles phi (real arithmetic)."""
    c, s = np.cos(phi), np.sin(phi)
    return u * c - v * s, u * s + v * c


def pin_ssdc_omega_zero_is_ssd3(lib, seed=41):
    """No rotation (omega = 0) leaves the real exponential-trapezoidal recurrence."""
    rng = _rng(seed)
    x, delta, lam, A, omega, B, C, D, z, h0 = _ssdc_case(rng)
    out, fin = oracle.ssdc_fwd(x, delta, lam, A, np.zeros_like(omega), B, C, D, z, h0, lib=lib)
    ref, ref_fin = oracle.ssd3_fwd(x, delta, lam, A, B, C, D, z, h0, lib=lib)
    _close(out, ref, 1e-13, "omega = 0 output vs real Mamba-3 form")
    _close(fin, ref_fin, 1e-13, "omega = 0 final state vs real Mamba-3 form")


def pin_ssdc_rope_bruteforce(lib, seed=42):
    """In the frame rotated back by Theta_t = sum_{r<=t} delta_r omega, the state follows the real
    recurrence with B and C rotated by -Theta_t (RoPE on B and C).  Built here with explicit cos/sin
    rotations and the unrolled trapezoidal weights, then the final state is rotated forward again."""
    rng = _rng(seed)
    x, delta, lam, A, omega, B, C, D, z, h0 = _ssdc_case(rng)
    out, fin = oracle.ssdc_fwd(x, delta, lam, A, omega, B, C, D, z, h0, nthreads=1, lib=lib)
    x64, d64, l64, B64, C64 = (v.astype(np.float64) for v in (x, delta, lam, B, C))
    om, h064 = omega.astype(np.float64), h0.astype(np.float64)
    bsz, L, H, P = x.shape
    N = B.shape[3]
    want, want_fin = np.zeros_like(out), np.zeros_like(fin)
    for b in range(bsz):
        for h in range(H):
            theta = np.cumsum(d64[b, :, h])[:, None] * om[h][None, :]                 # [L, N/2]
            Br = np.empty((L, N)); Cr = np.empty((L, N))
            Br[:, 0::2], Br[:, 1::2] = _rot(B64[b, :, 0, 0::2], B64[b, :, 0, 1::2], -theta)
            Cr[:, 0::2], Cr[:, 1::2] = _rot(C64[b, :, 0, 0::2], C64[b, :, 0, 1::2], -theta)
            ell = d64[b, :, h] * np.float64(A[h])
            wt = l64[b, :, h] * d64[b, :, h]
            wo = wt.copy()
            wo[:-1] += (1.0 - l64[b, 1:, h]) * d64[b, 1:, h]
            for p in range(P):
                for t in range(L):
                    tot = np.exp(np.sum(ell[:t + 1])) * np.dot(Cr[t], h064[b, h, p])
                    for s in range(t + 1):
                        w = wt[s] if s == t else wo[s]
                        tot += np.exp(np.sum(ell[s + 1:t + 1])) * np.dot(Cr[t], Br[s]) * w * x64[b, s, h, p]
                    tot += np.float64(D[h]) * x64[b, t, h, p]
                    want[b, t, h, p] = tot * _silu(np.float64(z[b, t, h, p]))
                g = np.exp(np.sum(ell)) * h064[b, h, p]
                for s in range(L):
                    w = wt[s] if s == L - 1 else wo[s]    # the last step has no later step to reach
                    g = g + np.exp(np.sum(ell[s + 1:])) * w * x64[b, s, h, p] * Br[s]
                want_fin[b, h, p, 0::2], want_fin[b, h, p, 1::2] = _rot(g[0::2], g[1::2], theta[-1])
    _close(out, want, 1e-11, "complex state: rotated-frame (RoPE) brute force")
    _close(fin, want_fin, 1e-11, "complex state: rotated-frame final state")


def pin_ssdc_geometric(lib, seed=43):
    """Constant inputs, one state pair, no previous token: with r = exp(d (a + i w)),
    h_0 = lam d b x and h_t = r h_{t-1} + ((1 - lam) r + lam) d b x, so
    h_t = r^t h_0 + c (1 - r^t) / (1 - r); y_t = Re(conj(c_C) h_t)."""
    L, d, lam, a, w, xv = 40, 0.25, 0.375, -0.5, 1.25, 0.75
    bc, cc = (0.5, -1.0), (1.5, 0.25)
    x = np.full((1, L, 1, 1), xv, np.float32)
    delta = np.full((1, L, 1), d, np.float32)
    lm = np.full((1, L, 1), lam, np.float32)
    B = np.tile(np.array(bc, np.float32), (1, L, 1, 1))
    C = np.tile(np.array(cc, np.float32), (1, L, 1, 1))
    out, fin = oracle.ssdc_fwd(x, delta, lm, np.array([a], np.float32), np.array([[w]], np.float32), B, C,
                               lib=lib)
    r = np.exp(d * (a + 1j * w))
    bx = (bc[0] + 1j * bc[1]) * xv
    h0 = lam * d * bx
    c = ((1.0 - lam) * r + lam) * d * bx
    t = np.arange(L)
    h = r ** t * h0 + c * (1.0 - r ** t) / (1.0 - r)
    y = np.real(np.conj(cc[0] + 1j * cc[1]) * h)
    _close(out[0, :, 0, 0], y, 1e-12, "complex state: geometric closed form")
    _close(fin[0, 0, 0], np.array([h[-1].real, h[-1].imag]), 1e-12, "complex state: final pair")


def pin_ssdc_previous_token(lib, seed=44):
    """Giving the token before step 0 (x_prev, B_prev) equals adding its left-end term,
    (1 - lam_0) d_0 x_prev B_prev (per complex pair), to h0."""
    rng = _rng(seed)
    x, delta, lam, A, omega, B, C, D, z, h0 = _ssdc_case(rng, G=1)
    bsz, L, H, P = x.shape
    N = B.shape[3]
    xp = rng.standard_normal((bsz, H, P)).astype(np.float32)
    bp = rng.standard_normal((bsz, 1, N)).astype(np.float32)
    out, fin = oracle.ssdc_fwd(x, delta, lam, A, omega, B, C, D, z, h0, xp, bp, lib=lib)
    w = (1.0 - lam[:, 0].astype(np.float64)) * delta[:, 0].astype(np.float64)     # [b, H]
    h1 = h0 + w[:, :, None, None] * xp.astype(np.float64)[:, :, :, None] * bp.astype(np.float64)[:, :, None, :]
    ref, ref_fin = oracle.ssdc_fwd(x, delta, lam, A, omega, B, C, D, z, h1.astype(np.float32), lib=lib)
    _close(out, ref, 1e-6, "complex state: previous token output")
    _close(fin, ref_fin, 1e-6, "complex state: previous token final state")


# ---------------------------------------------------------------------------
# Gradients of the Mamba-1 scan
# ---------------------------------------------------------------------------
def _fd_case(rng, bsz=2, L=9, d=3, n=4):
    x = rng.standard_normal((bsz, L, d)).astype(np.float32)
    delta = rng.uniform(0.05, 0.9, size=(bsz, L, d)).astype(np.float32)
    A = _neg_A(rng, d, n)
    B = rng.standard_normal((bsz, L, n)).astype(np.float32)
    C = rng.standard_normal((bsz, L, n)).astype(np.float32)
    D = rng.standard_normal(d).astype(np.float32)
    z = rng.standard_normal((bsz, L, d)).astype(np.float32)
    h0 = rng.standard_normal((bsz, d, n)).astype(np.float32)
    return dict(x=x, delta=delta, A=A, B=B, C=C, D=D, z=z, h0=h0)


def pin_scan_bwd_finite_differences(lib, seed=21):
    """d/dv [sum(out * R) + sum(final * Rf)] by central differences of scan_fwd, for every element v of
    every input, against scan_bwd.  The step is a power of two; the difference quotient divides by the
    step the fp32 inputs actually took, so input rounding does not enter."""
    rng = _rng(seed)
    for with_dz, with_h0, with_fin in ((True, True, True), (False, False, True), (True, True, False)):
        inp = _fd_case(rng)
        if not with_dz:
            inp["D"] = None
            inp["z"] = None
        if not with_h0:
            inp["h0"] = None
        R = rng.standard_normal(inp["x"].shape).astype(np.float32)
        Rf = rng.standard_normal((inp["x"].shape[0], inp["x"].shape[2], inp["A"].shape[1])).astype(np.float32)
        if not with_fin:
            Rf = np.zeros_like(Rf)

        def loss(**kw):
            out, fin = oracle.scan_fwd(**kw, lib=lib, nthreads=1)
            return float(np.sum(out * R.astype(np.float64)) + np.sum(fin * Rf.astype(np.float64)))

        g = oracle.scan_bwd(**inp, dout=R, dfinal=Rf if with_fin else None, lib=lib, nthreads=2)
        names = [k for k in ("x", "delta", "A", "B", "C", "D", "z", "h0") if inp[k] is not None]
        for k in names:
            base = inp[k]
            fd = np.zeros(base.shape)
            for idx in np.ndindex(base.shape):
                step = np.float32(2.0 ** -12) * max(np.float32(1.0), np.abs(base[idx]))
                vals = []
                for sgn in (1, -1):
                    pert = dict(inp)
                    arr = base.copy()
                    arr[idx] = base[idx] + np.float32(sgn) * step
                    pert[k] = arr
                    vals.append((loss(**pert), float(arr[idx])))
                fd[idx] = (vals[0][0] - vals[1][0]) / (vals[0][1] - vals[1][1])
            got = g["d" + k]
            _close(got, fd, 2e-6, f"scan gradient d{k} (D/z {with_dz}, h0 {with_h0}, final {with_fin})")
        if not with_dz:
            assert g["dD"] is None and g["dz"] is None


def pin_scan_bwd_linear_in_upstream(lib, seed=22):
    """The gradients are linear in (dout, dfinal), and a zero upstream gradient gives zero gradients."""
    rng = _rng(seed)
    inp = _fd_case(rng, bsz=3, L=17, d=2, n=5)
    shp_f = (3, 2, 5)
    R1, R2 = rng.standard_normal(inp["x"].shape).astype(np.float32), rng.standard_normal(inp["x"].shape).astype(np.float32)
    F1, F2 = rng.standard_normal(shp_f).astype(np.float32), rng.standard_normal(shp_f).astype(np.float32)
    g1 = oracle.scan_bwd(**inp, dout=R1, dfinal=F1, lib=lib)
    g2 = oracle.scan_bwd(**inp, dout=R2, dfinal=F2, lib=lib)
    g12 = oracle.scan_bwd(**inp, dout=R1 + R2, dfinal=F1 + F2, lib=lib)
    for k in g1:
        _close(g12[k], g1[k] + g2[k], 1e-6, f"gradient linearity d{k[1:]}")
    g0 = oracle.scan_bwd(**inp, lib=lib)
    for k, v in g0.items():
        assert np.all(v == 0), f"zero upstream gradient gave nonzero {k}"


# ---------------------------------------------------------------------------
# Short causal convolution + SiLU in front of the scan
# ---------------------------------------------------------------------------
def _conv_case(rng, bsz=2, L=23, d=5, W=4):
    xin = rng.standard_normal((bsz, L, d)).astype(np.float32)
    w = rng.standard_normal((d, W)).astype(np.float32)
    bias = rng.standard_normal(d).astype(np.float32)
    init = rng.standard_normal((bsz, W - 1, d)).astype(np.float32)
    return xin, w, bias, init


def pin_conv_numpy(lib, seed=31):
    """Every channel's pre-activation equals numpy.convolve of the padded input with the flipped taps."""
    rng = _rng(seed)
    for W in (1, 2, 3, 4):
        xin, w, bias, init = _conv_case(rng, W=W)
        for use_init in (False, True):
            x = oracle.conv_silu(xin, w, bias, init if use_init and W > 1 else None, lib=lib)
            bsz, L, d = xin.shape
            want = np.empty_like(x)
            for b in range(bsz):
                for c in range(d):
                    pre = (init[b, :, c] if use_init and W > 1 else np.zeros(W - 1, np.float32)).astype(np.float64)
                    seq = np.concatenate([pre, xin[b, :, c].astype(np.float64)])
                    full = np.convolve(seq, w[c, ::-1].astype(np.float64), mode="valid")   # length L
                    want[b, :, c] = _silu(full + np.float64(bias[c]))
            _close(x, want, 1e-13, f"conv W={W} init={use_init}")


def pin_conv_impulse(lib, seed=32):
    """A unit impulse at t0 gives silu(bias + w[c, W-1-(t-t0)]) for t0 <= t < t0+W and silu(bias) elsewhere."""
    rng = _rng(seed)
    _, w, bias, _ = _conv_case(rng, d=3, W=4)
    L, t0 = 12, 5
    xin = np.zeros((1, L, 3), np.float32)
    xin[0, t0, :] = 1.0
    x = oracle.conv_silu(xin, w, bias, lib=lib)
    want = np.empty((1, L, 3))
    for t in range(L):
        for c in range(3):
            k = t - t0
            want[0, t, c] = _silu(np.float64(bias[c]) + (np.float64(w[c, 3 - k]) if 0 <= k < 4 else 0.0))
    _close(x, want, 1e-14, "conv impulse response")


def pin_conv_chaining(lib, seed=33):
    """Convolving [L1, L) with init = the W-1 inputs before L1 gives the tail of the whole convolution."""
    rng = _rng(seed)
    xin, w, bias, init = _conv_case(rng, L=30, W=4)
    L1 = 11
    full = oracle.conv_silu(xin, w, bias, init, lib=lib)
    tail = oracle.conv_silu(xin[:, L1:], w, bias, np.ascontiguousarray(xin[:, L1 - 3:L1]), lib=lib)
    _close(tail, full[:, L1:], 1e-15, "conv chaining through the initial inputs")


def pin_conv_scan_composition(lib, seed=34):
    """conv_scan_fwd equals scan_fwd run on the convolved x (rounded to fp32, hence the tolerance), and the
    skip term uses the convolved x, not the raw input."""
    rng = _rng(seed)
    xin, w, bias, init = _conv_case(rng, bsz=2, L=37, d=4, W=3)
    n = 6
    delta = rng.uniform(0.05, 0.8, size=xin.shape).astype(np.float32)
    A = _neg_A(rng, 4, n)
    B = rng.standard_normal((2, 37, n)).astype(np.float32)
    C = rng.standard_normal((2, 37, n)).astype(np.float32)
    D = rng.standard_normal(4).astype(np.float32)
    z = rng.standard_normal(xin.shape).astype(np.float32)
    h0 = rng.standard_normal((2, 4, n)).astype(np.float32)
    out, fin = oracle.conv_scan_fwd(xin, w, bias, init, delta, A, B, C, D, z, h0, lib=lib)
    x32 = oracle.conv_silu(xin, w, bias, init, lib=lib).astype(np.float32)
    ref, ref_fin = oracle.scan_fwd(x32, delta, A, B, C, D, z, h0, lib=lib)
    _close(out, ref, 1e-6, "conv + scan == scan(conv)")
    _close(fin, ref_fin, 1e-6, "conv + scan final state")


SCAN_PINS = [pin_lti_convolution, pin_delta_zero, pin_geometric, pin_bruteforce, pin_chaining, pin_reset,
             pin_linearity_causality, pin_gate_skip, pin_bf16_codec]
SSD_PINS = [pin_ssd_equals_broadcast_scan, pin_ssd_geometric, pin_ssd_bruteforce, pin_ssd_chaining]
# ---------------------------------------------------------------------------
# Mamba-3 MIMO: R inputs and R outputs per channel on the head's one state
# ---------------------------------------------------------------------------
def _ssdm_case(rng, bsz=2, L=23, H=4, P=3, N=5, G=2, R=3, with_dz=True, with_h0=True, with_lam=True):
    x = rng.standard_normal((bsz, L, H, R, P)).astype(np.float32)
    delta = rng.uniform(0.01, 0.6, size=(bsz, L, H)).astype(np.float32)
    lam = rng.uniform(0.0, 1.0, (bsz, L, H)).astype(np.float32) if with_lam else None
    A = -(rng.uniform(0.3, 3.0, size=H)).astype(np.float32)
    B = rng.standard_normal((bsz, L, G, R, N)).astype(np.float32)
    C = rng.standard_normal((bsz, L, G, R, N)).astype(np.float32)
    D = rng.standard_normal(H).astype(np.float32) if with_dz else None
    z = rng.standard_normal((bsz, L, H, R, P)).astype(np.float32) if with_dz else None
    h0 = rng.standard_normal((bsz, H, P, N)).astype(np.float32) if with_h0 else None
    return x, delta, lam, A, B, C, D, z, h0


def pin_ssdm_rank_one_is_siso(lib, seed=51):
    """One input and one output per channel is the SISO recurrence: the exponential-trapezoidal rule with
    lam, the Mamba-2 rule without it."""
    rng = _rng(seed)
    x, delta, lam, A, B, C, D, z, h0 = _ssdm_case(rng, R=1)
    sq = lambda a: None if a is None else np.ascontiguousarray(a[:, :, :, 0])
    out, fin = oracle.ssdm_fwd(x, delta, lam, A, B, C, D, z, h0, lib=lib)
    ref, ref_fin = oracle.ssd3_fwd(sq(x), delta, lam, A, sq(B), sq(C), D, sq(z), h0, lib=lib)
    _close(out[:, :, :, 0], ref, 1e-13, "MIMO R = 1 output vs the SISO rule")
    _close(fin, ref_fin, 1e-13, "MIMO R = 1 final state vs the SISO rule")
    out, fin = oracle.ssdm_fwd(x, delta, None, A, B, C, D, z, h0, lib=lib)
    ref, ref_fin = oracle.ssd_fwd(sq(x), delta, A, sq(B), sq(C), D, sq(z), h0, lib=lib)
    _close(out[:, :, :, 0], ref, 1e-13, "MIMO R = 1 without lam vs the Mamba-2 form")
    _close(fin, ref_fin, 1e-13, "MIMO R = 1 without lam final state vs the Mamba-2 form")


def pin_ssdm_superposition(lib, seed=52):
    """The state is linear in the inputs, so it is the sum of R SISO states, one driven by each input rank
    (x_r', B_r'), and output r reads that sum through C_r: y_r = sum_r' SISO(x_r', B_r', C_r) + D x_r.
    R x R runs of the (separately pinned) SISO oracle, h0 carried by one of them."""
    rng = _rng(seed)
    x, delta, lam, A, B, C, D, z, h0 = _ssdm_case(rng, R=3, with_dz=False)
    D = rng.standard_normal(x.shape[2]).astype(np.float32)
    out, fin = oracle.ssdm_fwd(x, delta, lam, A, B, C, D, None, h0, lib=lib)
    R = x.shape[3]
    rk = lambda a, r: np.ascontiguousarray(a[:, :, :, r])
    want = np.zeros_like(out)
    want_fin = np.zeros_like(fin)
    for r_in in range(R):
        hh = h0 if r_in == 0 else None
        for r_out in range(R):
            o, f = oracle.ssd3_fwd(rk(x, r_in), delta, lam, A, rk(B, r_in), rk(C, r_out), None, None, hh, lib=lib)
            want[:, :, :, r_out] += o
        want_fin += f
    want += np.float64(1.0) * D.astype(np.float64)[None, None, :, None, None] * x.astype(np.float64)
    _close(out, want, 1e-12, "MIMO output vs the sum of SISO runs")
    _close(fin, want_fin, 1e-12, "MIMO final state vs the sum of SISO runs")


def pin_ssdm_bruteforce(lib, seed=53):
    """Unrolled: with U_s = sum_r x[s,r] (x) B[s,r] and the SISO weights
    w(t, s) = lam_s d_s + [s < t] (1 - lam_{s+1}) d_{s+1},
    y[t,r,p] = (C[t,r] . (exp(sum_{u<=t} d_u A) h0[p] + sum_{s<=t} exp(sum_{u=s+1..t} d_u A) w(t,s) U_s[p]) + D x) silu(z)."""
    rng = _rng(seed)
    x, delta, lam, A, B, C, D, z, h0 = _ssdm_case(rng, bsz=1, L=9, H=2, P=2, N=3, G=1, R=2)
    out, fin = oracle.ssdm_fwd(x, delta, lam, A, B, C, D, z, h0, nthreads=1, lib=lib)
    x64, d64, l64, B64, C64, z64 = (v.astype(np.float64) for v in (x, delta, lam, B, C, z))
    bsz, L, H, R, P = x.shape
    want = np.zeros_like(out)
    want_fin = np.zeros_like(fin)
    for b in range(bsz):
        for h in range(H):
            ell = d64[b, :, h] * np.float64(A[h])
            U = np.einsum("srp,srn->spn", x64[b, :, h], B64[b, :, 0])           # [L, P, N]
            for t in range(L + 1):
                st = np.exp(np.sum(ell[:t])) * h0[b, h].astype(np.float64)      # state after step t-1
                for s in range(t):
                    w = l64[b, s, h] * d64[b, s, h]
                    if s < t - 1:
                        w += (1.0 - l64[b, s + 1, h]) * d64[b, s + 1, h]
                    st = st + np.exp(np.sum(ell[s + 1:t])) * w * U[s]
                if t == L:
                    want_fin[b, h] = st
                    break
                # the output at step t reads the state after step t
                st_t = np.exp(np.sum(ell[:t + 1])) * h0[b, h].astype(np.float64)
                for s in range(t + 1):
                    w = l64[b, s, h] * d64[b, s, h]
                    if s < t:
                        w += (1.0 - l64[b, s + 1, h]) * d64[b, s + 1, h]
                    st_t = st_t + np.exp(np.sum(ell[s + 1:t + 1])) * w * U[s]
                for r in range(R):
                    for p in range(P):
                        y = np.dot(C64[b, t, 0, r], st_t[p]) + np.float64(D[h]) * x64[b, t, h, r, p]
                        want[b, t, h, r, p] = y * _silu(z64[b, t, h, r, p])
    _close(out, want, 1e-11, "MIMO brute-force unrolled sum")
    _close(fin, want_fin, 1e-11, "MIMO brute-force final state")


def pin_ssdm_resume(lib, seed=54):
    """Splitting at L1 and resuming from the first part's final state, with the token before the second part
    given as the previous token (x_prev, B_prev), reproduces the whole run; and a previous token is the same
    as adding its left-end term (1 - lam_0) d_0 sum_r x_prev[r] (x) B_prev[r] to h0."""
    rng = _rng(seed)
    x, delta, lam, A, B, C, D, z, h0 = _ssdm_case(rng, L=31)
    L1 = 12
    full, fin = oracle.ssdm_fwd(x, delta, lam, A, B, C, D, z, h0, lib=lib)
    _, mid = oracle.ssdm_fwd(x[:, :L1], delta[:, :L1], lam[:, :L1], A, B[:, :L1], C[:, :L1], D, z[:, :L1], h0,
                             lib=lib)
    tail, fin2 = oracle.ssdm_fwd(x[:, L1:], delta[:, L1:], lam[:, L1:], A, B[:, L1:], C[:, L1:], D, z[:, L1:],
                                 mid.astype(np.float32), x[:, L1 - 1], B[:, L1 - 1], lib=lib)
    _close(tail, full[:, L1:], 1e-6, "MIMO resumed output")
    _close(fin2, fin, 1e-6, "MIMO resumed final state")
    xp = rng.standard_normal(x[:, 0].shape).astype(np.float32)                # [b, H, R, P]
    bp = rng.standard_normal(B[:, 0].shape).astype(np.float32)                # [b, G, R, N]
    o1, f1 = oracle.ssdm_fwd(x, delta, lam, A, B, C, D, z, h0, xp, bp, lib=lib)
    H, G = x.shape[2], B.shape[2]
    bph = bp.astype(np.float64)[:, np.arange(H) // (H // G)]                   # [b, H, R, N]
    left = ((1.0 - lam[:, 0].astype(np.float64)) * delta[:, 0].astype(np.float64))[:, :, None, None] * \
        np.einsum("bhrp,bhrn->bhpn", xp.astype(np.float64), bph)
    h0p = (h0.astype(np.float64) + left).astype(np.float32)                  # the fp32 h0 the oracle takes
    o2, f2 = oracle.ssdm_fwd(x, delta, lam, A, B, C, D, z, h0p, lib=lib)
    _close(o1, o2, 1e-6, "MIMO previous token vs its left-end term added to h0 (output)")
    _close(f1, f2, 1e-6, "MIMO previous token vs its left-end term added to h0 (final state)")


SSD3_PINS = [pin_ssd3_lam_one_is_ssd, pin_ssd3_trapezoid_order, pin_ssd3_bruteforce, pin_ssd3_resume]
SSDC_PINS = [pin_ssdc_omega_zero_is_ssd3, pin_ssdc_rope_bruteforce, pin_ssdc_geometric, pin_ssdc_previous_token]
SSDM_PINS = [pin_ssdm_rank_one_is_siso, pin_ssdm_superposition, pin_ssdm_bruteforce, pin_ssdm_resume]
BWD_PINS = [pin_scan_bwd_finite_differences, pin_scan_bwd_linear_in_upstream]
CONV_PINS = [pin_conv_numpy, pin_conv_impulse, pin_conv_chaining, pin_conv_scan_composition]
ALL_PINS = SCAN_PINS + SSD_PINS + SSD3_PINS + SSDC_PINS + SSDM_PINS + BWD_PINS + CONV_PINS
