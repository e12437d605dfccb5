"""Seeded synthetic inputs for the selective-scan workloads.

This module is shared by the CPU oracle side (tests) and the GPU side (tests,
bench).  It holds the input recipe only -- shapes, value distributions and the
bf16 rounding of inputs -- and none of the scan's arithmetic.

Recipe (the workloads the pages describe, made concrete):
  * Mamba-1 selective scan (page "03 - Modelos de espacio de estados",
    sections "El mecanismo selectivo de Mamba" and "Discretizacion"): per-token
    step size delta, per-token B and C shared across channels, fixed diagonal
    negative A per (channel, state).
  * Mamba-2 scalar-A multi-head form (page "Mamba-2 y state-space models",
    section 4.2; page "Mamba-3", introduction: the transition is a scalar
    times the identity): per-(token, head) delta, scalar A per head, B/C per
    (token, group).
  * Mamba-3 MIMO (page "Mamba-3", "El modelo Mamba-3" item 3): R inputs and
    outputs per channel, x and z ~ N(0, 1) per rank, B and C ~ N(0, 1) per
    (token, group, rank).
  * Mamba-3 SISO rule (page "Mamba-3", "El modelo Mamba-3"): the weight lam
    per (token, head), sigmoid(N(0, 1)), as a gate computed from the token
    would give; for its decode step, the previous token's x and B ~ N(0, 1);
    for the complex-valued state, rotation rates omega ~ U(-pi, pi) per
    (head, state pair).

Distributions: x, z, B, C ~ N(0, 1); D ~ N(0, 1) per channel;
delta = softplus(0.5 * N(0, 1) - 2) evaluated in fp32; S4D-real A[c, n] =
-(n + 1); "A = -exp(log k)" evaluated in fp32; SSD A[h] = -exp(U(log 1, log 16)).

Random streams: tensor `k` of workload `cfg_id` is drawn in blocks of
``BLOCK`` elements; block `j` comes from numpy PCG64 seeded with
SeedSequence([ROOT_SEED + cfg_id, k, j]).  Values are drawn in fp32 and
rounded to bf16 (round-to-nearest-even) where the workload's I/O is bf16.
Blocks make generation streamable and deterministic for any size.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

ROOT_SEED = 1700
BLOCK = 1 << 22

# tensor ids (fixed order of the per-tensor streams)
T_X, T_DELTA, T_Z, T_B, T_C, T_D, T_A, T_H0, T_DOUT, T_DFIN, T_CW, T_CB, T_CI, T_LAM, T_XPREV, T_BPREV, T_OMEGA = \
    range(17)

F32 = "f32"
BF16 = "bf16"


@dataclasses.dataclass(frozen=True)
class ScanConfig:
    """Mamba-1 selective scan workload: x/delta/z [B, L, D], B/C [B, L, N], A [D, N]."""
    name: str
    cfg_id: int
    batch: int
    seqlen: int
    dim: int
    dstate: int
    io: str                 # "f32" or "bf16"
    a_kind: str             # "s4d_real" (-(n+1)) or "exp_log" (-exp(log k) in fp32)
    has_D: bool = True
    has_z: bool = True
    return_final: bool = True
    decode: bool = False    # token-by-token update of a stored state (read and written in place)
    backward: bool = False  # gradients: dout in, dx/ddelta/dz (io) and dB/dC/dA/dD (fp32) out
    conv_width: int = 0     # > 0: a short causal convolution + SiLU of this width makes x from its input
    train: bool = False     # training step: forward that stores checkpoints, then gradients from them

    @property
    def updates(self) -> int:
        return self.batch * self.seqlen * self.dim * self.dstate

    def algorithmic_bytes(self) -> int:
        """Every input read once, every output written once (a decode step also reads the state)."""
        e = 2 if self.io == BF16 else 4
        bld = self.batch * self.seqlen * self.dim
        bln = self.batch * self.seqlen * self.dstate
        if self.train:   # the forward pass, then the gradient pass (each reads its inputs once)
            fwd = dataclasses.replace(self, train=False, backward=False)
            bwd = dataclasses.replace(self, train=False, backward=True)
            return fwd.algorithmic_bytes() + bwd.algorithmic_bytes()
        if self.backward:
            zf = 2 if self.has_z else 0
            n = bld * e * (2 + 1 + 2 + zf)          # x, delta, dout in; dx, ddelta out; z in, dz out
            n += bln * e * 2 + bln * 4 * 2          # B, C in; dB, dC out (fp32)
            n += self.dim * self.dstate * 4 * 2     # A in, dA out
            n += self.dim * 4 * 2 if self.has_D else 0
            n += self.batch * self.dim * self.dstate * 4 * 2 if self.return_final else 0   # dfinal in, dh0 out
            return n
        n = bld * e * 2                     # x, delta
        n += bld * e if self.has_z else 0   # z
        n += bln * e * 2                    # B, C
        n += self.dim * self.dstate * 4     # A (fp32)
        n += self.dim * 4 if self.has_D else 0
        n += self.dim * (self.conv_width + 1) * 4 if self.conv_width else 0   # taps and bias
        n += bld * e                        # out
        n += self.batch * self.dim * self.dstate * 4 if self.return_final else 0
        n += self.batch * self.dim * self.dstate * 4 if self.decode else 0
        return n


@dataclasses.dataclass(frozen=True)
class SSDConfig:
    """Mamba-2 scalar-A multi-head workload: x/z [B, L, H, P], delta [B, L, H], B/C [B, L, G, N]."""
    name: str
    cfg_id: int
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    chunk: int
    io: str = BF16
    has_D: bool = False
    has_z: bool = False
    return_final: bool = True
    decode: bool = False    # token-by-token update of a stored state (read and written in place)
    trapezoidal: bool = False   # Mamba-3 exponential-trapezoidal input rule (one more [B, L, H] input, lam)
    complex_state: bool = False  # Mamba-3 complex-valued state: rotation rates omega [H, N/2] fp32
    rank: int = 1           # Mamba-3 MIMO: R inputs and outputs per channel, x/z/out [B, L, H, R, P], B/C [B, L, G, R, N]

    @property
    def updates(self) -> int:
        """State-element updates (each absorbs the R inputs of its step under MIMO)."""
        return self.batch * self.seqlen * self.nheads * self.headdim * self.dstate

    def algorithmic_bytes(self) -> int:
        e = 2 if self.io == BF16 else 4
        R = self.rank
        blhp = self.batch * self.seqlen * self.nheads * self.headdim * R
        n = blhp * e                                            # x
        n += self.batch * self.seqlen * self.nheads * e         # delta
        n += self.batch * self.seqlen * self.nheads * e if self.trapezoidal else 0   # lam
        n += 2 * self.batch * self.seqlen * self.ngroups * R * self.dstate * e  # B, C
        n += self.nheads * 4                                    # A
        n += self.nheads * 4 if self.has_D else 0
        n += blhp * e if self.has_z else 0
        n += blhp * e                                           # out
        n += self.batch * self.nheads * self.headdim * self.dstate * 4 if self.return_final else 0
        n += self.batch * self.nheads * self.headdim * self.dstate * 4 if self.decode else 0
        if self.decode and self.trapezoidal:   # the previous token's x and B
            n += (self.batch * self.nheads * self.headdim + self.batch * self.ngroups * self.dstate) * R * e
        n += self.nheads * (self.dstate // 2) * 4 if self.complex_state else 0   # omega
        return n


# The workloads by id.  1 is the small fp32 case; 2 is the 130M-like layer
# the throughput figure is quoted on; 3-5 are the larger forward layers and
# the SSD form; 6-12 add the decode step, gradients, the convolution in front,
# the training step and the Mamba-3 rule (13: with the complex state) on the same shapes.
CONFIGS = {
    1: ScanConfig("mamba1_tiny_f32", 1, 1, 256, 64, 16, F32, "s4d_real", return_final=True),
    2: ScanConfig("mamba1_130m_layer_bf16", 2, 8, 2048, 1536, 16, BF16, "exp_log", return_final=False),
    3: ScanConfig("mamba1_2p8b_layer_bf16", 3, 4, 8192, 5120, 16, BF16, "s4d_real", return_final=True),
    4: SSDConfig("mamba2_ssd_bf16", 4, 8, 4096, 32, 64, 128, 1, 256),
    5: ScanConfig("mamba1_long_1m_bf16", 5, 1, 1 << 20, 2048, 16, BF16, "s4d_real", return_final=True),
    # gradients of config 2's layer (one backward pass; no final-state gradient)
    8: ScanConfig("mamba1_130m_layer_bwd_bf16", 8, 8, 2048, 1536, 16, BF16, "exp_log", return_final=False,
                  backward=True),
    # config 2's layer with its width-4 short causal convolution + SiLU fused in front (x from its input)
    9: ScanConfig("mamba1_130m_layer_conv_bf16", 9, 8, 2048, 1536, 16, BF16, "exp_log", return_final=False,
                  conv_width=4),
    # a training step of config 2's layer: forward storing checkpoints, then the gradients from them
    10: ScanConfig("mamba1_130m_layer_train_bf16", 10, 8, 2048, 1536, 16, BF16, "exp_log", return_final=False,
                   train=True),
    # decode steps (one new token against a stored state), the configs' layer shapes at serving batch sizes
    6: ScanConfig("mamba1_2p8b_decode_bf16", 6, 256, 1, 5120, 16, BF16, "s4d_real", return_final=True, decode=True),
    7: SSDConfig("mamba2_decode_bf16", 7, 64, 1, 32, 64, 128, 1, 64, BF16, True, True, True, decode=True),
    # the Mamba-3 SISO recurrence (exponential-trapezoidal input rule) at config 4's shape: SISO keeps
    # Mamba-2's dimensions and state size
    11: SSDConfig("mamba3_siso_bf16", 11, 8, 4096, 32, 64, 128, 1, 256, trapezoidal=True),
    # its decode step at config 7's serving shape (the previous token's x and B are inputs too)
    12: SSDConfig("mamba3_siso_decode_bf16", 12, 64, 1, 32, 64, 128, 1, 64, BF16, True, True, True, decode=True,
                  trapezoidal=True),
    # the same decode step with the complex-valued state (each state pair rotated by delta * omega)
    13: SSDConfig("mamba3_siso_complex_decode_bf16", 13, 64, 1, 32, 64, 128, 1, 64, BF16, True, True, True,
                  decode=True, trapezoidal=True, complex_state=True),
    # Mamba-3 MIMO at config 4's shape: 4 inputs and 4 outputs per channel on each head's one state
    14: SSDConfig("mamba3_mimo_bf16", 14, 8, 4096, 32, 64, 128, 1, 256, trapezoidal=True, rank=4),
    # its decode step at config 7's serving shape (the previous token's 4 inputs and B rows too)
    15: SSDConfig("mamba3_mimo_decode_bf16", 15, 64, 1, 32, 64, 128, 1, 64, BF16, True, True, True, decode=True,
                  trapezoidal=True, rank=4),
    # gradients of config 2's layer with 128 states per channel (the larger state sizes of the d_state sweep)
    16: ScanConfig("mamba1_130m_layer_bwd_n128_bf16", 16, 8, 2048, 1536, 128, BF16, "exp_log", return_final=False,
                   backward=True),
    # config 4's shape with 256 states per head (the largest state size of the d_state sweep)
    17: SSDConfig("mamba2_ssd_n256_bf16", 17, 8, 4096, 32, 64, 256, 1, 256),
}


# ----------------------------------------------------------------------------
# fp32 -> bf16 (round to nearest even), as raw uint16 bit patterns
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (RNE); returns uint16 bit patterns. Inputs are finite."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ----------------------------------------------------------------------------
# blocked, seeded streams
# ----------------------------------------------------------------------------
def _stream(cfg_id: int, tensor: int, block: int, seed_base: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed_base + cfg_id, tensor, block])))


def _blocks(n: int):
    for j, s in enumerate(range(0, n, BLOCK)):
        yield j, s, min(n, s + BLOCK)


_WORKERS = max(1, min(16, len(os.sched_getaffinity(0))))


def _for_blocks(n: int, fn) -> None:
    """Run fn(j, s, e) for every block (independent streams, so order does not matter)."""
    blocks = list(_blocks(n))
    if len(blocks) <= 1:
        for blk in blocks:
            fn(*blk)
        return
    with ThreadPoolExecutor(max_workers=_WORKERS) as ex:
        list(ex.map(lambda blk: fn(*blk), blocks))


def _alloc(n: int, io: str) -> np.ndarray:
    return np.empty(n, dtype=np.uint16 if io == BF16 else np.float32)


def _store(out: np.ndarray, s: int, e: int, v: np.ndarray) -> None:
    out[s:e] = f32_to_bf16_bits(v) if out.dtype == np.uint16 else v


def normal(cfg_id: int, tensor: int, n: int, io: str = F32, seed_base: int = ROOT_SEED) -> np.ndarray:
    """N(0,1) drawn in fp32, stored in io dtype (bf16 bits rounded to nearest even)."""
    out = _alloc(n, io)

    def fill(j, s, e):
        _store(out, s, e, _stream(cfg_id, tensor, j, seed_base).standard_normal(e - s, dtype=np.float32))

    _for_blocks(n, fill)
    return out


def normal_f32(cfg_id: int, tensor: int, n: int, seed_base: int = ROOT_SEED) -> np.ndarray:
    return normal(cfg_id, tensor, n, F32, seed_base)


def uniform_f32(cfg_id: int, tensor: int, n: int, lo: float, hi: float, seed_base: int = ROOT_SEED) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    for j, s, e in _blocks(n):
        g = _stream(cfg_id, tensor, j, seed_base)
        out[s:e] = g.random(e - s, dtype=np.float32) * np.float32(hi - lo) + np.float32(lo)
    return out


def softplus_delta(cfg_id: int, n: int, io: str = F32, seed_base: int = ROOT_SEED) -> np.ndarray:
    """delta = softplus(0.5 * N(0,1) - 2), evaluated in fp32, stored in io dtype."""
    out = _alloc(n, io)

    def fill(j, s, e):
        v = _stream(cfg_id, T_DELTA, j, seed_base).standard_normal(e - s, dtype=np.float32)
        v *= np.float32(0.5)
        v -= np.float32(2.0)
        np.log1p(np.exp(v), out=v)
        _store(out, s, e, v)

    _for_blocks(n, fill)
    return out


def softplus_delta_f32(cfg_id: int, n: int, seed_base: int = ROOT_SEED) -> np.ndarray:
    return softplus_delta(cfg_id, n, F32, seed_base)


def s4d_real_A(dim: int, dstate: int) -> np.ndarray:
    return -np.tile(np.arange(1, dstate + 1, dtype=np.float32), (dim, 1))


def exp_log_A(dim: int, dstate: int) -> np.ndarray:
    k = np.arange(1, dstate + 1, dtype=np.float32)
    a = -np.exp(np.log(k))          # fp32 arithmetic throughout
    return np.tile(a.astype(np.float32), (dim, 1))


@dataclasses.dataclass
class ScanInputs:
    """Host arrays. Tensors in io dtype are uint16 (bf16 bits) or float32."""
    x: np.ndarray
    delta: np.ndarray
    A: np.ndarray
    B: np.ndarray
    C: np.ndarray
    D: Optional[np.ndarray]
    z: Optional[np.ndarray]
    h0: Optional[np.ndarray]
    io: str


def make_scan_inputs(cfg: ScanConfig, seed_base: int = ROOT_SEED, with_h0: bool = False) -> ScanInputs:
    b, l, d, n = cfg.batch, cfg.seqlen, cfg.dim, cfg.dstate
    cid = cfg.cfg_id
    x = normal(cid, T_X, b * l * d, cfg.io, seed_base).reshape(b, l, d)
    delta = softplus_delta(cid, b * l * d, cfg.io, seed_base).reshape(b, l, d)
    z = normal(cid, T_Z, b * l * d, cfg.io, seed_base).reshape(b, l, d) if cfg.has_z else None
    Bm = normal(cid, T_B, b * l * n, cfg.io, seed_base).reshape(b, l, n)
    Cm = normal(cid, T_C, b * l * n, cfg.io, seed_base).reshape(b, l, n)
    D = normal_f32(cid, T_D, d, seed_base) if cfg.has_D else None
    if cfg.a_kind == "s4d_real":
        A = s4d_real_A(d, n)
    elif cfg.a_kind == "exp_log":
        A = exp_log_A(d, n)
    else:
        raise ValueError(cfg.a_kind)
    h0 = normal_f32(cid, T_H0, b * d * n, seed_base).reshape(b, d, n) if with_h0 else None
    return ScanInputs(x, delta, np.ascontiguousarray(A), Bm, Cm, D, z, h0, cfg.io)


def make_scan_grads(cfg: ScanConfig, seed_base: int = ROOT_SEED, with_dfinal: bool = True):
    """Upstream gradients for the scan: dout [B, L, D] ~ N(0, 1) in io dtype, dfinal [B, D, N] ~ N(0, 1) fp32."""
    b, l, d, n = cfg.batch, cfg.seqlen, cfg.dim, cfg.dstate
    dout = normal(cfg.cfg_id, T_DOUT, b * l * d, cfg.io, seed_base).reshape(b, l, d)
    dfin = normal_f32(cfg.cfg_id, T_DFIN, b * d * n, seed_base).reshape(b, d, n) if with_dfinal else None
    return dout, dfin


def make_conv_inputs(cfg: ScanConfig, width: int, seed_base: int = ROOT_SEED, with_bias: bool = True,
                     with_init: bool = True):
    """Short-convolution parameters: taps [D, W] ~ U(-1, 1) / sqrt(W) fp32, bias [D] ~ N(0, 1) / 4 fp32,
    init [B, W-1, D] ~ N(0, 1) in io dtype (the inputs before t = 0)."""
    b, d = cfg.batch, cfg.dim
    w = uniform_f32(cfg.cfg_id, T_CW, d * width, -1.0, 1.0, seed_base).reshape(d, width)
    w = (w / np.float32(np.sqrt(width))).astype(np.float32)
    bias = (normal_f32(cfg.cfg_id, T_CB, d, seed_base) * np.float32(0.25)).astype(np.float32) if with_bias else None
    init = None
    if with_init and width > 1:
        init = normal(cfg.cfg_id, T_CI, b * (width - 1) * d, cfg.io, seed_base).reshape(b, width - 1, d)
    return w, bias, init


@dataclasses.dataclass
class SSDInputs:
    x: np.ndarray       # [B, L, H, P]
    delta: np.ndarray   # [B, L, H]
    A: np.ndarray       # [H] fp32
    B: np.ndarray       # [B, L, G, N]
    C: np.ndarray       # [B, L, G, N]
    D: Optional[np.ndarray]
    z: Optional[np.ndarray]
    h0: Optional[np.ndarray]   # [B, H, P, N] fp32
    io: str


def make_ssd_inputs(cfg: SSDConfig, seed_base: int = ROOT_SEED, with_D: Optional[bool] = None,
                    with_z: Optional[bool] = None, with_h0: bool = False) -> SSDInputs:
    """x, z [B, L, H, P] and B, C [B, L, G, N]; with cfg.rank R > 1 (MIMO) x, z [B, L, H, R, P] and
    B, C [B, L, G, R, N]."""
    b, l, h, p, n, g = cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim, cfg.dstate, cfg.ngroups
    R = cfg.rank
    xs = (b, l, h, p) if R == 1 else (b, l, h, R, p)
    bs = (b, l, g, n) if R == 1 else (b, l, g, R, n)
    cid = cfg.cfg_id
    with_D = cfg.has_D if with_D is None else with_D
    with_z = cfg.has_z if with_z is None else with_z
    x = normal(cid, T_X, b * l * h * R * p, cfg.io, seed_base).reshape(xs)
    delta = softplus_delta(cid, b * l * h, cfg.io, seed_base).reshape(b, l, h)
    Bm = normal(cid, T_B, b * l * g * R * n, cfg.io, seed_base).reshape(bs)
    Cm = normal(cid, T_C, b * l * g * R * n, cfg.io, seed_base).reshape(bs)
    u = uniform_f32(cid, T_A, h, float(np.log(np.float32(1.0))), float(np.log(np.float32(16.0))), seed_base)
    A = (-np.exp(u)).astype(np.float32)
    D = normal_f32(cid, T_D, h, seed_base) if with_D else None
    z = normal(cid, T_Z, b * l * h * R * p, cfg.io, seed_base).reshape(xs) if with_z else None
    h0 = normal_f32(cid, T_H0, b * h * p * n, seed_base).reshape(b, h, p, n) if with_h0 else None
    return SSDInputs(x, delta, A, Bm, Cm, D, z, h0, cfg.io)


def make_ssd_lam(cfg: SSDConfig, seed_base: int = ROOT_SEED) -> np.ndarray:
    """The Mamba-3 trapezoidal weight lam [B, L, H]: sigmoid of N(0, 1), as a gate computed from the token
    would give (values in (0, 1), most near 1/2), stored in io dtype."""
    n = cfg.batch * cfg.seqlen * cfg.nheads
    out = _alloc(n, cfg.io)

    def fill(j, s, e):
        v = _stream(cfg.cfg_id, T_LAM, j, seed_base).standard_normal(e - s, dtype=np.float32)
        _store(out, s, e, (1.0 / (1.0 + np.exp(-v))).astype(np.float32))

    _for_blocks(n, fill)
    return out.reshape(cfg.batch, cfg.seqlen, cfg.nheads)


def make_ssd_prev(cfg: SSDConfig, seed_base: int = ROOT_SEED):
    """The token before a decode step's first: x_prev [B, H, P] and B_prev [B, G, N] ([B, H, R, P] and
    [B, G, R, N] under MIMO), N(0, 1) in io dtype."""
    R = cfg.rank
    xp = normal(cfg.cfg_id, T_XPREV, cfg.batch * cfg.nheads * R * cfg.headdim, cfg.io, seed_base)
    bp = normal(cfg.cfg_id, T_BPREV, cfg.batch * cfg.ngroups * R * cfg.dstate, cfg.io, seed_base)
    if R == 1:
        return xp.reshape(cfg.batch, cfg.nheads, cfg.headdim), bp.reshape(cfg.batch, cfg.ngroups, cfg.dstate)
    return (xp.reshape(cfg.batch, cfg.nheads, R, cfg.headdim),
            bp.reshape(cfg.batch, cfg.ngroups, R, cfg.dstate))


def make_ssd_omega(cfg: SSDConfig, seed_base: int = ROOT_SEED) -> np.ndarray:
    """Rotation rates of the complex-valued state, omega [H, N/2] fp32 ~ U(-pi, pi): with the workloads'
    delta a state pair turns by a few tenths of a radian per step."""
    n = cfg.nheads * (cfg.dstate // 2)
    return uniform_f32(cfg.cfg_id, T_OMEGA, n, -np.pi, np.pi, seed_base).reshape(cfg.nheads, cfg.dstate // 2)


def scan_config(batch: int, seqlen: int, dim: int, dstate: int, io: str = F32, a_kind: str = "s4d_real",
                has_D: bool = True, has_z: bool = True, cfg_id: int = 100) -> ScanConfig:
    """An ad-hoc Mamba-1 workload with the standard distributions (for tests)."""
    return ScanConfig(f"scan_b{batch}_l{seqlen}_d{dim}_n{dstate}_{io}", cfg_id, batch, seqlen, dim, dstate, io,
                      a_kind, has_D, has_z, True)


def ssd_config(batch: int, seqlen: int, nheads: int, headdim: int, dstate: int, ngroups: int = 1,
               chunk: int = 64, io: str = BF16, has_D: bool = False, has_z: bool = False,
               cfg_id: int = 200, rank: int = 1) -> SSDConfig:
    return SSDConfig(f"ssd_b{batch}_l{seqlen}_h{nheads}_p{headdim}_n{dstate}_g{ngroups}_r{rank}", cfg_id, batch,
                     seqlen, nheads, headdim, dstate, ngroups, chunk, io, has_D, has_z, True, rank=rank)
