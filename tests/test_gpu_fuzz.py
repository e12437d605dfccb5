"""Seeded random shapes through every entry point that computes (forward, decode, gradients, training-mode
forward, convolution in front), against the fp64 oracle.

The hand-picked cases elsewhere cover the known corners; these draw batch, length, widths, state size,
I/O type and the optional operands at random (fixed seeds, so every run sees the same shapes), to reach
planner choices, ragged tails and partial blocks that no one thought to list. Sizes stay small enough
for the oracle to finish each case in well under a second."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import RTOL, check, dev, host64, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import selective_state_space_17_amd as m
    return m


def _scan_case(seed):
    r = np.random.default_rng(seed)
    b = int(r.integers(1, 4))
    l = int(r.integers(1, 900))
    d = int(r.integers(1, 300))
    n = int(r.choice([1, 2, 3, 4, 7, 8, 12, 16, 16, 16, 24, 32, 48, 64]))
    io = str(r.choice(["f32", "bf16"]))
    return b, l, d, n, io, bool(r.integers(2)), bool(r.integers(2)), bool(r.integers(2))


def _ssd_case(seed):
    r = np.random.default_rng(seed)
    g = int(r.choice([1, 1, 2, 4]))
    h = g * int(r.integers(1, 4))
    p = int(r.choice([64, 64, 128]))
    n = 16 * int(r.integers(1, 9))
    b = int(r.integers(1, 3))
    l = int(r.integers(1, 300))
    return b, l, h, p, n, g, bool(r.integers(2)), bool(r.integers(2)), bool(r.integers(2))


def _ssd_case_any(seed):
    """Shapes off the 64/128 grid: either I/O type, headdims that are or are not a multiple of 8 and dstate
    up to 256, so that random cases reach the recurrent route, the cut headdim slices and the two-share
    block route as well."""
    r = np.random.default_rng(seed)
    g = int(r.choice([1, 1, 2, 4]))
    h = g * int(r.integers(1, 4))
    p = int(8 * r.integers(1, 21)) if r.integers(2) else int(r.integers(1, 161))
    n = int(r.integers(1, 257))
    io = str(r.choice(["f32", "bf16", "bf16"]))
    b, l = int(r.integers(1, 3)), int(r.integers(1, 300))
    return b, l, h, p, n, g, io, bool(r.integers(2)), bool(r.integers(2)), bool(r.integers(2))


SCAN_SEEDS = list(range(7100, 7114))
SSD_SEEDS = list(range(7200, 7210))


@pytest.mark.parametrize("seed", SCAN_SEEDS)
def test_fuzz_scan_fwd(M, seed):
    import torch
    b, l, d, n, io, hd, hz, hh = case = _scan_case(seed)
    say("fuzz scan fwd", seed, case)
    cfg = W.scan_config(b, l, d, n, io=io, has_D=hd, has_z=hz, cfg_id=seed)
    inp = W.make_scan_inputs(cfg, with_h0=hh)
    out, fin = M.selective_scan_fwd(dev(inp.x), dev(inp.delta), dev(inp.A), dev(inp.B), dev(inp.C), dev(inp.D),
                                    dev(inp.z), dev(inp.h0), return_final_state=True)
    torch.cuda.synchronize()
    ref, ref_fin = oracle.scan_fwd(inp.x, inp.delta, inp.A, inp.B, inp.C, inp.D, inp.z, inp.h0)
    check(host64(out), ref, RTOL[io], f"{case} out")
    check(host64(fin), ref_fin, RTOL[io], f"{case} final_state")


@pytest.mark.parametrize("seed", SCAN_SEEDS[:8])
def test_fuzz_scan_update(M, seed):
    """The decode step over a few tokens from a stored state, at random widths and state sizes (up to 256)."""
    import torch
    r = np.random.default_rng(seed + 50)
    b, d = int(r.integers(1, 9)), int(r.integers(1, 400))
    n = int(r.integers(1, 257))
    l = int(r.integers(1, 5))
    io = str(r.choice(["f32", "bf16"]))
    hd, hz = bool(r.integers(2)), bool(r.integers(2))
    say("fuzz scan update", seed, (b, l, d, n, io, hd, hz))
    cfg = W.scan_config(b, l, d, n, io=io, has_D=hd, has_z=hz, cfg_id=seed + 50)
    inp = W.make_scan_inputs(cfg, with_h0=True)
    state = dev(inp.h0).clone()
    out = M.selective_state_update(state, dev(inp.x), dev(inp.delta), dev(inp.A), dev(inp.B), dev(inp.C),
                                   dev(inp.D), dev(inp.z))
    torch.cuda.synchronize()
    ref, ref_fin = oracle.scan_fwd(inp.x, inp.delta, inp.A, inp.B, inp.C, inp.D, inp.z, inp.h0)
    check(host64(out), ref, RTOL[io], "update out")
    check(host64(state), ref_fin, RTOL[io], "update state")


@pytest.mark.parametrize("seed", SSD_SEEDS)
def test_fuzz_ssd_fwd(M, seed):
    import torch
    b, l, h, p, n, g, hd, hz, hh = case = _ssd_case(seed)
    say("fuzz ssd fwd", seed, case)
    cfg = W.ssd_config(b, l, h, p, n, g, cfg_id=seed)
    s = W.make_ssd_inputs(cfg, with_D=hd, with_z=hz, with_h0=hh)
    out, fin = M.ssd_fwd(dev(s.x), dev(s.delta), dev(s.A), dev(s.B), dev(s.C), dev(s.D), dev(s.z), dev(s.h0),
                         return_final_state=True)
    torch.cuda.synchronize()
    ref, ref_fin = oracle.ssd_fwd(s.x, s.delta, s.A, s.B, s.C, s.D, s.z, s.h0)
    check(host64(out), ref, RTOL["bf16"], f"{case} out")
    check(host64(fin), ref_fin, RTOL["bf16"], f"{case} final_state")


@pytest.mark.parametrize("seed", list(range(7220, 7232)))
def test_fuzz_ssd_fwd_any_shape(M, seed):
    import torch
    b, l, h, p, n, g, io, hd, hz, hh = case = _ssd_case_any(seed)
    say("fuzz ssd fwd any shape", seed, case)
    cfg = W.ssd_config(b, l, h, p, n, g, io=io, cfg_id=seed)
    s = W.make_ssd_inputs(cfg, with_D=hd, with_z=hz, with_h0=hh)
    out, fin = M.ssd_fwd(dev(s.x), dev(s.delta), dev(s.A), dev(s.B), dev(s.C), dev(s.D), dev(s.z), dev(s.h0),
                         return_final_state=True)
    torch.cuda.synchronize()
    ref, ref_fin = oracle.ssd_fwd(s.x, s.delta, s.A, s.B, s.C, s.D, s.z, s.h0)
    check(host64(out), ref, RTOL[io], f"{case} out")
    check(host64(fin), ref_fin, RTOL[io], f"{case} final_state")


@pytest.mark.parametrize("seed", SSD_SEEDS[:6])
def test_fuzz_ssd_trapezoidal_fwd(M, seed):
    import torch
    b, l, h, p, n, g, hd, hz, hh = case = _ssd_case(seed + 30)
    say("fuzz ssd trapezoidal fwd", seed, case)
    cfg = W.ssd_config(b, l, h, p, n, g, cfg_id=seed + 30)
    s = W.make_ssd_inputs(cfg, with_D=hd, with_z=hz, with_h0=hh)
    lam = W.make_ssd_lam(cfg)
    out, fin = M.ssd_trapezoidal_fwd(dev(s.x), dev(s.delta), dev(lam), dev(s.A), dev(s.B), dev(s.C), dev(s.D),
                                     dev(s.z), dev(s.h0), return_final_state=True)
    torch.cuda.synchronize()
    ref, ref_fin = oracle.ssd3_fwd(s.x, s.delta, lam, s.A, s.B, s.C, s.D, s.z, s.h0)
    check(host64(out), ref, RTOL["bf16"], f"{case} out")
    check(host64(fin), ref_fin, RTOL["bf16"], f"{case} final_state")


@pytest.mark.parametrize("seed", SSD_SEEDS[:8])
def test_fuzz_ssd_updates(M, seed):
    """The three multi-head decode steps (Mamba-2, the trapezoidal rule, the complex state) at random
    head counts, headdims (any size) and even state sizes up to 256, with either I/O type."""
    import torch
    r = np.random.default_rng(seed + 70)
    g = int(r.choice([1, 2]))
    h = g * int(r.integers(1, 5))
    p = int(r.integers(1, 96))
    n = 2 * int(r.integers(1, 129))
    b, l = int(r.integers(1, 5)), int(r.integers(1, 5))
    io = str(r.choice(["f32", "bf16"]))
    hd, hz = bool(r.integers(2)), bool(r.integers(2))
    case = (b, l, h, p, n, g, io, hd, hz)
    say("fuzz ssd updates", seed, case)
    cfg = W.ssd_config(b, l, h, p, n, g, io=io, cfg_id=seed + 70)
    s = W.make_ssd_inputs(cfg, with_D=hd, with_z=hz, with_h0=True)
    lam, om = W.make_ssd_lam(cfg), W.make_ssd_omega(cfg)
    xp, bp = W.make_ssd_prev(cfg)
    args = [dev(a) for a in (s.x, s.delta)]

    st = dev(s.h0).clone()
    out = M.ssd_state_update(st, *args, dev(s.A), dev(s.B), dev(s.C), dev(s.D), dev(s.z))
    torch.cuda.synchronize()
    ref, ref_fin = oracle.ssd_fwd(s.x, s.delta, s.A, s.B, s.C, s.D, s.z, s.h0)
    check(host64(out), ref, RTOL[io], f"{case} mamba-2 out")
    check(host64(st), ref_fin, RTOL[io], f"{case} mamba-2 state")

    st = dev(s.h0).clone()
    out = M.ssd_trapezoidal_state_update(st, *args, dev(lam), dev(s.A), dev(s.B), dev(s.C), dev(s.D), dev(s.z),
                                         x_prev=dev(xp), B_prev=dev(bp))
    torch.cuda.synchronize()
    ref, ref_fin = oracle.ssdc_fwd(s.x, s.delta, lam, s.A, np.zeros_like(om), s.B, s.C, s.D, s.z, s.h0, xp, bp)
    check(host64(out), ref, RTOL[io], f"{case} trapezoidal out")
    check(host64(st), ref_fin, RTOL[io], f"{case} trapezoidal state")

    st = dev(s.h0).clone()
    out = M.mamba3_siso_update(st, *args, dev(lam), dev(s.A), dev(om), dev(s.B), dev(s.C), dev(s.D), dev(s.z),
                               x_prev=dev(xp), B_prev=dev(bp))
    torch.cuda.synchronize()
    ref, ref_fin = oracle.ssdc_fwd(s.x, s.delta, lam, s.A, om, s.B, s.C, s.D, s.z, s.h0, xp, bp)
    check(host64(out), ref, RTOL[io], f"{case} complex out")
    check(host64(st), ref_fin, RTOL[io], f"{case} complex state")


GRADS = ("dx", "ddelta", "dz", "dB", "dC", "dA", "dD", "dh0")


def _compare_grads(g, ref, io, what):
    for k in GRADS:
        if ref[k] is None or g[k] is None:
            assert (ref[k] is None) == (g[k] is None) or k == "dh0", f"{what}: {k} presence differs"
            continue
        check(host64(g[k]), ref[k], RTOL[io], f"{what} {k}")


@pytest.mark.parametrize("seed", list(range(7300, 7308)))
def test_fuzz_scan_bwd(M, seed):
    """Gradients at random shapes with dstate up to 16. Cases that the training-mode forward takes (dstate
    16, rows a multiple of 16 bytes) also go through it: the gradients from its checkpoints must match too."""
    import torch
    r = np.random.default_rng(seed)
    io = str(r.choice(["f32", "bf16"]))
    b, l = int(r.integers(1, 4)), int(r.integers(1, 400))
    via_ckpt = bool(r.integers(2))
    if via_ckpt:
        n, d = 16, (8 if io == "bf16" else 4) * int(r.integers(1, 30))
    else:
        n, d = int(r.integers(1, 17)), int(r.integers(1, 200))
    hd, hz, hh, hf = (bool(v) for v in r.integers(2, size=4))
    case = (b, l, d, n, io, hd, hz, hh, hf, via_ckpt)
    say("fuzz scan bwd", seed, case)
    cfg = W.scan_config(b, l, d, n, io=io, has_D=hd, has_z=hz, cfg_id=seed)
    inp = W.make_scan_inputs(cfg, with_h0=hh)
    dout, dfin = W.make_scan_grads(cfg, with_dfinal=hf)
    ref = oracle.scan_bwd(inp.x, inp.delta, inp.A, inp.B, inp.C, inp.D, inp.z, inp.h0, dout, dfin)
    args = [dev(a) for a in (inp.x, inp.delta, inp.A, inp.B, inp.C, inp.D, inp.z, inp.h0)]
    g = M.selective_scan_bwd(*args, dev(dout), dev(dfin))
    torch.cuda.synchronize()
    _compare_grads(g, ref, io, f"{case}")
    if via_ckpt:
        _, ck = M.selective_scan_fwd_ckpt(*args)
        g = M.selective_scan_bwd(*args, dev(dout), dev(dfin), checkpoints=ck)
        torch.cuda.synchronize()
        _compare_grads(g, ref, io, f"{case} from checkpoints")


@pytest.mark.parametrize("seed", list(range(7310, 7316)))
def test_fuzz_scan_bwd_wide_state(M, seed):
    """Gradients with dstate above 16 (one to sixteen slices of 16 states, the last one ragged)."""
    import torch
    r = np.random.default_rng(seed)
    io = str(r.choice(["f32", "bf16"]))
    b, l, d = int(r.integers(1, 3)), int(r.integers(1, 300)), int(r.integers(1, 100))
    n = int(r.integers(17, 257))
    hd, hz, hh, hf = (bool(v) for v in r.integers(2, size=4))
    case = (b, l, d, n, io, hd, hz, hh, hf)
    say("fuzz scan bwd wide state", seed, case)
    cfg = W.scan_config(b, l, d, n, io=io, has_D=hd, has_z=hz, cfg_id=seed)
    inp = W.make_scan_inputs(cfg, with_h0=hh)
    dout, dfin = W.make_scan_grads(cfg, with_dfinal=hf)
    ref = oracle.scan_bwd(inp.x, inp.delta, inp.A, inp.B, inp.C, inp.D, inp.z, inp.h0, dout, dfin)
    g = M.selective_scan_bwd(*[dev(a) for a in (inp.x, inp.delta, inp.A, inp.B, inp.C, inp.D, inp.z, inp.h0)],
                             dev(dout), dev(dfin))
    torch.cuda.synchronize()
    _compare_grads(g, ref, io, f"{case}")


@pytest.mark.parametrize("seed", list(range(7400, 7406)))
def test_fuzz_conv_scan(M, seed):
    """The convolution fused in front of the scan (dstate 16, rows a multiple of 16 bytes), random width,
    bias, initial inputs, state and optional operands."""
    import torch
    r = np.random.default_rng(seed)
    io = str(r.choice(["f32", "bf16"]))
    b, l = int(r.integers(1, 4)), int(r.integers(1, 500))
    d = (8 if io == "bf16" else 4) * int(r.integers(1, 40))
    width = int(r.integers(1, 5))
    hb, hi, hh, hd, hz = (bool(v) for v in r.integers(2, size=5))
    case = (b, l, d, width, io, hb, hi, hh, hd, hz)
    say("fuzz conv scan", seed, case)
    cfg = W.scan_config(b, l, d, 16, io=io, has_D=hd, has_z=hz, cfg_id=seed)
    inp = W.make_scan_inputs(cfg, with_h0=hh)
    w, bias, init = W.make_conv_inputs(cfg, width, with_bias=hb, with_init=hi)
    out, fin = M.selective_scan_conv_fwd(dev(inp.x), dev(w), dev(bias), dev(init), dev(inp.delta), dev(inp.A),
                                         dev(inp.B), dev(inp.C), dev(inp.D), dev(inp.z), dev(inp.h0),
                                         return_final_state=True)
    torch.cuda.synchronize()
    ref, ref_fin = oracle.conv_scan_fwd(inp.x, w, bias, init, inp.delta, inp.A, inp.B, inp.C, inp.D, inp.z, inp.h0)
    check(host64(out), ref, RTOL[io], f"{case} out")
    check(host64(fin), ref_fin, RTOL[io], f"{case} final_state")


@pytest.mark.parametrize("seed", list(range(7500, 7506)))
def test_fuzz_conv_update(M, seed):
    """The decode step with the convolution window, any dstate: outputs and state against the fused
    oracle started from the window, and the new window equal to the last W-1 inputs bit for bit."""
    import torch
    r = np.random.default_rng(seed)
    io = str(r.choice(["f32", "bf16"]))
    b, t, d = int(r.integers(1, 6)), int(r.integers(1, 6)), int(r.integers(1, 300))
    n, width = int(r.integers(1, 129)), int(r.integers(1, 5))
    hb, hd, hz = (bool(v) for v in r.integers(2, size=3))
    case = (b, t, d, n, width, io, hb, hd, hz)
    say("fuzz conv update", seed, case)
    cfg = W.scan_config(b, t, d, n, io=io, has_D=hd, has_z=hz, cfg_id=seed)
    inp = W.make_scan_inputs(cfg, with_h0=True)
    w, bias, init = W.make_conv_inputs(cfg, width, with_bias=hb)
    state = dev(inp.h0).clone()
    cstate = dev(init).clone() if init is not None else None
    out = M.selective_state_update_conv(state, cstate, dev(inp.x), dev(w), dev(bias), dev(inp.delta), dev(inp.A),
                                        dev(inp.B), dev(inp.C), dev(inp.D), dev(inp.z))
    torch.cuda.synchronize()
    ref, ref_fin = oracle.conv_scan_fwd(inp.x, w, bias, init, inp.delta, inp.A, inp.B, inp.C, inp.D, inp.z, inp.h0)
    check(host64(out), ref, RTOL[io], f"{case} out")
    check(host64(state), ref_fin, RTOL[io], f"{case} state")
    if width > 1:
        want = np.concatenate([init, inp.x], axis=1)[:, -(width - 1):]
        assert np.array_equal(host_raw(cstate), want), f"{case}: window"


def host_raw(t):
    """A device tensor's elements as stored (bf16 as its uint16 bits), for bit-exact comparisons."""
    import torch
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def _ssd_any_case(seed):
    """Any multi-head problem: either I/O type, any headdim, dstate up to 256, several groups -- mostly
    shapes the matrix-core block kernel does not take, which run through the recurrent update kernel."""
    r = np.random.default_rng(seed)
    io = str(r.choice(["f32", "bf16"]))
    g = int(r.choice([1, 2, 3]))
    h = g * int(r.integers(1, 4))
    p = int(r.integers(1, 140))
    n = int(r.integers(1, 257))
    b, l = int(r.integers(1, 3)), int(r.integers(1, 200))
    return b, l, h, p, n, g, io, bool(r.integers(2)), bool(r.integers(2)), bool(r.integers(2))


@pytest.mark.parametrize("seed", list(range(7600, 7610)))
def test_fuzz_ssd_any_shape(M, seed):
    """Both multi-head sequence entry points (the Mamba-2 and the Mamba-3 rule) at random shapes and I/O
    types off the block kernel's grid; each draw states the route the library takes."""
    import torch
    b, l, h, p, n, g, io, hd, hz, hh = case = _ssd_any_case(seed)
    route = M.ssd_plan(b, l, h, p, n, g, 0, M.MSSM_BF16 if io == "bf16" else M.MSSM_F32)
    say("fuzz ssd any shape", seed, case, "route", route)
    cfg = W.ssd_config(b, l, h, p, n, g, io=io, cfg_id=seed)
    s = W.make_ssd_inputs(cfg, with_D=hd, with_z=hz, with_h0=hh)
    out, fin = M.ssd_fwd(dev(s.x), dev(s.delta), dev(s.A), dev(s.B), dev(s.C), dev(s.D), dev(s.z), dev(s.h0),
                         return_final_state=True)
    torch.cuda.synchronize()
    ref, ref_fin = oracle.ssd_fwd(s.x, s.delta, s.A, s.B, s.C, s.D, s.z, s.h0)
    check(host64(out), ref, RTOL[io], f"{case} out")
    check(host64(fin), ref_fin, RTOL[io], f"{case} final_state")
    lam = W.make_ssd_lam(cfg)
    out, fin = M.ssd_trapezoidal_fwd(dev(s.x), dev(s.delta), dev(lam), dev(s.A), dev(s.B), dev(s.C), dev(s.D),
                                     dev(s.z), dev(s.h0), return_final_state=True)
    torch.cuda.synchronize()
    ref, ref_fin = oracle.ssd3_fwd(s.x, s.delta, lam, s.A, s.B, s.C, s.D, s.z, s.h0)
    check(host64(out), ref, RTOL[io], f"{case} trapezoidal out")
    check(host64(fin), ref_fin, RTOL[io], f"{case} trapezoidal final_state")


@pytest.mark.parametrize("seed", list(range(7700, 7706)))
def test_fuzz_conv_scan_any_shape(M, seed):
    """The convolution + scan at shapes the fused kernel does not take (any dstate up to 256, rows that are
    not a multiple of 16 bytes): the recurrent route, against the fused oracle."""
    import torch
    r = np.random.default_rng(seed)
    io = str(r.choice(["f32", "bf16"]))
    b, l, d = int(r.integers(1, 3)), int(r.integers(1, 300)), int(r.integers(1, 200))
    n = int(r.integers(1, 257))
    width = int(r.integers(1, 5))
    hb, hi, hh, hd, hz = (bool(v) for v in r.integers(2, size=5))
    case = (b, l, d, n, width, io, hb, hi, hh, hd, hz)
    say("fuzz conv scan any shape", seed, case)
    cfg = W.scan_config(b, l, d, n, io=io, has_D=hd, has_z=hz, cfg_id=seed)
    inp = W.make_scan_inputs(cfg, with_h0=hh)
    w, bias, init = W.make_conv_inputs(cfg, width, with_bias=hb, with_init=hi)
    out, fin = M.selective_scan_conv_fwd(dev(inp.x), dev(w), dev(bias), dev(init), dev(inp.delta), dev(inp.A),
                                         dev(inp.B), dev(inp.C), dev(inp.D), dev(inp.z), dev(inp.h0),
                                         return_final_state=True)
    torch.cuda.synchronize()
    ref, ref_fin = oracle.conv_scan_fwd(inp.x, w, bias, init, inp.delta, inp.A, inp.B, inp.C, inp.D, inp.z, inp.h0)
    check(host64(out), ref, RTOL[io], f"{case} out")
    check(host64(fin), ref_fin, RTOL[io], f"{case} final_state")
