"""Gradients of the Mamba-1 scan on the GPU, through the C ABI, against the fp64 oracle.

Every output (dx, ddelta, dz, dB, dC, dA, dD, dh0) is compared element by
element with oracle.scan_bwd on the same seeded inputs and upstream
gradients, under the tolerance rule of gpu_util (1e-4 for fp32 I/O, 2e-2 for
bf16 I/O): small cases that span several 16-step tiles and 16-channel blocks
with ragged tails, dstate below 16, dstate above 16 (several 16-state slices,
ragged ones too, whose partial sums a finishing kernel adds), and the full
8 x 2048 x 1536 layer."""
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


def run_case(M, cfg, with_h0, with_dfinal, want_dh0=True):
    import torch
    inp = W.make_scan_inputs(cfg, with_h0=with_h0)
    dout, dfin = W.make_scan_grads(cfg, with_dfinal=with_dfinal)
    g = M.selective_scan_bwd(dev(inp.x), dev(inp.delta), dev(inp.A), dev(inp.B), dev(inp.C), dev(inp.D),
                             dev(inp.z), dev(inp.h0), dev(dout), dev(dfin), want_dh0=want_dh0)
    torch.cuda.synchronize()
    ref = oracle.scan_bwd(inp.x, inp.delta, inp.A, inp.B, inp.C, inp.D, inp.z, inp.h0, dout, dfin)
    return g, ref


def compare(g, ref, io, what):
    for k in ("dx", "ddelta", "dz", "dB", "dC", "dA", "dD", "dh0"):
        if ref[k] is None or g[k] is None:
            assert (ref[k] is None) == (g[k] is None) or k == "dh0", f"{what}: {k} presence differs"
            continue
        check(host64(g[k]), ref[k], RTOL[io], f"{what} {k}")


# (batch, seqlen, dim, dstate, io, D, z, h0, dfinal)
CASES = [
    (2, 40, 40, 16, "f32", True, True, True, True),      # ragged tile and channel block
    (1, 16, 16, 16, "f32", True, True, False, False),    # one exact tile
    (3, 100, 64, 16, "bf16", True, True, True, True),
    (2, 33, 24, 5, "f32", False, False, False, True),    # dstate < 16, no D / z
    (1, 17, 20, 1, "f32", True, False, True, False),     # dstate 1
    (2, 1, 48, 16, "bf16", True, True, False, True),     # a single step
    (1, 300, 32, 8, "f32", True, True, True, True),
    (2, 257, 100, 16, "bf16", False, True, True, False),
    (1, 20000, 64, 16, "bf16", True, True, True, True),   # 1250 tiles: checkpoint indexing far along
    (1, 256, 5120, 16, "bf16", True, True, False, False), # the 2.8B layer's width: 320 channel blocks
    (2, 40, 40, 17, "f32", True, True, True, True),      # two slices, the second with one state
    (2, 33, 24, 32, "bf16", True, True, True, True),
    (1, 50, 40, 64, "f32", False, True, False, True),
    (2, 40, 48, 128, "bf16", True, True, True, True),
    (1, 37, 20, 256, "f32", True, False, True, True),    # the largest dstate, no z
    (1, 300, 32, 100, "bf16", True, True, True, False),  # a ragged last slice
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "b{}_l{}_d{}_n{}_{}".format(*c[:5]))
def test_scan_bwd_matches_oracle(M, case):
    b, l, d, n, io, hd, hz, h0, dfin = case
    cfg = W.scan_config(b, l, d, n, io=io, has_D=hd, has_z=hz, cfg_id=800 + l + n)
    say("scan bwd", case)
    g, ref = run_case(M, cfg, h0, dfin)
    compare(g, ref, io, f"bwd {case}")


def test_scan_bwd_empty_sequence(M):
    """No steps: dh0 = dfinal, dA = dD = 0, nothing else to write."""
    cfg = W.scan_config(2, 0, 24, 16, io="f32", cfg_id=850)
    say("scan bwd empty sequence")
    g, ref = run_case(M, cfg, True, True)
    assert np.array_equal(host64(g["dh0"]), ref["dh0"])
    assert not host64(g["dA"]).any() and not host64(g["dD"]).any()
    assert g["dB"].numel() == 0


def test_scan_bwd_empty_batch(M):
    """No batch rows: dA and dD are empty sums (zero); nothing else has elements."""
    import torch
    cfg = W.scan_config(0, 32, 24, 16, io="f32", cfg_id=852)
    g, ref = run_case(M, cfg, False, False)
    assert not host64(g["dA"]).any() and not host64(g["dD"]).any()
    assert g["dx"].numel() == 0 and g["dB"].numel() == 0


def test_scan_bwd_deterministic(M):
    """Every sum is taken in a fixed order: two calls agree bit for bit."""
    import torch
    cfg = W.scan_config(4, 200, 96, 16, io="bf16", cfg_id=851)
    inp = W.make_scan_inputs(cfg, with_h0=True)
    dout, dfin = W.make_scan_grads(cfg)
    args = [dev(a) for a in (inp.x, inp.delta, inp.A, inp.B, inp.C, inp.D, inp.z, inp.h0, dout, dfin)]
    say("scan bwd determinism")
    g1 = M.selective_scan_bwd(*args)
    g2 = M.selective_scan_bwd(*args)
    torch.cuda.synchronize()
    for k in g1:
        if g1[k] is not None:
            assert torch.equal(g1[k], g2[k]), f"{k} differs between identical calls"


def test_scan_bwd_deterministic_slices(M):
    """The same with 64 states: the slices' partial sums are added in slice order."""
    import torch
    cfg = W.scan_config(2, 70, 40, 64, io="bf16", cfg_id=853)
    inp = W.make_scan_inputs(cfg, with_h0=True)
    dout, dfin = W.make_scan_grads(cfg)
    args = [dev(a) for a in (inp.x, inp.delta, inp.A, inp.B, inp.C, inp.D, inp.z, inp.h0, dout, dfin)]
    say("scan bwd determinism, 4 slices")
    g1 = M.selective_scan_bwd(*args)
    g2 = M.selective_scan_bwd(*args)
    torch.cuda.synchronize()
    for k in g1:
        if g1[k] is not None:
            assert torch.equal(g1[k], g2[k]), f"{k} differs between identical calls"


def test_scan_bwd_full_layer(M):
    """The 8 x 2048 x 1536 x 16 bf16 layer the backward benchmark times, every element checked."""
    cfg = W.CONFIGS[8]
    say("scan bwd full layer", cfg.name)
    g, ref = run_case(M, cfg, False, False, want_dh0=False)
    compare(g, ref, cfg.io, cfg.name)


def test_scan_bwd_full_layer_n128(M):
    """The same layer with 128 states per channel (eight slices), every element checked."""
    cfg = W.CONFIGS[16]
    say("scan bwd full layer", cfg.name)
    g, ref = run_case(M, cfg, False, False, want_dh0=False)
    compare(g, ref, cfg.io, cfg.name)
