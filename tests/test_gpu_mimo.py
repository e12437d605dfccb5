"""Mamba-3 MIMO on the GPU (mssm_ssd_mimo_fwd, mssm_ssd_mimo_state_update) against the fp64 oracle
(oracle_ssdm_fwd): R inputs and outputs per channel on one state per head."""
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


def inputs(cfg, **kw):
    """The workload's inputs with the rank axis present also at rank 1 (x, z [b, l, h, r, p]; B, C [b, l, g, r, n])."""
    s = W.make_ssd_inputs(cfg, **kw)
    if cfg.rank == 1:
        r = lambda a: None if a is None else np.ascontiguousarray(a[:, :, :, None])
        s = W.SSDInputs(r(s.x), s.delta, s.A, r(s.B), r(s.C), s.D, r(s.z), s.h0, s.io)
    return s


def run(M, s, lam, chunk=0):
    import torch
    out, fin = M.ssd_mimo_fwd(dev(s.x), dev(s.delta), dev(lam), dev(s.A), dev(s.B), dev(s.C), dev(s.D), dev(s.z),
                              dev(s.h0), chunk=chunk, return_final_state=True)
    torch.cuda.synchronize()
    return out, fin


def compare(M, cfg, s, lam, what, chunk=0):
    out, fin = run(M, s, lam, chunk)
    ref, ref_fin = oracle.ssdm_fwd(s.x, s.delta, lam, s.A, s.B, s.C, s.D, s.z, s.h0)
    st = check(host64(out), ref, RTOL[cfg.io], what + " out")
    check(host64(fin), ref_fin, RTOL[cfg.io], what + " final_state")
    return st


# (batch, seqlen, nheads, headdim, dstate, ngroups, rank, lam, D, z, h0): the block kernel (bf16, headdim a
# multiple of 8, dstate a multiple of 16 up to 128, rank a power of two up to 16) -- ragged lengths, one step
# across several blocks, padded states, groups, an odd unit count, headdim slices cut short
BLOCK = [
    (1, 16, 2, 64, 64, 1, 4, True, False, False, True),
    (2, 100, 4, 64, 128, 1, 4, True, True, True, True),
    (1, 33, 2, 64, 48, 2, 2, True, False, False, False),
    (2, 37, 2, 64, 64, 1, 8, False, True, False, True),
    (1, 9, 4, 128, 64, 2, 16, True, False, True, False),
    (1, 200, 3, 64, 32, 1, 4, True, True, False, True),
    (2, 130, 2, 64, 128, 1, 1, True, False, False, True),
    (1, 257, 4, 64, 128, 4, 2, False, False, False, False),
    (1, 60, 2, 48, 64, 1, 4, True, True, True, True),
    (2, 40, 3, 96, 32, 1, 2, False, True, False, True),
]


@pytest.mark.parametrize("case", BLOCK, ids=lambda c: "b{}_l{}_h{}_p{}_n{}_g{}_r{}".format(*c[:7]))
def test_mimo_block(M, case):
    b, l, h, p, n, g, r, wl, hd, hz, hh = case
    assert M.ssd_mimo_plan(b, l, h, p, n, g, r) == M.SSD_ROUTE_BLOCK
    cfg = W.ssd_config(b, l, h, p, n, g, cfg_id=1500 + l + n + r, rank=r)
    s = inputs(cfg, with_D=hd, with_z=hz, with_h0=hh)
    lam = W.make_ssd_lam(cfg) if wl else None
    say("mimo block", case)
    compare(M, cfg, s, lam, f"mimo {case}")


@pytest.mark.parametrize("chunk", [64, 128, 256])
def test_mimo_chunk_argument(M, chunk):
    cfg = W.ssd_config(1, 300, 2, 64, 64, 1, cfg_id=1560, rank=4)
    s = W.make_ssd_inputs(cfg, with_h0=True)
    compare(M, cfg, s, W.make_ssd_lam(cfg), f"mimo chunk {chunk}", chunk=chunk)


def test_mimo_rank_one_is_siso(M):
    """Rank 1 on the block kernel equals the single-input entry points bit for bit (one kernel, one row per step)."""
    import torch
    cfg = W.ssd_config(2, 150, 4, 64, 64, 2, cfg_id=1561)
    s = W.make_ssd_inputs(cfg, with_D=True, with_z=True, with_h0=True)
    lam = W.make_ssd_lam(cfg)
    x5 = lambda a: None if a is None else dev(a)[:, :, :, None, :].contiguous()
    b5 = lambda a: dev(a)[:, :, :, None, :].contiguous()
    o1, f1 = M.ssd_mimo_fwd(x5(s.x), dev(s.delta), dev(lam), dev(s.A), b5(s.B), b5(s.C), dev(s.D), x5(s.z),
                            dev(s.h0), return_final_state=True)
    o2, f2 = M.ssd_trapezoidal_fwd(dev(s.x), dev(s.delta), dev(lam), dev(s.A), dev(s.B), dev(s.C), dev(s.D),
                                   dev(s.z), dev(s.h0), return_final_state=True)
    o3, f3 = M.ssd_mimo_fwd(x5(s.x), dev(s.delta), None, dev(s.A), b5(s.B), b5(s.C), dev(s.D), x5(s.z), dev(s.h0),
                            return_final_state=True)
    o4, f4 = M.ssd_fwd(dev(s.x), dev(s.delta), dev(s.A), dev(s.B), dev(s.C), dev(s.D), dev(s.z), dev(s.h0),
                       return_final_state=True)
    torch.cuda.synchronize()
    assert torch.equal(o1[:, :, :, 0].view(torch.int16), o2.view(torch.int16)) and torch.equal(f1, f2)
    assert torch.equal(o3[:, :, :, 0].view(torch.int16), o4.view(torch.int16)) and torch.equal(f3, f4)


# the recurrent route: fp32, ranks the block kernel does not take, other headdims and state sizes
RECURRENT = [
    (2, 40, 3, 24, 20, 1, 3, "f32", True),
    (1, 25, 2, 64, 64, 1, 4, "f32", False),
    (2, 30, 4, 16, 256, 2, 2, "bf16", True),
    (1, 50, 2, 64, 128, 1, 5, "bf16", True),
    (1, 17, 2, 7, 9, 2, 32, "f32", False),
]


@pytest.mark.parametrize("case", RECURRENT, ids=lambda c: "b{}_l{}_h{}_p{}_n{}_g{}_r{}_{}".format(*c[:8]))
def test_mimo_recurrent(M, case):
    b, l, h, p, n, g, r, io, wl = case
    assert M.ssd_mimo_plan(b, l, h, p, n, g, r, io_dtype=M.MSSM_BF16 if io == "bf16" else M.MSSM_F32) == \
        M.SSD_ROUTE_RECURRENT
    cfg = W.ssd_config(b, l, h, p, n, g, io=io, cfg_id=1600 + l + r, rank=r)
    s = W.make_ssd_inputs(cfg, with_D=True, with_z=True, with_h0=True)
    lam = W.make_ssd_lam(cfg) if wl else None
    say("mimo recurrent", case)
    compare(M, cfg, s, lam, f"mimo recurrent {case}")


@pytest.mark.parametrize("case", [(2, 9, 4, 64, 128, 1, 4, "bf16"), (3, 6, 2, 24, 20, 2, 3, "f32"),
                                  (1, 5, 2, 64, 64, 1, 16, "bf16")])
@pytest.mark.parametrize("wl", [True, False])
def test_mimo_decode_token_by_token(M, case, wl):
    """Stepping one token at a time, each step given the previous token's rank inputs and B rows, reproduces
    the sequence oracle's outputs and final state."""
    import torch
    b, l, h, p, n, g, r, io = case
    cfg = W.ssd_config(b, l, h, p, n, g, io=io, cfg_id=1700 + l + r, rank=r)
    s = W.make_ssd_inputs(cfg, with_D=True, with_z=True, with_h0=True)
    lam = W.make_ssd_lam(cfg) if wl else None
    ref, ref_fin = oracle.ssdm_fwd(s.x, s.delta, lam, s.A, s.B, s.C, s.D, s.z, s.h0)
    state = dev(s.h0).clone()
    outs = []
    for t in range(l):
        sl = lambda a: None if a is None else dev(np.ascontiguousarray(a[:, t:t + 1]))
        xp = dev(np.ascontiguousarray(s.x[:, t - 1])) if t > 0 else None
        bp = dev(np.ascontiguousarray(s.B[:, t - 1])) if t > 0 else None
        outs.append(M.ssd_mimo_state_update(state, sl(s.x), sl(s.delta), sl(lam), dev(s.A), sl(s.B), sl(s.C),
                                            dev(s.D), sl(s.z), x_prev=xp, B_prev=bp))
    torch.cuda.synchronize()
    got = np.concatenate([host64(o) for o in outs], axis=1)
    check(got, ref, RTOL[io], "mimo decode out")
    check(host64(state), ref_fin, RTOL[io], "mimo decode state")


def test_mimo_full_layer(M):
    """The 8 x 4096 x 32-head x 4-rank x 64 x 128 workload the benchmark times: every element."""
    cfg = W.CONFIGS[14]
    s = W.make_ssd_inputs(cfg)
    lam = W.make_ssd_lam(cfg)
    say("mimo full layer", cfg.name)
    st = compare(M, cfg, s, lam, cfg.name, chunk=cfg.chunk)
    say(cfg.name, st)


def test_mimo_decode_workload(M):
    """The MIMO decode workload the benchmark times (64 x 32 heads x 64 x 128, rank 4, one token, previous
    token given): every element of the output and the state."""
    import torch
    cfg = W.CONFIGS[15]
    s = W.make_ssd_inputs(cfg, with_h0=True)
    lam = W.make_ssd_lam(cfg)
    xp, bp = W.make_ssd_prev(cfg)
    ref, ref_fin = oracle.ssdm_fwd(s.x, s.delta, lam, s.A, s.B, s.C, s.D, s.z, s.h0, xp, bp)
    state = dev(s.h0).clone()
    out = M.ssd_mimo_state_update(state, dev(s.x), dev(s.delta), dev(lam), dev(s.A), dev(s.B), dev(s.C), dev(s.D),
                                  dev(s.z), x_prev=dev(xp), B_prev=dev(bp))
    torch.cuda.synchronize()
    check(host64(out), ref, RTOL["bf16"], "mimo decode workload out")
    check(host64(state), ref_fin, RTOL["bf16"], "mimo decode workload state")
