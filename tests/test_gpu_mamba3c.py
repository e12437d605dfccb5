"""Mamba-3 SISO recurrence with a complex-valued state on the GPU (mssm_mamba3_siso_update, through the C
ABI) against the fp64 oracle written in complex arithmetic (oracle.ssdc_fwd).

The update kernel keeps the state in its own frame and rotates each state pair by delta * omega per step.
Cases: whole sequences in one call (the recurrent sequence form), token by token with the previous
token passed along, a given previous token, fp32 and bf16, 8 and 4 states per lane and the scalar path,
omega = 0 against the real trapezoidal update bit for bit, rotation rates large enough that one step
turns a pair by hundreds of radians, and the decode workload the benchmark times."""
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


def inputs(case, cfg_id):
    b, l, h, p, n, g, io, hd, hz = case
    cfg = W.ssd_config(b, l, h, p, n, g, io=io, cfg_id=cfg_id)
    s = W.make_ssd_inputs(cfg, with_D=hd, with_z=hz, with_h0=True)
    return cfg, s, W.make_ssd_lam(cfg), W.make_ssd_omega(cfg)


# (batch, tokens, nheads, headdim, dstate, ngroups, io, D, z)
CASES = [
    (2, 200, 4, 64, 128, 1, "bf16", True, True),   # 8 states (4 pairs) per lane
    (3, 57, 4, 32, 64, 2, "f32", True, False),
    (1, 90, 2, 16, 20, 1, "bf16", False, True),    # 4 states per lane
    (2, 40, 6, 8, 6, 3, "f32", False, False),      # dstate 6: the scalar path, pairs inside a lane
    (1, 1, 2, 64, 256, 2, "bf16", True, True),     # one token, the largest dstate
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "b{}_l{}_h{}_p{}_n{}_g{}_{}".format(*c[:7]))
def test_mamba3_complex_sequence(M, case):
    """All tokens in one call from h0: the recurrent sequence form."""
    import torch
    cfg, s, lam, om = inputs(case, 1400 + case[1] + case[4])
    say("mamba3 complex sequence", case)
    ref, ref_fin = oracle.ssdc_fwd(s.x, s.delta, lam, s.A, om, s.B, s.C, s.D, s.z, s.h0)
    state = dev(s.h0).clone()
    out = M.mamba3_siso_update(state, dev(s.x), dev(s.delta), dev(lam), dev(s.A), dev(om), dev(s.B), dev(s.C),
                               dev(s.D), dev(s.z))
    torch.cuda.synchronize()
    check(host64(out), ref, RTOL[case[6]], f"{case} out")
    check(host64(state), ref_fin, RTOL[case[6]], f"{case} state")


@pytest.mark.parametrize("case", [CASES[0], CASES[3]], ids=["n128_bf16", "n6_f32"])
def test_mamba3_complex_token_by_token(M, case):
    """One token per call, each given the previous token's x and B, reproduces the sequence oracle."""
    import torch
    cfg, s, lam, om = inputs(case, 1450 + case[4])
    l = min(case[1], 40)
    sl = lambda a: None if a is None else a[:, :l]
    ref, ref_fin = oracle.ssdc_fwd(sl(s.x), sl(s.delta), sl(lam), s.A, om, sl(s.B), sl(s.C), s.D, sl(s.z), s.h0)
    x, dl, lm, Bm, Cm, z = (dev(a) for a in (s.x, s.delta, lam, s.B, s.C, s.z))
    state = dev(s.h0).clone()
    outs = []
    for t in range(l):
        one = lambda v: None if v is None else v[:, t:t + 1].contiguous()
        outs.append(M.mamba3_siso_update(state, one(x), one(dl), one(lm), dev(s.A), dev(om), one(Bm), one(Cm),
                                         dev(s.D), one(z), x_prev=x[:, t - 1].contiguous() if t else None,
                                         B_prev=Bm[:, t - 1].contiguous() if t else None))
    torch.cuda.synchronize()
    got = np.concatenate([host64(o) for o in outs], axis=1)
    check(got, ref, RTOL[case[6]], f"{case} token by token out")
    check(host64(state), ref_fin, RTOL[case[6]], f"{case} token by token state")


def test_mamba3_complex_given_previous_token(M):
    """Several tokens from a stored state and a given previous token, against the oracle's own
    previous-token inputs."""
    import torch
    case = (2, 7, 4, 64, 64, 2, "bf16", True, True)
    cfg, s, lam, om = inputs(case, 1460)
    xp, bp = W.make_ssd_prev(cfg)
    ref, ref_fin = oracle.ssdc_fwd(s.x, s.delta, lam, s.A, om, s.B, s.C, s.D, s.z, s.h0, xp, bp)
    state = dev(s.h0).clone()
    out = M.mamba3_siso_update(state, dev(s.x), dev(s.delta), dev(lam), dev(s.A), dev(om), dev(s.B), dev(s.C),
                               dev(s.D), dev(s.z), x_prev=dev(xp), B_prev=dev(bp))
    torch.cuda.synchronize()
    check(host64(out), ref, RTOL["bf16"], "given previous token out")
    check(host64(state), ref_fin, RTOL["bf16"], "given previous token state")


def test_mamba3_complex_omega_zero_is_real_bitwise(M):
    """omega = 0: cos = 1 and sin = 0 exactly, so the rotation is the identity and the result equals
    the real trapezoidal update bit for bit."""
    import torch
    case = (2, 5, 4, 64, 128, 1, "bf16", True, True)
    cfg, s, lam, om = inputs(case, 1461)
    xp, bp = W.make_ssd_prev(cfg)
    st_c, st_r = dev(s.h0).clone(), dev(s.h0).clone()
    args = [dev(a) for a in (s.x, s.delta, lam)]
    oc = M.mamba3_siso_update(st_c, *args, dev(s.A), dev(np.zeros_like(om)), dev(s.B), dev(s.C), dev(s.D),
                              dev(s.z), x_prev=dev(xp), B_prev=dev(bp))
    orl = M.ssd_trapezoidal_state_update(st_r, *args, dev(s.A), dev(s.B), dev(s.C), dev(s.D), dev(s.z),
                                         x_prev=dev(xp), B_prev=dev(bp))
    torch.cuda.synchronize()
    assert torch.equal(oc, orl) and torch.equal(st_c, st_r)


def test_mamba3_complex_decode_config_full(M):
    """The decode workload the benchmark times (64 x 32 heads x 64 x 128, one token, previous token
    given, complex state), every element."""
    import torch
    cfg = W.CONFIGS[13]
    s = W.make_ssd_inputs(cfg, with_h0=True)
    lam, om = W.make_ssd_lam(cfg), W.make_ssd_omega(cfg)
    xp, bp = W.make_ssd_prev(cfg)
    say("mamba3 complex decode config", cfg.name)
    ref, ref_fin = oracle.ssdc_fwd(s.x, s.delta, lam, s.A, om, s.B, s.C, s.D, s.z, s.h0, xp, bp)
    state = dev(s.h0).clone()
    out = M.mamba3_siso_update(state, dev(s.x), dev(s.delta), dev(lam), dev(s.A), dev(om), dev(s.B), dev(s.C),
                               dev(s.D), dev(s.z), x_prev=dev(xp), B_prev=dev(bp))
    torch.cuda.synchronize()
    check(host64(out), ref, RTOL["bf16"], f"{cfg.name} out")
    check(host64(state), ref_fin, RTOL["bf16"], f"{cfg.name} state")


def test_mamba3_complex_large_angles(M):
    """Rotation rates up to 300 per unit delta, so each step turns a pair by tens to hundreds of radians.
    The angle reaches the hardware sine and cosine after reduction to revolutions, whose error grows
    like |angle| * 2^-24 revolutions; at the bf16 bar the results still agree with the oracle's exact
    complex exponential."""
    import torch
    case = (2, 120, 4, 32, 32, 1, "bf16", True, True)
    cfg, s, lam, om = inputs(case, 1470)
    om = (om * (300.0 / np.pi)).astype(np.float32)
    say("mamba3 complex large angles")
    ref, ref_fin = oracle.ssdc_fwd(s.x, s.delta, lam, s.A, om, s.B, s.C, s.D, s.z, s.h0)
    state = dev(s.h0).clone()
    out = M.mamba3_siso_update(state, dev(s.x), dev(s.delta), dev(lam), dev(s.A), dev(om), dev(s.B), dev(s.C),
                               dev(s.D), dev(s.z))
    torch.cuda.synchronize()
    check(host64(out), ref, RTOL["bf16"], "large angles out")
    check(host64(state), ref_fin, RTOL["bf16"], "large angles state")
