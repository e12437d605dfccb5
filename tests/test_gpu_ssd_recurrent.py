"""The SSD entry points on problems the matrix-core block kernel does not take (float32 I/O, headdim not a
multiple of 8, dstate not a multiple of 16): the library runs them through the recurrent update kernel, h0
in and final_state out, and the results must meet the same bar against the fp64 oracle."""
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


# (batch, seqlen, nheads, headdim, dstate, ngroups, io, D, z, h0, final_state)
CASES = [
    (2, 150, 4, 36, 64, 1, "bf16", True, True, True, True),      # headdim 36
    (1, 70, 2, 100, 128, 2, "bf16", False, True, False, True),   # headdim 100
    (2, 40, 2, 44, 256, 1, "bf16", True, False, True, True),     # dstate 256 (headdim 44)
    (1, 65, 3, 64, 20, 3, "bf16", True, True, True, False),      # dstate 20, no final state
    (2, 100, 4, 64, 128, 2, "f32", True, True, True, True),      # float32 I/O at the block kernel's shape
    (1, 33, 2, 7, 5, 1, "f32", False, False, False, True),       # odd sizes: the scalar state path
    (2, 0, 2, 16, 16, 1, "f32", True, True, True, True),         # no steps: final state = h0
    (1, 0, 2, 12, 16, 1, "bf16", False, False, False, True),     # no steps, no h0: final state = 0
]


def _run(M, case, trap):
    import torch
    b, l, h, p, n, g, io, hd, hz, hh, hf = case
    iod = M.MSSM_BF16 if io == "bf16" else M.MSSM_F32
    assert M.ssd_plan(b, l, h, p, n, g, io_dtype=iod) == M.SSD_ROUTE_RECURRENT, case
    cfg = W.ssd_config(b, l, h, p, n, g, io=io, cfg_id=7800 + l + p + n + (50 if trap else 0))
    s = W.make_ssd_inputs(cfg, with_D=hd, with_z=hz, with_h0=hh)
    lam = W.make_ssd_lam(cfg) if trap else None
    args = [dev(a) for a in (s.x, s.delta)]
    fin = torch.full((b, h, p, n), float("nan"), dtype=torch.float32, device="cuda") if hf else None
    tail = [dev(a) for a in (s.A, s.B, s.C, s.D, s.z, s.h0)]
    if trap:
        out = M.ssd_trapezoidal_fwd(*args, dev(lam), *tail, final_state=fin)
        ref, ref_fin = oracle.ssd3_fwd(s.x, s.delta, lam, s.A, s.B, s.C, s.D, s.z, s.h0)
    else:
        out = M.ssd_fwd(*args, *tail, final_state=fin)
        ref, ref_fin = oracle.ssd_fwd(s.x, s.delta, s.A, s.B, s.C, s.D, s.z, s.h0)
    torch.cuda.synchronize()
    if l > 0:
        check(host64(out), ref, RTOL[io], f"{case} out")
    if hf:
        if l == 0:   # nothing ran but the copy: exact
            want = s.h0 if hh else np.zeros((b, h, p, n), np.float32)
            assert np.array_equal(fin.cpu().numpy(), want), f"{case}: final state with no steps"
        else:
            check(host64(fin), ref_fin, RTOL[io], f"{case} final_state")


@pytest.mark.parametrize("case", CASES, ids=lambda c: "b{}_l{}_h{}_p{}_n{}_g{}_{}".format(*c[:7]))
def test_ssd_recurrent_route(M, case):
    say("ssd recurrent route", case)
    _run(M, case, trap=False)


@pytest.mark.parametrize("case", CASES[:6], ids=lambda c: "b{}_l{}_h{}_p{}_n{}_g{}_{}".format(*c[:7]))
def test_ssd_trapezoidal_recurrent_route(M, case):
    say("ssd trapezoidal recurrent route", case)
    _run(M, case, trap=True)


def test_ssd_recurrent_route_matches_update(M):
    """The routed sequence is the update entry point from h0, bit for bit (same kernel, same order)."""
    import torch
    assert M.ssd_plan(2, 50, 4, 36, 64, 2) == M.SSD_ROUTE_RECURRENT
    cfg = W.ssd_config(2, 50, 4, 36, 64, 2, io="bf16", cfg_id=7890)
    s = W.make_ssd_inputs(cfg, with_D=True, with_z=True, with_h0=True)
    ins = [dev(a) for a in (s.x, s.delta, s.A, s.B, s.C, s.D, s.z)]
    out, fin = M.ssd_fwd(*ins[:2], *ins[2:], dev(s.h0), return_final_state=True)
    st = dev(s.h0).clone()
    out2 = M.ssd_state_update(st, *ins)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(fin, st)
