"""Mamba-2 scalar-A multi-head form on the GPU (through the C ABI) against the fp64 oracle."""
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


def run_gpu(M, s, chunk=0):
    import torch
    out, fin = M.ssd_fwd(dev(s.x), dev(s.delta), dev(s.A), dev(s.B), dev(s.C), dev(s.D), dev(s.z), dev(s.h0),
                         chunk=chunk, return_final_state=True)
    torch.cuda.synchronize()
    return out, fin


def compare(M, s, what, hd0=0, hd1=None, chunk=0):
    out, fin = run_gpu(M, s, chunk)
    ref, ref_fin = oracle.ssd_fwd(s.x, s.delta, s.A, s.B, s.C, s.D, s.z, s.h0, hd0=hd0, hd1=hd1)
    hd1 = s.x.shape[2] if hd1 is None else hd1
    st = check(host64(out[:, :, hd0:hd1].contiguous()), ref, RTOL["bf16"], what + " out")
    check(host64(fin[:, hd0:hd1].contiguous()), ref_fin, RTOL["bf16"], what + " final_state")
    return st


# (batch, seqlen, nheads, headdim, dstate, ngroups, D, z, h0)
CASES = [
    (1, 1, 2, 64, 16, 1, False, False, False),
    (2, 63, 4, 64, 32, 2, True, True, True),
    (1, 64, 2, 64, 64, 1, True, False, True),
    (2, 65, 4, 128, 64, 4, False, True, False),
    (1, 200, 6, 64, 128, 3, True, True, True),
    (2, 1000, 4, 64, 48, 1, True, True, True),
    (1, 777, 2, 192, 80, 2, False, False, True),
    (2, 300, 4, 64, 112, 2, True, True, False),
    # more than 128 states: two shares of the states, added with D x and the gate by a third kernel
    (2, 200, 4, 64, 256, 1, True, True, True),
    (1, 130, 2, 128, 144, 2, False, True, False),   # a second share of 16 states
    (2, 65, 3, 64, 192, 3, True, False, True),
    (1, 1, 2, 64, 256, 1, True, True, True),
    # headdims that are multiples of 8: the last 64-wide slice is cut at headdim
    (2, 150, 4, 96, 64, 2, True, True, True),      # second slice of 32 columns
    (1, 70, 3, 24, 128, 1, True, True, True),      # one slice of 24: a state wave with half its lanes
    (2, 65, 2, 8, 32, 1, False, True, True),       # 8 columns
    (1, 300, 2, 136, 48, 2, True, False, True),    # third slice of 8 columns
    (2, 100, 2, 40, 256, 1, True, True, True),     # a cut slice with two shares of the states
    (2, 0, 2, 16, 32, 1, True, True, True),        # no steps: the final state is h0
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "b{}_l{}_h{}_p{}_n{}_g{}".format(*c[:6]))
def test_ssd_sweep(M, case):
    b, l, h, p, n, g, hd, hz, hh = case
    cfg = W.ssd_config(b, l, h, p, n, g, cfg_id=500 + l + n)
    s = W.make_ssd_inputs(cfg, with_D=hd, with_z=hz, with_h0=hh)
    say("ssd sweep", case)
    compare(M, s, f"ssd {case}")


@pytest.mark.parametrize("chunk", [0, 64, 128, 256])
def test_ssd_chunk_argument(M, chunk):
    cfg = W.ssd_config(2, 700, 4, 64, 64, 1, cfg_id=601)
    s = W.make_ssd_inputs(cfg, with_D=True, with_z=True, with_h0=True)
    compare(M, s, f"chunk={chunk}", chunk=chunk)


@pytest.mark.parametrize("dstate", [64, 256])
def test_ssd_delta_zero_keeps_state(M, dstate):
    cfg = W.ssd_config(1, 300, 2, 64, dstate, 1, cfg_id=602 + dstate)
    s = W.make_ssd_inputs(cfg, with_h0=True)
    s.delta[:] = 0
    _, fin = run_gpu(M, s)
    assert np.array_equal(fin.cpu().numpy(), s.h0), "delta=0 must keep the state bitwise"


def test_ssd_chaining(M):
    import torch
    cfg = W.ssd_config(2, 500, 4, 64, 64, 2, cfg_id=603)
    s = W.make_ssd_inputs(cfg, with_D=True, with_z=True)
    full, fin = run_gpu(M, s)
    L1 = 192
    a = W.SSDInputs(s.x[:, :L1], s.delta[:, :L1], s.A, s.B[:, :L1], s.C[:, :L1], s.D, s.z[:, :L1], None, "bf16")
    _, mid = run_gpu(M, a)
    bb = W.SSDInputs(s.x[:, L1:], s.delta[:, L1:], s.A, s.B[:, L1:], s.C[:, L1:], s.D, s.z[:, L1:],
                     mid.cpu().numpy(), "bf16")
    tail, fin2 = run_gpu(M, bb)
    check(host64(tail), host64(full)[:, L1:], 2e-2, "ssd chained tail")
    check(host64(fin2), host64(fin), 2e-2, "ssd chained final")


def test_ssd_matches_broadcast_scan_on_gpu(M):
    # the two GPU paths agree where the forms coincide (scalar A broadcast over a head's channels)
    cfg = W.ssd_config(1, 400, 2, 64, 16, 1, cfg_id=604)
    s = W.make_ssd_inputs(cfg, with_D=True, with_z=True, with_h0=True)
    out, fin = run_gpu(M, s)
    b, l, h, p = s.x.shape
    xe = np.ascontiguousarray(s.x.reshape(b, l, h * p))
    de = np.ascontiguousarray(np.repeat(s.delta, p, axis=2))
    Ae = np.ascontiguousarray(np.repeat(np.repeat(s.A, p)[:, None], 16, axis=1))
    De = np.repeat(s.D, p)
    ze = np.ascontiguousarray(s.z.reshape(b, l, h * p))
    h0e = np.ascontiguousarray(s.h0.reshape(b, h * p, 16))
    o2, f2 = M.selective_scan_fwd(dev(xe), dev(de), dev(Ae), dev(s.B[:, :, 0]), dev(s.C[:, :, 0]), dev(De), dev(ze),
                                  dev(h0e), return_final_state=True)
    check(host64(out).reshape(b, l, h * p), host64(o2), 2e-2, "ssd vs scan out")
    check(host64(fin).reshape(b, h * p, 16), host64(f2), 2e-2, "ssd vs scan final")


def test_config4_full(M):
    """The 8 x 4096 x 32-head x 64 x 128 workload the benchmark times: every output and final-state element
    against the oracle."""
    cfg = W.CONFIGS[4]
    say("config", cfg.name)
    s = W.make_ssd_inputs(cfg)
    out, fin = run_gpu(M, s, chunk=cfg.chunk)
    ref, ref_fin = oracle.ssd_fwd(s.x, s.delta, s.A, s.B, s.C, None, None, None)
    st = check(host64(out), ref, RTOL["bf16"], "config4 out")
    check(host64(fin), ref_fin, RTOL["bf16"], "config4 final")
    say("config4", st)


@pytest.mark.parametrize("dstate", [48, 80, 208])
def test_ssd_padded_states_ignore_stale_lds(M, dstate):
    """dstate 48, 80 or 208 (padded to 64 or 128 inside, 208 as shares of 128 and 80): state rows past
    dstate must not pick up whatever an earlier kernel left in LDS.  A forward scan over NaN inputs first
    leaves NaNs in the LDS of every CU."""
    import torch
    big = W.scan_config(8, 512, 1536, 16, io="bf16", cfg_id=610)
    poison = W.make_scan_inputs(big)
    nan_x = torch.full((8, 512, 1536), float("nan"), dtype=torch.bfloat16, device="cuda")
    M.selective_scan_fwd(nan_x, dev(poison.delta), dev(poison.A), dev(poison.B), dev(poison.C), dev(poison.D),
                         dev(poison.z), split_state=16)
    torch.cuda.synchronize()
    cfg = W.ssd_config(2, 1000, 4, 64, dstate, 1, cfg_id=611 + dstate)
    s = W.make_ssd_inputs(cfg, with_D=True, with_z=True, with_h0=True)
    compare(M, s, f"ssd dstate {dstate} after NaN in LDS")


def test_config17_full(M):
    """Config 4's shape with 256 states (two shares of the states): every output and final-state element
    against the oracle."""
    cfg = W.CONFIGS[17]
    say("config", cfg.name)
    s = W.make_ssd_inputs(cfg)
    out, fin = run_gpu(M, s, chunk=cfg.chunk)
    ref, ref_fin = oracle.ssd_fwd(s.x, s.delta, s.A, s.B, s.C, None, None, None)
    st = check(host64(out), ref, RTOL["bf16"], "config17 out")
    check(host64(fin), ref_fin, RTOL["bf16"], "config17 final")
    say("config17", st)
