"""Training mode on the GPU: the forward that stores the state entering every 16-step tile, and the
gradients started from those checkpoints, against the fp64 oracle.

Checkpoint k of (b, c, n) is h[n] before step 16k, i.e. the final state of the oracle run over the
first 16k steps; sampled tiles are checked that way, including sequences split into chunks (the
chunk pass writes zero-start states that the carry pass overwrites)."""
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


def ck_view(ck, b, L, dim):
    """[batch, tiles, dim, 16] view of a checkpoint array (channels padded to 16)."""
    d16 = (dim + 15) // 16 * 16
    return ck[: b * ((L + 15) // 16) * d16 * 16].view(b, (L + 15) // 16, d16, 16)[:, :, :dim, :]


# (batch, seqlen, dim, io, split_seq)
CASES = [
    (2, 100, 32, "f32", 0),
    (3, 257, 48, "bf16", 0),
    (1, 4096, 32, "bf16", 4),     # split into chunks: carried states overwrite the chunk pass's
    (2, 1000, 16, "f32", 3),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "b{}_l{}_d{}_{}_k{}".format(*c))
def test_fwd_ckpt(M, case):
    import torch
    b, l, d, io, k = case
    cfg = W.scan_config(b, l, d, 16, io=io, cfg_id=960 + l)
    inp = W.make_scan_inputs(cfg, with_h0=True)
    say("fwd ckpt", case)
    out, fin, ck = M.selective_scan_fwd_ckpt(dev(inp.x), dev(inp.delta), dev(inp.A), dev(inp.B), dev(inp.C),
                                             dev(inp.D), dev(inp.z), dev(inp.h0), return_final_state=True,
                                             split_seq=k)
    torch.cuda.synchronize()
    ref, ref_fin = oracle.scan_fwd(inp.x, inp.delta, inp.A, inp.B, inp.C, inp.D, inp.z, inp.h0)
    check(host64(out), ref, RTOL[io], f"{case} out")
    check(host64(fin), ref_fin, RTOL[io], f"{case} final")
    cv = ck_view(ck, b, l, d)
    nt = (l + 15) // 16
    for kt in sorted({0, 1, nt // 3, nt // 2, nt - 1}):
        L1 = 16 * kt
        if L1 == 0:
            want = inp.h0.astype(np.float64)
        else:
            _, want = oracle.scan_fwd(inp.x[:, :L1], inp.delta[:, :L1], inp.A, inp.B[:, :L1], inp.C[:, :L1],
                                      inp.D, inp.z[:, :L1], inp.h0)
        check(host64(cv[:, kt].contiguous()), want, RTOL[io], f"{case} checkpoint {kt}")


@pytest.mark.parametrize("case", [(2, 100, 40, "f32"), (3, 300, 64, "bf16")], ids=lambda c: "b{}_l{}_d{}_{}".format(*c))
def test_bwd_from_checkpoints(M, case):
    """Gradients started from the training forward's checkpoints match the oracle and the
    self-contained backward."""
    import torch
    b, l, d, io = case
    cfg = W.scan_config(b, l, d, 16, io=io, cfg_id=970 + l)
    inp = W.make_scan_inputs(cfg, with_h0=True)
    dout, dfin = W.make_scan_grads(cfg)
    args = [dev(a) for a in (inp.x, inp.delta, inp.A, inp.B, inp.C, inp.D, inp.z, inp.h0)]
    say("bwd from checkpoints", case)
    _, ck = M.selective_scan_fwd_ckpt(*args)
    g = M.selective_scan_bwd(*args, dev(dout), dev(dfin), checkpoints=ck)
    g0 = M.selective_scan_bwd(*args, dev(dout), dev(dfin))
    torch.cuda.synchronize()
    ref = oracle.scan_bwd(inp.x, inp.delta, inp.A, inp.B, inp.C, inp.D, inp.z, inp.h0, dout, dfin)
    for k in ref:
        if ref[k] is None:
            continue
        check(host64(g[k]), ref[k], RTOL[io], f"{case} {k} (checkpoints)")
        check(host64(g[k]), host64(g0[k]), 1e-5 if io == "f32" else 1e-2, f"{case} {k} vs own walk")


def test_training_step_full_layer(M):
    """The 8 x 2048 x 1536 bf16 layer: training forward, then gradients from its checkpoints."""
    import torch
    cfg = W.CONFIGS[8]
    inp = W.make_scan_inputs(cfg)
    dout, _ = W.make_scan_grads(cfg, with_dfinal=False)
    args = [dev(a) for a in (inp.x, inp.delta, inp.A, inp.B, inp.C, inp.D, inp.z)]
    say("training step full layer")
    out, ck = M.selective_scan_fwd_ckpt(*args)
    g = M.selective_scan_bwd(*args, None, dev(dout), None, want_dh0=False, checkpoints=ck)
    torch.cuda.synchronize()
    ref_out, _ = oracle.scan_fwd(inp.x, inp.delta, inp.A, inp.B, inp.C, inp.D, inp.z)
    check(host64(out), ref_out, RTOL[cfg.io], "training forward out")
    ref = oracle.scan_bwd(inp.x, inp.delta, inp.A, inp.B, inp.C, inp.D, inp.z, None, dout, None)
    for k in ("dx", "ddelta", "dz", "dB", "dC", "dA", "dD"):
        check(host64(g[k]), ref[k], RTOL[cfg.io], f"training step {k}")
