"""The entry points captured in a HIP graph (torch.cuda.graph) and replayed.

Serving loops capture the decode step to take launch overhead off the critical path. The library
enqueues only kernels on the stream it is given: no allocation, memset or synchronisation, and every
workspace element is written by a kernel before one reads it. So a captured call must replay exactly as
it runs eagerly. Each graph here is replayed several times, with eager work and synchronisations between
the replays, and every replay is compared bit for bit with the eager calls (the kernels are
deterministic)."""
import pytest

import workloads as W
from gpu_util import dev, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import selective_state_space_17_amd as m
    return m


def _capture(fn):
    """Warm fn up eagerly on a side stream, then capture one call of it."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn(warm=True)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn(warm=False)
    torch.cuda.synchronize()
    return g


def _eager_noise():
    """Unrelated eager work between replays, on the same stream."""
    import torch
    a = torch.randn(1 << 20, device="cuda")
    (a * 3).sum().item()
    torch.cuda.synchronize()


def test_graph_ssd_decode_steps(M):
    """A captured multi-head decode step replayed 4 times advances the state as 4 eager steps do."""
    import torch
    cfg = W.ssd_config(4, 1, 8, 64, 128, 1, io="bf16", cfg_id=7600)
    s = W.make_ssd_inputs(cfg, with_D=True, with_z=True, with_h0=True)
    ins = [dev(a) for a in (s.x, s.delta, s.A, s.B, s.C, s.D, s.z)]
    say("graph ssd decode")
    st_e, outs_e, states_e = dev(s.h0).clone(), [], []
    for _ in range(4):
        outs_e.append(M.ssd_state_update(st_e, *ins).clone())
        states_e.append(st_e.clone())
    st_g, out_g = dev(s.h0).clone(), torch.empty_like(outs_e[0])
    g = _capture(lambda warm: M.ssd_state_update(st_g.clone() if warm else st_g, *ins, out=out_g))
    assert torch.equal(st_g, dev(s.h0)), "capture must not run the step"
    for i in range(4):
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, outs_e[i]), f"replay {i}: out"
        assert torch.equal(st_g, states_e[i]), f"replay {i}: state"
        _eager_noise()


def test_graph_conv_decode_steps(M):
    """The Mamba-1 decode step with the convolution window: state and window both advance per replay."""
    import torch
    cfg = W.scan_config(8, 1, 256, 16, io="bf16", cfg_id=7610)
    inp = W.make_scan_inputs(cfg, with_h0=True)
    w, bias, init = W.make_conv_inputs(cfg, 4)
    ins = dict(xin=dev(inp.x), conv_w=dev(w), conv_b=dev(bias), delta=dev(inp.delta), A=dev(inp.A), B=dev(inp.B),
               C=dev(inp.C), D=dev(inp.D), z=dev(inp.z))
    say("graph conv decode")

    def step(state, cstate, out=None):
        return M.selective_state_update_conv(state, cstate, ins["xin"], ins["conv_w"], ins["conv_b"], ins["delta"],
                                             ins["A"], ins["B"], ins["C"], ins["D"], ins["z"], out=out)

    st_e, cs_e, ref = dev(inp.h0).clone(), dev(init).clone(), []
    for _ in range(3):
        o = step(st_e, cs_e).clone()
        ref.append((o, st_e.clone(), cs_e.clone()))
    st_g, cs_g = dev(inp.h0).clone(), dev(init).clone()
    out_g = torch.empty_like(ref[0][0])
    g = _capture(lambda warm: step(st_g.clone(), cs_g.clone(), out_g) if warm else step(st_g, cs_g, out_g))
    for i in range(3):
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, ref[i][0]) and torch.equal(st_g, ref[i][1]) and torch.equal(cs_g, ref[i][2]), \
            f"replay {i}"
        _eager_noise()


@pytest.mark.parametrize("split_seq", [1, 4])
def test_graph_scan_fwd(M, split_seq):
    """The Mamba-1 forward, single pass and split into 4 chunks (chunk, carry and fix-up kernels through
    the workspace), replays to the eager outputs."""
    import torch
    cfg = W.scan_config(2, 3000, 128, 16, io="bf16", cfg_id=7620)
    inp = W.make_scan_inputs(cfg, with_h0=True)
    args = [dev(a) for a in (inp.x, inp.delta, inp.A, inp.B, inp.C, inp.D, inp.z, inp.h0)]
    say("graph scan fwd", split_seq)
    ref_out, ref_fin = M.selective_scan_fwd(*args, return_final_state=True, split_seq=split_seq)
    out_g, fin_g = torch.empty_like(ref_out), torch.empty_like(ref_fin)
    ws = torch.empty(max(M.selective_scan_workspace_size(2, 3000, 128, 16, split_seq=split_seq), 1),
                     dtype=torch.uint8, device="cuda")
    g = _capture(lambda warm: M.selective_scan_fwd(*args, return_final_state=True, split_seq=split_seq,
                                                   out=out_g, final_state=fin_g, workspace=ws))
    for i in range(3):
        out_g.fill_(0)
        fin_g.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, ref_out) and torch.equal(fin_g, ref_fin), f"replay {i}"
        _eager_noise()


def test_graph_ssd_fwd(M):
    import torch
    cfg = W.ssd_config(2, 300, 4, 64, 128, 1, cfg_id=7630)
    s = W.make_ssd_inputs(cfg, with_D=True, with_z=True, with_h0=True)
    args = [dev(a) for a in (s.x, s.delta, s.A, s.B, s.C, s.D, s.z, s.h0)]
    say("graph ssd fwd")
    ref_out, ref_fin = M.ssd_fwd(*args, return_final_state=True)
    out_g, fin_g = torch.empty_like(ref_out), torch.empty_like(ref_fin)
    g = _capture(lambda warm: M.ssd_fwd(*args, return_final_state=True, out=out_g, final_state=fin_g))
    for i in range(3):
        out_g.fill_(0)
        fin_g.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, ref_out) and torch.equal(fin_g, ref_fin), f"replay {i}"
        _eager_noise()


def test_graph_scan_bwd(M):
    """The gradients (the gradient kernel and the two fixed-order sum kernels) replay to the eager result."""
    import torch
    cfg = W.scan_config(2, 500, 64, 16, io="bf16", cfg_id=7640)
    inp = W.make_scan_inputs(cfg, with_h0=True)
    dout, dfin = W.make_scan_grads(cfg)
    args = [dev(a) for a in (inp.x, inp.delta, inp.A, inp.B, inp.C, inp.D, inp.z, inp.h0, dout, dfin)]
    say("graph scan bwd")
    ref = M.selective_scan_bwd(*args)
    held = {}

    def run(warm):
        g = M.selective_scan_bwd(*args)
        if not warm:
            held.update(g)

    graph = _capture(run)
    for i in range(3):
        for t in held.values():
            if t is not None:
                t.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, t in ref.items():
            if t is not None:
                assert torch.equal(held[k], t), f"replay {i}: {k}"
        _eager_noise()
