"""The Python binding's argument checks (GPU tensors needed; every case raises before the C ABI is called,
so no kernel sees a bad argument)."""
import numpy as np
import pytest

import workloads as W
from gpu_util import dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import selective_state_space_17_amd as m
    return m


@pytest.fixture(scope="module")
def args():
    cfg = W.scan_config(2, 32, 64, 16, io="bf16", cfg_id=990)
    inp = W.make_scan_inputs(cfg)
    return [dev(a) for a in (inp.x, inp.delta, inp.A, inp.B, inp.C, inp.D, inp.z)]


def test_binding_accepts_good_arguments(M, args):
    import torch
    out = M.selective_scan_fwd(*args, stream=torch.cuda.current_stream())
    torch.cuda.synchronize()
    assert out.shape == args[0].shape and torch.isfinite(out.float()).all()


def test_binding_rejects_host_tensor(M, args):
    bad = list(args)
    bad[1] = bad[1].cpu()
    with pytest.raises(ValueError, match="GPU tensor"):
        M.selective_scan_fwd(*bad)


def test_binding_rejects_wrong_dtype(M, args):
    import torch
    bad = list(args)
    bad[3] = bad[3].to(torch.float32)
    with pytest.raises(TypeError):
        M.selective_scan_fwd(*bad)


def test_binding_rejects_noncontiguous(M, args):
    import torch
    bad = list(args)
    x = bad[0]
    bad[0] = torch.empty((x.shape[0], x.shape[1], 2 * x.shape[2]), dtype=x.dtype, device=x.device)[:, :, ::2]
    with pytest.raises(ValueError, match="contiguous"):
        M.selective_scan_fwd(*bad)


def test_binding_rejects_wrong_shape(M, args):
    bad = list(args)
    bad[5] = bad[5][:-1].contiguous()   # D one channel short
    with pytest.raises(ValueError, match="shape"):
        M.selective_scan_fwd(*bad)


def test_binding_requires_lam(M):
    cfg = W.ssd_config(1, 64, 2, 64, 64, 1, cfg_id=991)
    s = W.make_ssd_inputs(cfg)
    with pytest.raises(ValueError, match="lam"):
        M.ssd_trapezoidal_fwd(dev(s.x), dev(s.delta), None, dev(s.A), dev(s.B), dev(s.C))
