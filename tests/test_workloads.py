"""Seeded input generators (no GPU)."""
import numpy as np
import torch

import workloads as W


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-8, 8, 100000),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.0e38, -1e-40], np.float32)])
    ours = W.f32_to_bf16_bits(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(W.bf16_bits_to_f32(ours), torch.from_numpy(v).to(torch.bfloat16).float().numpy())


def test_generator_deterministic_and_blocked():
    cfg = W.scan_config(2, 40, 5, 4, io=W.BF16)
    a = W.make_scan_inputs(cfg)
    b = W.make_scan_inputs(cfg)
    for k in ("x", "delta", "B", "C", "z", "D", "A"):
        assert np.array_equal(getattr(a, k), getattr(b, k))
    # a block boundary does not change earlier values
    n = W.BLOCK + 10
    assert np.array_equal(W.normal_f32(9, 0, n)[:1000], W.normal_f32(9, 0, 1000))


def test_delta_distribution():
    d = W.softplus_delta_f32(1, 1 << 20)
    assert d.dtype == np.float32 and np.all(d > 0)
    assert abs(float(d.mean()) - 0.14) < 0.005


def test_config_bytes():
    assert W.CONFIGS[2].algorithmic_bytes() == 202_479_616
    assert W.CONFIGS[1].algorithmic_bytes() == 299_264 + 4096
    assert W.CONFIGS[2].updates == 402_653_184


def test_exp_log_A_is_fp32_rounded():
    A = W.exp_log_A(2, 16)
    assert A.dtype == np.float32 and A.shape == (2, 16)
    assert A[0, 0] == -1.0 and A[0, 4] != -5.0   # -exp(log 5) in fp32 is not exactly -5


def test_mimo_inputs():
    cfg = W.ssd_config(2, 5, 3, 4, 6, 1, cfg_id=77, rank=3)
    s = W.make_ssd_inputs(cfg, with_D=True, with_z=True, with_h0=True)
    assert s.x.shape == (2, 5, 3, 3, 4) and s.z.shape == (2, 5, 3, 3, 4)
    assert s.B.shape == (2, 5, 1, 3, 6) and s.C.shape == (2, 5, 1, 3, 6)
    xp, bp = W.make_ssd_prev(cfg)
    assert xp.shape == (2, 3, 3, 4) and bp.shape == (2, 1, 3, 6)
    # rank 1 keeps the single-input shapes and values
    one = W.make_ssd_inputs(W.ssd_config(2, 5, 3, 4, 6, 1, cfg_id=77))
    assert one.x.shape == (2, 5, 3, 4)
    assert np.array_equal(one.x.reshape(-1), s.x.reshape(-1)[:one.x.size])
    m = W.CONFIGS[14]
    assert m.rank == 4 and m.algorithmic_bytes() > 4 * (W.CONFIGS[4].algorithmic_bytes() - 8 * 32 * 64 * 128 * 4) * 0.9
