"""The CPU oracle against what the pages and the mathematics fix (no GPU)."""
import os
import subprocess
import tempfile

import pytest

import oracle
import pins

ORACLE_SRC = os.path.join(os.path.dirname(oracle.__file__), "mssm_oracle.c")


@pytest.fixture(scope="module")
def lib():
    return oracle.load_library()


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(lib, pin):
    pin(lib)


# Plausible mistakes, planted in a copy of the oracle source on the CPU.
# Each one must make at least one pin fail.
MUTANTS = {
    "decay_sign": ("exp(d * (double)j->A[c * N + n])", "exp(-d * (double)j->A[c * N + n])"),
    "decay_without_delta": ("exp(d * (double)j->A[c * N + n])", "exp((double)j->A[c * N + n])"),
    "input_without_delta": ("const double dBx = d * load_io(j->Bm", "const double dBx = load_io(j->Bm"),
    "A_transposed": ("j->A[c * N + n]", "j->A[(n * D + c) % (D * N)]"),
    "readout_before_update": (
        "h[n] = dA * h[n] + dBx;\n            acc += load_io(j->Cm, j->io, r + n) * h[n];",
        "acc += load_io(j->Cm, j->io, r + n) * h[n];\n            h[n] = dA * h[n] + dBx;"),
    "B_for_C": ("acc += load_io(j->Cm, j->io, r + n) * h[n];", "acc += load_io(j->Bm, j->io, r + n) * h[n];"),
    "skip_dropped": ("(j->Dv ? (double)j->Dv[c] * u : 0.0)", "0.0"),
    "gate_sigmoid_not_silu": ("return v / (1.0 + exp(-v));", "return 1.0 / (1.0 + exp(-v));"),
    "h0_ignored": ("j->h0 ? (double)j->h0[(b * D + c) * N + n] : 0.0", "0.0"),
    "bf16_halfulp": ("uint32_t u = ((uint32_t)bits) << 16;", "uint32_t u = (((uint32_t)bits) << 16) | 0x8000u;"),
    "C_index_off_by_one_t": ("const int64_t r = (b * L + t) * N;", "const int64_t r = (b * L + (t > 0 ? t - 1 : 0)) * N;"),
    "ssd_group_index": ("const int64_t g = hd / (H / G);", "const int64_t g = hd % G;"),
    "ssd_decay_sign": ("exp(d * (double)j->A[hd])", "exp(-d * (double)j->A[hd])"),
    "ssd_input_without_delta": ("a * S[p * N + n] + d * load_io(j->Bm", "a * S[p * N + n] + load_io(j->Bm"),
    "ssd_h0_layout": ("j->h0[((b * H + hd) * P + p) * N + n]", "j->h0[((b * H + hd) * N + (n % P)) * P + (p % N)]"),
    "ssd_skip_dropped": ("(j->Dv ? (double)j->Dv[hd] * u : 0.0)", "0.0"),
    # Mamba-3 exponential-trapezoidal rule
    "ssd3_left_without_decay": ("w_left = (1.0 - lam) * d * a,", "w_left = (1.0 - lam) * d,"),
    "ssd3_weights_swapped": ("w_left = (1.0 - lam) * d * a, w_right = lam * d;",
                             "w_left = lam * d * a, w_right = (1.0 - lam) * d;"),
    "ssd3_left_uses_current_input": (
        "S[p * N + n] = a * S[p * N + n] + w_left * bx_prev[p * N + n] + w_right * bx;\n                bx_prev[p * N + n] = bx;",
        "bx_prev[p * N + n] = bx;\n                S[p * N + n] = a * S[p * N + n] + w_left * bx_prev[p * N + n] + w_right * bx;"),
    "ssd3_left_without_delta": ("w_left = (1.0 - lam) * d * a,", "w_left = (1.0 - lam) * a,"),
    "ssd3_prev_input_not_reset": ("bx_prev[p * N + n] = 0.0;                           /* B_{-1} x_{-1} */", ";"),
    # Mamba-3 complex-valued state
    "ssdc_rotation_sign": ("(double)j->A[hd] + I * (double)j->omega[hd * K + k]",
                           "(double)j->A[hd] - I * (double)j->omega[hd * K + k]"),
    "ssdc_readout_without_conj": ("acc += creal(conj(ck) * S[p * K + k]);", "acc += creal(ck * S[p * K + k]);"),
    "ssdc_one_rate_per_head": ("(double)j->omega[hd * K + k]", "(double)j->omega[hd * K]"),
    "ssdc_left_end_not_rotated": ("(1.0 - lam) * d * a * bx_prev[p * K + k]",
                                  "(1.0 - lam) * d * cabs(a) * bx_prev[p * K + k]"),
    "ssdc_previous_token_ignored": ("if (j->x_prev && j->B_prev) {", "if (0) {"),
    # Mamba-3 MIMO
    "ssdm_readout_rank0_C": ("acc += load_io(j->Cm, j->io, (bc + r) * N + n) * S[p * N + n];",
                             "acc += load_io(j->Cm, j->io, bc * N + n) * S[p * N + n];"),
    "ssdm_first_input_only": ("for (int64_t r = 0; r < R; ++r)\n                    u += load_io(j->Bm",
                              "for (int64_t r = 0; r < 1; ++r)\n                    u += load_io(j->Bm"),
    "ssdm_B_rank_reversed": ("u += load_io(j->Bm, j->io, (bc + r) * N + n) * load_io(j->x, j->io, (xr + r) * P + p);",
                             "u += load_io(j->Bm, j->io, (bc + R - 1 - r) * N + n) * load_io(j->x, j->io, (xr + r) * P + p);"),
    "ssdm_default_lam_half": ("? load_io(j->lam, j->io, (b * L + t) * H + hd) : 1.0;",
                              "? load_io(j->lam, j->io, (b * L + t) * H + hd) : 0.5;"),
    "ssdm_previous_token_rank0": ("for (int64_t r = 0; r < R; ++r)\n                    u += load_io(j->B_prev",
                                  "for (int64_t r = 0; r < 1; ++r)\n                    u += load_io(j->B_prev"),
    "ssdm_skip_rank0_x": ("double y = acc + (j->Dv ? (double)j->Dv[hd] * load_io(j->x, j->io, i) : 0.0);",
                          "double y = acc + (j->Dv ? (double)j->Dv[hd] * load_io(j->x, j->io, xr * P + p) : 0.0);"),
    "ssdm_left_end_current": ("S[p * N + n] = a * S[p * N + n] + w_left * U_prev[p * N + n] + w_right * u;",
                              "S[p * N + n] = a * S[p * N + n] + w_left * u + w_right * u;"),
    # gradients
    "bwd_no_adjoint_decay": ("lam[n] *= a;", ";"),
    "bwd_dsilu_is_sigmoid": ("return s * (1.0 + v * (1.0 - s));", "return s;"),
    "bwd_dB_without_delta": ("j->dB[r + n] += lam[n] * d * u;", "j->dB[r + n] += lam[n] * u;"),
    "bwd_dC_previous_state": ("j->dC[r + n] += dy * h;", "j->dC[r + n] += dy * hprev;"),
    "bwd_adjoint_from_B": ("lam[n] += Cn * dy;", "lam[n] += Bn * dy;"),
    "bwd_ddelta_without_A": ("hprev * a * An", "hprev * a"),
    "bwd_dA_without_delta": ("lam[n] * hprev * a * d;", "lam[n] * hprev * a;"),
    "bwd_gate_sees_no_skip": ("ys[t] = acc + ", "ys[t] = acc + 0.0 * "),
    "bwd_dx_skip_dropped": ("du = dy * (double)j->Dv[c];", "du = 0.0;"),
    "bwd_dD_ungated": ("j->dD[c] += dy * u;", "j->dD[c] += g * u;"),
    "bwd_dx_without_delta": ("du += lam[n] * d * Bn;", "du += lam[n] * Bn;"),
    "bwd_dfinal_ignored": ("j->dfinal ? (double)j->dfinal[(b * D + c) * N + n] : 0.0", "0.0"),
    # short convolution front end
    "conv_taps_reversed": ("acc += (double)w[c * W + k] * v;", "acc += (double)w[c * W + (W - 1 - k)] * v;"),
    "conv_init_ignored": ("else if (init)", "else if (0)"),
    "conv_init_newest_first": ("load_io(init, io, (b * (W - 1) + (W - 1) + s) * D + c)",
                               "load_io(init, io, (b * (W - 1) + (-1 - s)) * D + c)"),
    "conv_bias_dropped": ("double acc = bias ? (double)bias[c] : 0.0;", "double acc = 0.0;"),
    "conv_no_silu": ("x[(b * L + t) * D + c] = silu(acc);", "x[(b * L + t) * D + c] = acc;"),
    "conv_not_causal": ("const int64_t s = t - (W - 1) + k;", "const int64_t s = t + k;"),
    "conv_skip_dropped": ("double y = acc + (j->Dv ? (double)j->Dv[c] * u : 0.0);",
                          "double y = acc + (j->Dv ? (double)j->Dv[c] * (j->x64 ? 0.0 : u) : 0.0);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name):
    old, new = MUTANTS[name]
    src = open(ORACLE_SRC).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "mutant.c")
        so = os.path.join(d, "libmutant.so")
        with open(path, "w") as f:
            f.write(src.replace(old, new))
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-std=c99", "-o", so, path, "-lm", "-lpthread"])
        lib = oracle.load_library(so)
        failed = []
        for pin in pins.ALL_PINS:
            try:
                pin(lib)
            except AssertionError:
                failed.append(pin.__name__)
        assert failed, f"no pin caught mutant {name}"
