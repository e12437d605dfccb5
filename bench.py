"""Throughput of the selective-scan forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2]

A step is one full forward pass (the whole hot path) over one batch of the
workload, with inputs already resident in HBM.  The default workload is the
largest one-GPU configuration: the long-context Mamba-1 scan (batch 1,
L 2^20, d_inner 2048, d_state 16, bf16 I/O, fp32 state, final state
returned), which the library splits into sequence chunks with an exact
inter-chunk carry.  Prints one JSON line on stdout; progress goes to stderr.

The roofline object leads with the HBM fraction (algorithmic bytes over the
measured call time, against 8 TB/s); the VALU-issue and, for the multi-head
form, matrix-core fractions stand beside it, and `limiter` names the ceiling
the call is closest to.

Inputs rotate over several resident copies so that consecutive steps never
read data the 256 MB memory-side cache still holds from the previous step.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0                      # MI355X HBM3E
PEAK_VALU_TSLOT = 256 * 4 * 32 * 2.4e9 / 1e12
# VALU issue: each SIMD retires a full-rate fp32 instruction (mul, add, FMA) for 32 of a wave's 64 lanes per
# cycle -- 256 CUs x 4 SIMDs x 32 lanes x 2.4 GHz = 78.6 T lane-slots/s, the published 157.3 TFLOP/s fp32 vector
# rate with an FMA counted as 2.  Measured on MI355X: a wave64 mul or FMA issues every ~2.1 cycles; exp2 and rcp
# (transcendental) every ~8.1 cycles, so each counts as 4 slots.  packed fp32 is not used.
PEAK_BF16_MFMA_TFLOPS = 2500.0
# algorithmic VALU issue slots: per state update mul + exp2 (4) + mul + FMA + FMA = 8;
# per (b, t, c): delta*x (1), D*x + y (1), and the silu gate: mul, exp2 (4), add, rcp (4), mul, mul = 12
SLOTS_PER_UPDATE = 8.0
SLOTS_PER_STEP_CHANNEL = 14.0
# gradients, per state update: the forward update (mul, exp2, mul, FMA = 7) and its readout term (2); the adjoint
# FMA and decay (2); the dC, dB, dA, ddelta and dx terms with their sums (10).  Per (b, t, c): delta*x, the gate
# (with its exp2 and rcp) and its derivative, and the ddelta / dx / dz finish (17).
SLOTS_PER_UPDATE_BWD = 21.0
SLOTS_PER_STEP_CHANNEL_BWD = 17.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_digest(is_ssd: bool, decode: bool = False, backward: bool = False, train: bool = False) -> str:
    """Hash of the sources that make the workload's kernels (counters go stale when they change)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "selective_state_space_17_amd", "csrc")
    kern = "bwd_m1.hip" if backward else ("decode.hip" if decode else ("ssd_m2.hip" if is_ssd else "scan_m1.hip"))
    h.update(open(os.path.join(csrc, kern), "rb").read())
    if train:   # a training step runs the checkpointing forward too
        h.update(open(os.path.join(csrc, "scan_m1.hip"), "rb").read())
    return h.hexdigest()[:16]


def kernel_tags(is_ssd: bool, decode: bool = False, backward: bool = False, train: bool = False):
    """Name fragments of every kernel one call of the workload launches (the first names the dominant one)."""
    if backward:
        return ("scan_bwd_kernel", "bwd_reduce", "bwd_finish") + (("wide_kernel",) if train else ())
    if decode:
        return ("ssd_update_kernel", "ssdm_update_kernel") if is_ssd else ("scan_update_kernel",)
    return ("ssd_kernel", "ssd_add_shares") if is_ssd else ("wide_kernel", "lane_kernel", "scan_kernel", "carry_kernel",
                                                             "carry_serial_kernel")


def load_traffic(workload: str, is_ssd: bool, decode: bool = False, backward: bool = False, train: bool = False):
    """HBM bytes per launch of the dominant kernel from committed rocprofv3 counters, if they were
    taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    t = json.load(open(path))
    if t.get("source_digest") != source_digest(is_ssd, decode, backward, train):
        return None
    return t.get("hbm_bytes_per_launch")


def _counter_rows(d, counter):
    import csv
    rows = list(csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))))
    return [(r["Kernel_Name"], float(r["Counter_Value"])) for r in rows if r["Counter_Name"] == counter]


def summarize_counters(cfg, is_ssd, d, copy_mib):
    """Turn the four rocprofv3 --pmc runs under d (workload FETCH_SIZE / WRITE_SIZE, copy FETCH_SIZE /
    WRITE_SIZE) into HBM bytes per call of the workload (every kernel the call launches, summed; the
    calls are counted by the dispatches of the kernel a call launches least often), each counter scaled by
    what it reads for a device copy of copy_mib MiB, and write profiles/traffic_<workload>.json."""
    train = getattr(cfg, "train", False)
    bwd = getattr(cfg, "backward", False) or train   # the gradient kernel dominates
    tags = kernel_tags(is_ssd, cfg.decode, bwd, train)
    copy_bytes = copy_mib << 20
    res = {"workload": cfg.name, "source_digest": source_digest(is_ssd, cfg.decode, bwd, train),
           "copy_bytes": copy_bytes, "algorithmic_bytes_per_launch": cfg.algorithmic_bytes()}
    total = 0.0
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        cd = os.path.join(d, "copy_" + counter.lower())
        if not os.path.isdir(cd):    # copy runs shared by several workloads sit one level up
            cd = os.path.join(os.path.dirname(os.path.abspath(d)), "copy_" + counter.lower())
        copy_kib = max(v for _, v in _counter_rows(cd, counter))
        factor = copy_bytes / (copy_kib * 1024.0)
        rows = [(n, v) for n, v in _counter_rows(os.path.join(d, "pmc_" + counter.lower()), counter)
                if any(tag in n for tag in tags)]
        if not rows:
            raise SystemExit(f"no {tags} dispatches with {counter} under {d}")
        names = sorted(set(n for n, _ in rows))
        # the dominant kernel: the one moving the most bytes.  Per call, each kernel's average bytes per
        # dispatch times the dispatches a call makes of it: a whole multiple of the fewest dispatches of any
        # of the call's kernels (the SSD kernel runs twice per call above 128 states), else once (the set-up
        # of a training-step run launches the gradient kernels alone as well)
        name = max(names, key=lambda k: sum(v for n, v in rows if n == k))
        count = {k: sum(1 for n, _ in rows if n == k) for k in names}
        calls = min(count.values())
        mult = {k: (count[k] // calls if count[k] % calls == 0 else 1) for k in names}
        kib = sum(sum(v for n, v in rows if n == k) / count[k] * mult[k] for k in names)
        res["kernel"] = name
        res["kernels_per_call"] = mult
        res[counter] = {"kib_per_call": kib, "calls": calls, "copy_kib": copy_kib,
                        "scale": factor, "bytes_per_launch": kib * 1024.0 * factor}
        total += kib * 1024.0 * factor
    res["hbm_bytes_per_launch"] = total
    res["traffic_over_algorithmic"] = total / cfg.algorithmic_bytes()
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    out = os.path.join(ROOT, "profiles", f"traffic_{cfg.name}.json")
    json.dump(res, open(out, "w"), indent=1)
    print(json.dumps(res, indent=1))


def dev(a):
    import numpy as np
    import torch
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def _timed_passes(run, min_seconds=10.0, max_passes=5000):
    """Repeat one bounded oracle pass until about min_seconds of CPU work have been timed."""
    passes, t = 0, time.perf_counter()
    while True:
        run()
        passes += 1
        dt = time.perf_counter() - t
        if dt >= min_seconds or passes >= max_passes:
            return passes, dt


def cpu_baseline_scan(inp, cfg):
    import oracle
    threads = oracle.default_threads()
    # bounded sample: whole batch and sequence, channels up to ~4e9 updates, repeated to ~10 s
    per_ch = cfg.batch * cfg.seqlen * cfg.dstate
    nc = int(min(cfg.dim, max(1, 4e9 // per_ch)))
    passes, dt = _timed_passes(lambda: oracle.scan_fwd(inp.x, inp.delta, inp.A, inp.B, inp.C, inp.D, inp.z, inp.h0,
                                                       c0=0, c1=nc, nthreads=threads))
    n = per_ch * nc * passes
    return {"value": n / dt, "unit": "state-updates/s", "cores": threads, "kind": "oracle",
            "sample": f"channels 0..{nc} of {cfg.dim}, all batches and steps, {passes} pass(es) "
                      f"({n:.3e} updates in {dt:.2f} s, fp64 sequential recurrence)"}


def cpu_baseline_scan_bwd(inp, cfg, dout):
    import oracle
    threads = oracle.default_threads()
    # the oracle splits the work over batch rows; dB/dC need every channel, so the sample is whole rows
    rows = min(cfg.batch, threads)
    sl = slice(0, rows)
    passes, dt = _timed_passes(lambda: oracle.scan_bwd(inp.x[sl], inp.delta[sl], inp.A, inp.B[sl], inp.C[sl], inp.D,
                                                       None if inp.z is None else inp.z[sl], None, dout[sl], None,
                                                       nthreads=threads))
    n = rows * cfg.seqlen * cfg.dim * cfg.dstate * passes
    return {"value": n / dt, "unit": "state-updates/s", "cores": min(threads, rows), "kind": "oracle",
            "sample": f"batch rows 0..{rows} of {cfg.batch} (all steps and channels), {passes} pass(es) "
                      f"({n:.3e} updates in {dt:.2f} s, fp64 forward then reverse recurrence)"}


def cpu_baseline_conv_scan(inp, cfg, conv):
    import oracle
    threads = oracle.default_threads()
    w, bias, _ = conv
    per_ch = cfg.batch * cfg.seqlen * cfg.dstate
    nc = int(min(cfg.dim, max(1, 4e9 // per_ch)))
    passes, dt = _timed_passes(lambda: oracle.conv_scan_fwd(inp.x, w, bias, None, inp.delta, inp.A, inp.B, inp.C,
                                                            inp.D, inp.z, None, c0=0, c1=nc, nthreads=threads))
    n = per_ch * nc * passes
    return {"value": n / dt, "unit": "state-updates/s", "cores": threads, "kind": "oracle",
            "sample": f"channels 0..{nc} of {cfg.dim} (the convolution over all channels), all batches and steps, "
                      f"{passes} pass(es) ({n:.3e} updates in {dt:.2f} s, fp64)"}


def cpu_baseline_ssd(inp, cfg, lam=None, omega=None):
    import numpy as np
    import oracle
    threads = oracle.default_threads()
    per_head = cfg.batch * cfg.seqlen * cfg.headdim * cfg.dstate
    nh = int(min(cfg.nheads, max(1, 4e9 // per_head)))
    if cfg.rank > 1:
        # MIMO: the first nh heads (one group shared by all heads), every rank, through the MIMO oracle
        assert cfg.ngroups == 1
        hs = lambda a: None if a is None else np.ascontiguousarray(a[:, :, :nh])
        x, delta, z, lm = hs(inp.x), hs(inp.delta), hs(inp.z), hs(lam)
        A = np.ascontiguousarray(inp.A[:nh])
        D = None if inp.D is None else np.ascontiguousarray(inp.D[:nh])
        h0 = None if inp.h0 is None else np.ascontiguousarray(inp.h0[:, :nh])
        run = lambda: oracle.ssdm_fwd(x, delta, lm, A, inp.B, inp.C, D, z, h0, nthreads=threads)
    elif lam is None:
        run = lambda: oracle.ssd_fwd(inp.x, inp.delta, inp.A, inp.B, inp.C, inp.D, inp.z, inp.h0, hd0=0, hd1=nh,
                                     nthreads=threads)
    else:
        # the Mamba-3 oracle runs whole problems: hand it the first nh heads (one group shared by all heads)
        assert cfg.ngroups == 1
        hs = lambda a: None if a is None else np.ascontiguousarray(a[:, :, :nh])
        x, delta, z, lm = hs(inp.x), hs(inp.delta), hs(inp.z), hs(lam)
        A = np.ascontiguousarray(inp.A[:nh])
        D = None if inp.D is None else np.ascontiguousarray(inp.D[:nh])
        h0 = None if inp.h0 is None else np.ascontiguousarray(inp.h0[:, :nh])
        if omega is None:
            run = lambda: oracle.ssd3_fwd(x, delta, lm, A, inp.B, inp.C, D, z, h0, nthreads=threads)
        else:   # the complex-valued state
            om = np.ascontiguousarray(omega[:nh])
            run = lambda: oracle.ssdc_fwd(x, delta, lm, A, om, inp.B, inp.C, D, z, h0, nthreads=threads)
    passes, dt = _timed_passes(run)
    n = per_head * nh * passes
    return {"value": n / dt, "unit": "state-updates/s", "cores": threads, "kind": "oracle",
            "sample": f"heads 0..{nh} of {cfg.nheads}, all batches and steps, {passes} pass(es) "
                      f"({n:.3e} updates in {dt:.2f} s, fp64 sequential recurrence)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=5,
                    help="workload id (1-16; 6, 7: decode steps; 8: gradients; 9: convolution fused in front; "
                         "10: training step; 11, 12: Mamba-3 SISO recurrence and its decode step; 13: that decode "
                         "step with the complex-valued state; 14, 15: Mamba-3 MIMO and its decode step; 16: "
                         "gradients with 128 states; 17: the SSD form with 256 states); the "
                         "default, 5, is the largest one-GPU configuration, the one the metric is quoted on")
    ap.add_argument("--sets", type=int, default=0, help="resident input copies to rotate over (0: auto)")
    ap.add_argument("--chunk", type=int, default=0, help="SSD time-chunk length (0: the workload's)")
    ap.add_argument("--split-seq", type=int, default=0, help="force the sequence-chunk count (0: the planner's)")
    ap.add_argument("--split-state", type=int, default=0, help="force lanes per channel (0: the planner's)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB 5 times (scales the HBM byte counters)")
    ap.add_argument("--summarize-counters", metavar="DIR", default="",
                    help="only turn rocprofv3 FETCH_SIZE/WRITE_SIZE runs under DIR (pmc_fetch_size, "
                         "pmc_write_size; copy_fetch_size, copy_write_size there or one level up) into "
                         "profiles/traffic_<workload>.json; --calibrate-copy gives the copy runs' MiB")
    args = ap.parse_args()

    if args.summarize_counters:
        import workloads as W
        cfg = W.CONFIGS[args.config]
        summarize_counters(cfg, isinstance(cfg, W.SSDConfig), args.summarize_counters, args.calibrate_copy or 1024)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the path is not sharded across GPUs in this build", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {n} bytes 5 times (reads {n}, writes {n} per copy)")
        return

    import selective_state_space_17_amd as M
    import workloads as W

    cfg = W.CONFIGS[args.config]
    is_ssd = isinstance(cfg, W.SSDConfig)
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    alg_bytes = cfg.algorithmic_bytes()
    sets = args.sets or max(1, min(8, int(np.ceil(768e6 / alg_bytes))))
    log(f"workload {cfg.name}: {cfg.updates:.3e} updates, {alg_bytes / 1e6:.1f} MB algorithmic, {sets} input set(s)")

    t = time.perf_counter()
    decode = cfg.decode
    backward = getattr(cfg, "backward", False)
    train = getattr(cfg, "train", False)
    if train:
        # one training step of the layer: the forward storing checkpoints, then the gradients from them
        host = [W.make_scan_inputs(cfg, seed_base=W.ROOT_SEED + 1000 * i) for i in range(sets)]
        douts = [W.make_scan_grads(cfg, seed_base=W.ROOT_SEED + 1000 * i, with_dfinal=False)[0] for i in range(sets)]
        ins = [dict(x=dev(h.x), delta=dev(h.delta), A=dev(h.A), B=dev(h.B), C=dev(h.C), D=dev(h.D), z=dev(h.z),
                    dout=dev(g)) for h, g in zip(host, douts)]
        io = M.MSSM_BF16 if cfg.io == W.BF16 else M.MSSM_F32
        ws_n = M.selective_scan_bwd_workspace_size(cfg.batch, cfg.seqlen, cfg.dim, cfg.dstate, io)
        ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device="cuda")
        ck = torch.empty(M.selective_scan_checkpoint_size(cfg.batch, cfg.seqlen, cfg.dim, 16, io) // 4,
                         dtype=torch.float32, device="cuda")
        outs = [torch.empty_like(a["x"]) for a in ins]
        grads = [M.selective_scan_bwd(a["x"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"], None, a["dout"],
                                      None, want_dh0=False, workspace=ws) for a in ins]

        def step(i):
            a = ins[i % sets]
            M.selective_scan_fwd_ckpt(a["x"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"], None,
                                      checkpoints=ck, out=outs[i % sets])
            M.selective_scan_bwd(a["x"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"], None, a["dout"], None,
                                 want_dh0=False, grads=grads[i % sets], checkpoints=ck, workspace=ws)
        plan = {"tokens_per_tile": 16, "channels_per_block": 16, "checkpoints": True}
    elif backward:
        # one backward pass of the layer: the loss gradient dout in, every input's gradient out
        host = [W.make_scan_inputs(cfg, seed_base=W.ROOT_SEED + 1000 * i) for i in range(sets)]
        douts = [W.make_scan_grads(cfg, seed_base=W.ROOT_SEED + 1000 * i, with_dfinal=False)[0] for i in range(sets)]
        ins = [dict(x=dev(h.x), delta=dev(h.delta), A=dev(h.A), B=dev(h.B), C=dev(h.C), D=dev(h.D), z=dev(h.z),
                    dout=dev(g)) for h, g in zip(host, douts)]
        io = M.MSSM_BF16 if cfg.io == W.BF16 else M.MSSM_F32
        ws_n = M.selective_scan_bwd_workspace_size(cfg.batch, cfg.seqlen, cfg.dim, cfg.dstate, io)
        ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device="cuda")
        a0 = ins[0]
        grads = [M.selective_scan_bwd(a["x"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"], None, a["dout"],
                                      None, want_dh0=False, workspace=ws) for a in ins]

        def step(i):
            a = ins[i % sets]
            M.selective_scan_bwd(a["x"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"], None, a["dout"], None,
                                 want_dh0=False, grads=grads[i % sets], workspace=ws)
        plan = {"tokens_per_tile": 16, "channels_per_block": 16, "state_slices": (cfg.dstate + 15) // 16}
        del a0
    elif decode:
        # token-by-token update: each input set carries its own state, advanced in place every step
        if is_ssd:
            host = [W.make_ssd_inputs(cfg, seed_base=W.ROOT_SEED + 1000 * i, with_h0=True) for i in range(sets)]
        else:
            host = [W.make_scan_inputs(cfg, seed_base=W.ROOT_SEED + 1000 * i, with_h0=True) for i in range(sets)]
        ins = [dict(x=dev(h.x), delta=dev(h.delta), A=dev(h.A), B=dev(h.B), C=dev(h.C), D=dev(h.D), z=dev(h.z),
                    state=dev(h.h0)) for h in host]
        outs = [torch.empty_like(i["x"]) for i in ins]
        upd = M.ssd_state_update if is_ssd else M.selective_state_update
        trap = is_ssd and cfg.trapezoidal
        mimo = is_ssd and cfg.rank > 1
        lams = [W.make_ssd_lam(cfg, seed_base=W.ROOT_SEED + 1000 * i) if trap else None for i in range(sets)]
        if trap:   # the Mamba-3 rule also reads the previous token's x and B
            for i, a in enumerate(ins):
                xp, bp = W.make_ssd_prev(cfg, seed_base=W.ROOT_SEED + 1000 * i)
                a.update(lam=dev(lams[i]), x_prev=dev(xp), B_prev=dev(bp))
                if cfg.complex_state:
                    a["omega"] = dev(W.make_ssd_omega(cfg, seed_base=W.ROOT_SEED + 1000 * i))

        def step(i):
            a, o = ins[i % sets], outs[i % sets]
            if mimo:
                M.ssd_mimo_state_update(a["state"], a["x"], a["delta"], a.get("lam"), a["A"], a["B"], a["C"], a["D"],
                                        a["z"], x_prev=a.get("x_prev"), B_prev=a.get("B_prev"), out=o)
            elif trap and cfg.complex_state:
                M.mamba3_siso_update(a["state"], a["x"], a["delta"], a["lam"], a["A"], a["omega"], a["B"], a["C"],
                                     a["D"], a["z"], x_prev=a["x_prev"], B_prev=a["B_prev"], out=o)
            elif trap:
                M.ssd_trapezoidal_state_update(a["state"], a["x"], a["delta"], a["lam"], a["A"], a["B"], a["C"],
                                               a["D"], a["z"], x_prev=a["x_prev"], B_prev=a["B_prev"], out=o)
            else:
                upd(a["state"], a["x"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"], out=o)
        plan = {"tokens": cfg.seqlen}
    elif is_ssd:
        chunk = args.chunk or cfg.chunk
        host = [W.make_ssd_inputs(cfg, seed_base=W.ROOT_SEED + 1000 * i) for i in range(sets)]
        lams = [W.make_ssd_lam(cfg, seed_base=W.ROOT_SEED + 1000 * i) if cfg.trapezoidal else None
                for i in range(sets)]
        ins = [dict(x=dev(h.x), delta=dev(h.delta), A=dev(h.A), B=dev(h.B), C=dev(h.C), D=dev(h.D), z=dev(h.z),
                    lam=dev(lm)) for h, lm in zip(host, lams)]
        outs = [(torch.empty_like(i["x"]),
                 torch.empty((cfg.batch, cfg.nheads, cfg.headdim, cfg.dstate), dtype=torch.float32, device="cuda"))
                for i in ins]
        ws_n = M.ssd_workspace_size(cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim, cfg.dstate, cfg.ngroups, chunk)
        ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device="cuda")

        def step(i):
            a, (o, f) = ins[i % sets], outs[i % sets]
            if cfg.rank > 1:
                M.ssd_mimo_fwd(a["x"], a["delta"], a["lam"], a["A"], a["B"], a["C"], a["D"], a["z"], None, chunk=chunk,
                               out=o, final_state=f, return_final_state=True, workspace=ws if ws_n else None)
            elif cfg.trapezoidal:
                M.ssd_trapezoidal_fwd(a["x"], a["delta"], a["lam"], a["A"], a["B"], a["C"], a["D"], a["z"], None,
                                      chunk=chunk, out=o, final_state=f, return_final_state=True,
                                      workspace=ws if ws_n else None)
            else:
                M.ssd_fwd(a["x"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"], None, chunk=chunk,
                          out=o, final_state=f, return_final_state=True, workspace=ws if ws_n else None)
        plan = {"chunk": chunk}
    elif getattr(cfg, "conv_width", 0):
        # the scan with its short causal convolution fused in front: x is made on chip from its input
        host = [W.make_scan_inputs(cfg, seed_base=W.ROOT_SEED + 1000 * i) for i in range(sets)]
        convs = [W.make_conv_inputs(cfg, cfg.conv_width, seed_base=W.ROOT_SEED + 1000 * i, with_init=False)
                 for i in range(sets)]
        ins = [dict(x=dev(h.x), delta=dev(h.delta), A=dev(h.A), B=dev(h.B), C=dev(h.C), D=dev(h.D), z=dev(h.z),
                    w=dev(cw), bias=dev(cb)) for h, (cw, cb, _) in zip(host, convs)]
        outs = [torch.empty_like(i["x"]) for i in ins]
        io = M.MSSM_BF16 if cfg.io == W.BF16 else M.MSSM_F32
        ws_n = M.selective_scan_conv_workspace_size(cfg.batch, cfg.seqlen, cfg.dim, cfg.dstate, io,
                                                    split_seq=args.split_seq)
        ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device="cuda")

        def step(i):
            a, o = ins[i % sets], outs[i % sets]
            M.selective_scan_conv_fwd(a["x"], a["w"], a["bias"], None, a["delta"], a["A"], a["B"], a["C"], a["D"],
                                      a["z"], None, out=o, split_seq=args.split_seq,
                                      workspace=ws if ws_n else None)
        plan = {"conv_width": cfg.conv_width, "split_state": 16}
    else:
        host = [W.make_scan_inputs(cfg, seed_base=W.ROOT_SEED + 1000 * i) for i in range(sets)]
        ins = [dict(x=dev(h.x), delta=dev(h.delta), A=dev(h.A), B=dev(h.B), C=dev(h.C), D=dev(h.D), z=dev(h.z))
               for h in host]
        outs = [(torch.empty_like(i["x"]),
                 torch.empty((cfg.batch, cfg.dim, cfg.dstate), dtype=torch.float32, device="cuda")
                 if cfg.return_final else None) for i in ins]
        io = M.MSSM_BF16 if cfg.io == W.BF16 else M.MSSM_F32
        K, G = M.selective_scan_plan(cfg.batch, cfg.seqlen, cfg.dim, cfg.dstate, io,
                                     split_seq=args.split_seq, split_state=args.split_state)
        ws_n = M.selective_scan_workspace_size(cfg.batch, cfg.seqlen, cfg.dim, cfg.dstate, io,
                                               split_seq=K, split_state=G)
        ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device="cuda")

        def step(i):
            a, (o, f) = ins[i % sets], outs[i % sets]
            M.selective_scan_fwd(a["x"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"], None,
                                 out=o, final_state=f, return_final_state=f is not None,
                                 split_seq=K, split_state=G, workspace=ws if ws_n else None)
        plan = {"split_seq": K, "split_state": G}
    del host[1:]
    if backward or train:
        del douts[1:]
    if getattr(cfg, "conv_width", 0):
        del convs[1:]
    torch.cuda.synchronize()
    log(f"inputs ready in {time.perf_counter() - t:.1f}s; plan {plan}")

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} done")

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        step(args.warmup + i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = [a.elapsed_time(b) for a, b in ev]
    ms = float(np.mean(step_ms))
    log(f"timed {args.steps} steps: wall {wall * 1e3 / args.steps:.3f} ms/step, events mean {ms:.3f} "
        f"median {float(np.median(step_ms)):.3f} min {min(step_ms):.3f} ms")

    upd_s = cfg.updates / (wall / args.steps)
    kern_s = ms * 1e-3
    traffic = load_traffic(cfg.name, is_ssd, decode, backward or train, train)
    # the headline roofline is HBM: algorithmic bytes over the event-timed call
    roof = {"bound": "hbm", "achieved": alg_bytes / kern_s / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / PEAK_HBM_GBS
    roof["traffic"] = traffic

    def alu_obj(slots):
        a = {"achieved": slots / kern_s / 1e12, "peak": PEAK_VALU_TSLOT, "unit": "Tslot/s"}
        a["frac"] = a["achieved"] / a["peak"]
        return a

    if backward or train:
        # the whole backward call (gradient kernel and the two small fixed-order sum kernels); a training
        # step adds the forward before it
        slots = cfg.updates * SLOTS_PER_UPDATE_BWD + cfg.batch * cfg.seqlen * cfg.dim * SLOTS_PER_STEP_CHANNEL_BWD
        if train:
            slots += cfg.updates * SLOTS_PER_UPDATE + cfg.batch * cfg.seqlen * cfg.dim * SLOTS_PER_STEP_CHANNEL
        roof["alu"] = alu_obj(slots)
    elif decode:
        # a few operations per byte of state: the HBM roofline bounds it
        roof["alu"] = alu_obj(cfg.updates * (SLOTS_PER_UPDATE if not is_ssd else 4.0))
    elif is_ssd:
        Q = 64   # the kernel evaluates any chunk length as 64-row blocks (a row is a step, or one of its R ranks)
        # matrix-core work of the block form per launch: per row and head the causal in-block Q*P/2 and the
        # state readout and update 2*N*P; per row and group C.B^T Q*N/2 (causal)
        macs = cfg.batch * cfg.seqlen * cfg.rank * (cfg.nheads * (Q * cfg.headdim / 2 + 2 * cfg.dstate * cfg.headdim)
                                                    + cfg.ngroups * Q * cfg.dstate / 2)
        mf = {"achieved": 2 * macs / kern_s / 1e12, "peak": PEAK_BF16_MFMA_TFLOPS, "unit": "TFLOP/s"}
        mf["frac"] = mf["achieved"] / mf["peak"]
        roof["mfma"] = mf
    else:
        per_tc = SLOTS_PER_STEP_CHANNEL
        if getattr(cfg, "conv_width", 0):
            # the fused convolution: one FMA per tap, then its SiLU (mul, exp2 (4), add, rcp (4), mul)
            per_tc += cfg.conv_width + 11
        roof["alu"] = alu_obj(cfg.updates * SLOTS_PER_UPDATE + cfg.batch * cfg.seqlen * cfg.dim * per_tc)
    # the ceiling the call sits closest to
    fr = {"hbm": roof["frac"], "alu": roof.get("alu", {}).get("frac", 0.0),
          "mfma": roof.get("mfma", {}).get("frac", 0.0)}
    roof["limiter"] = max(fr, key=fr.get)
    if backward:
        roof["scope"] = ("whole backward call: scan_bwd_kernel, then bwd_reduce_bc and bwd_reduce_ad"
                         + (", and bwd_finish adding the state slices' sums" if cfg.dstate > 16 else ""))
    elif train:
        roof["scope"] = ("whole training step: wide_kernel storing checkpoints, then scan_bwd_kernel from them, "
                         "bwd_reduce_bc and bwd_reduce_ad")
    elif not decode and not is_ssd and plan.get("split_seq", 1) > 1:
        roof["scope"] = ("whole call: the chunk pass, carry_kernel (the scan over the chunks' maps), "
                         "then the fix-up pass")

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        h = host[0]
        if backward or train:
            cpu = cpu_baseline_scan_bwd(h, cfg, douts[0])
            if train:
                cpu["sample"] += " (the gradient pass only; the oracle's gradients include their own forward)"
        elif getattr(cfg, "conv_width", 0):
            cpu = cpu_baseline_conv_scan(h, cfg, convs[0])
        else:
            cpu = (cpu_baseline_ssd(h, cfg, lams[0] if cfg.trapezoidal else None,
                                    W.make_ssd_omega(cfg) if getattr(cfg, "complex_state", False) else None) if is_ssd
                   else cpu_baseline_scan(h, cfg))
        if decode:
            cpu["sample"] += "; the same recurrence from the stored state (h0)"
        log(f"cpu baseline: {cpu}")

    conf = {"workload": cfg.name, "batch": cfg.batch, "seqlen": cfg.seqlen}
    if decode:
        conf["decode"] = True
    if backward:
        conf["backward"] = True
    if train:
        conf["training_step"] = True
    if is_ssd:
        conf.update(nheads=cfg.nheads, headdim=cfg.headdim, d_state=cfg.dstate, ngroups=cfg.ngroups, io="bf16",
                    **plan)
        if cfg.trapezoidal:
            conf["rule"] = "exponential-trapezoidal"
        if cfg.rank > 1:
            conf["mimo_rank"] = cfg.rank
        if getattr(cfg, "complex_state", False):
            conf["state"] = "complex (rotation per state pair)"
    else:
        conf.update(d_inner=cfg.dim, d_state=cfg.dstate, io=cfg.io, D=cfg.has_D, z_gate=cfg.has_z,
                    final_state=cfg.return_final, **plan)
    conf["input_sets"] = sets
    line = {
        "metric": ("selective-scan training-step state updates/s (B*L*d_inner*N per forward + gradients), 1 GPU"
                   if train else "selective-scan gradient state updates/s (B*L*d_inner*N), 1 GPU" if backward else
                   "selective-scan state updates/s (B*L*d_inner*N), 1 GPU"),
        "value": upd_s,
        "unit": "state-updates/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": conf,
        "hbm_gbs": alg_bytes / (wall / args.steps) / 1e9,
        "kernel_ms": ms,
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
