"""Properties of the compiled kernels that wait for direct global->LDS loads by count (no GPU needed).

The SSD block kernel and the one-channel-per-lane scan wait for their direct global->LDS loads with
explicit `s_waitcnt vmcnt(n)`, n counting the vector-memory operations the wave issued after the load it
needs.  In the SSD kernel that count must be exact: the loop bodies may contain no vector-memory instruction
other than those loads and the output stores, since a register spill reload, or a load the compiler adds,
would let a needed load still be in flight at the barrier.  (The scan's count covers only loads issued
unconditionally, so an extra operation there would only make a wait stricter; a spill would still cost
time.)  These tests compile the sources to gfx950 assembly with the library's own flags and check every
loop block (by the compiler's loop annotations) of every instantiation.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "selective_state_space_17_amd", "csrc")
ALLOWED = re.compile(r"global_load_lds_(dwordx4|ushort)|global_store_dwordx[24] ")
VMEM = re.compile(r"(global_|buffer_|scratch_|flat_)")


def _kernels(asm: str, kernel: str = "10ssd_kernel"):
    out, name = {}, None
    for ln in asm.split("\n"):
        m = re.match(r"^(_ZN4mssm12_GLOBAL__N_1" + kernel + r"[^:]*):", ln)
        if m:
            name = m.group(1)
            out[name] = []
            continue
        if name and ln.startswith(".Lfunc_end"):
            name = None
            continue
        if name:
            out[name].append(ln)
    return out


def _loop_vmem(body):
    inloop, seen, bad = False, 0, []
    for ln in body:
        if re.match(r"^(\.LBB\d+_\d+:|; %bb\.\d+:)", ln):
            inloop = ("Loop Header" in ln) or ("in Loop:" in ln)
            continue
        t = ln.strip()
        if inloop and VMEM.match(t):
            seen += 1
            if not ALLOWED.match(t):
                bad.append(t)
    return seen, bad


def _device_asm(tmp_path_factory, src):
    from selective_state_space_17_amd.build import FLAGS, HIPCC
    if not shutil.which(HIPCC) and not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    out = str(tmp_path_factory.mktemp("asm") / (os.path.splitext(src)[0] + ".s"))
    flags = [f for f in FLAGS if f not in ("-shared", "-fPIC", "-Wall", "-Wno-unused-function")]
    subprocess.check_call([HIPCC] + flags + ["--cuda-device-only", "-S", "-I", CSRC, "-I",
                           os.path.join(ROOT, "include"), "-o", out, os.path.join(CSRC, src)],
                          stderr=subprocess.DEVNULL)
    return open(out).read()


@pytest.fixture(scope="module")
def ssd_asm(tmp_path_factory):
    return _device_asm(tmp_path_factory, "ssd_m2.hip")


@pytest.fixture(scope="module")
def scan_asm(tmp_path_factory):
    return _device_asm(tmp_path_factory, "scan_m1.hip")


def test_ssd_loops_hold_only_the_counted_memory_operations(ssd_asm):
    ks = _kernels(ssd_asm)
    # 64/128 states x two rules x (with / without the D, z epilogue, or a share of the states in fp32)
    assert len(ks) == 12, sorted(ks)
    for name, body in ks.items():
        seen, bad = _loop_vmem(body)
        assert seen > 0, name
        assert not bad, (name, bad[:4])


def test_ssd_no_vector_register_spills(ssd_asm):
    spills = [int(v) for v in re.findall(r"\.vgpr_spill_count:\s+(\d+)", ssd_asm)]
    assert spills and all(v == 0 for v in spills), spills


LANE_ALLOWED = re.compile(r"global_load_lds_dwordx4|global_store_dwordx4 ")


def test_lane_kernel_loops_and_spills(scan_asm):
    # the one-channel-per-lane scan waits for its direct loads by count as well: its loops may hold only
    # those loads and the output stores, and no instantiation may spill
    ks = _kernels(scan_asm, "11lane_kernel")
    assert len(ks) == 6, sorted(ks)   # fp32 / bf16 x single pass, chunk pass, fix-up pass
    for name, body in ks.items():
        ops = _loop_ops(body)
        assert ops, name
        assert all(LANE_ALLOWED.match(t) for t in ops), (name, [t for t in ops if not LANE_ALLOWED.match(t)][:4])
    spills = {}
    for name in ks:
        md = scan_asm[scan_asm.index(".name:           " + name):]
        spills[name] = int(re.search(r"\.vgpr_spill_count:\s+(\d+)", md).group(1))
    assert all(v == 0 for v in spills.values()), spills


def _loop_ops(body):
    inloop, ops = False, []
    for ln in body:
        if re.match(r"^(\.LBB\d+_\d+:|; %bb\.\d+:)", ln):
            inloop = ("Loop Header" in ln) or ("in Loop:" in ln)
            continue
        t = ln.strip()
        if inloop and VMEM.match(t):
            ops.append(t)
    return ops


def test_checker_flags_an_extra_load():
    body = [".LBB0_1:                               ; =>This Inner Loop Header: Depth=1",
            "\tglobal_load_lds_dwordx4 v[0:1], off",
            "\tscratch_load_dwordx2 v[4:5], off, off ; 8-byte Folded Reload",
            "\tglobal_store_dwordx2 v[2:3], v[6:7], off",
            "; %bb.2:",
            "\tglobal_load_dwordx4 v[8:11], v[0:1], off"]
    seen, bad = _loop_vmem(body)
    assert seen == 3 and bad == ["scratch_load_dwordx2 v[4:5], off, off ; 8-byte Folded Reload"]
