"""The C-ABI library loads, exports what include/mssm.h declares, and rejects
bad arguments on the host before any HIP call (no GPU needed)."""
import ctypes
import os
import re

import pytest

import selective_state_space_17_amd as M

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "mssm.h")

BASE = 0x7F0000000000   # fake device addresses: validation never dereferences them
MB = 1 << 20


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mssm_[a-z_0-9]+)\s*\(", src)))


def test_header_symbols_exported():
    names = declared_functions()
    assert names, "no declarations found"
    assert set(names) == set(M.SIGNATURES), "binding signatures and header disagree"
    for n in names:
        assert hasattr(M.lib, n), f"{n} not exported"
    out = os.popen(f"nm -D --defined-only {M.LIB_PATH}").read()
    for n in names:
        assert re.search(rf"\bT {n}\b", out), f"{n} not a defined dynamic symbol"


def test_version_and_status_strings():
    assert M.abi_version() == 1
    for st in (0, -1, -2, -3, -4, -5):
        assert M.lib.mssm_status_string(st)
    assert M.lib.mssm_status_string(123) == b"unknown status"


def _scan_call(desc, x=BASE, delta=BASE + 100 * MB, A=BASE + 200 * MB, B=BASE + 300 * MB, C=BASE + 400 * MB,
               D=None, z=None, h0=None, out=BASE + 500 * MB, final=None, ws=None, ws_bytes=0):
    return M.lib.mssm_selective_scan_fwd(ctypes.byref(desc) if desc is not None else None, x, delta, A, B, C, D, z,
                                         h0, out, final, ws, ws_bytes, None)


def small(**kw):
    a = dict(batch=2, seqlen=64, dim=32, dstate=16, io_dtype=M.MSSM_BF16, split_seq=1, split_state=1)
    a.update(kw)
    return M.scan_desc(**a)


@pytest.mark.parametrize("case,expect", [
    ("null_desc", M.MSSM_ERR_INVALID_ARG),
    ("dim0", M.MSSM_ERR_INVALID_ARG),
    ("neg_batch", M.MSSM_ERR_INVALID_ARG),
    ("dstate0", M.MSSM_ERR_INVALID_ARG),
    ("dstate_big", M.MSSM_ERR_UNSUPPORTED),
    ("bad_dtype", M.MSSM_ERR_UNSUPPORTED),
    ("flags", M.MSSM_ERR_INVALID_ARG),
    ("split_state_3", M.MSSM_ERR_UNSUPPORTED),
    ("split_state_too_small", M.MSSM_ERR_UNSUPPORTED),
    ("split_seq_big", M.MSSM_ERR_INVALID_ARG),
    ("overflow", M.MSSM_ERR_INVALID_ARG),
    ("null_x", M.MSSM_ERR_INVALID_ARG),
    ("null_A", M.MSSM_ERR_INVALID_ARG),
    ("null_out", M.MSSM_ERR_INVALID_ARG),
    ("misaligned_x", M.MSSM_ERR_MISALIGNED),
    ("misaligned_A", M.MSSM_ERR_MISALIGNED),
    ("out_aliases_x", M.MSSM_ERR_INVALID_ARG),
    ("final_aliases_h0", M.MSSM_ERR_INVALID_ARG),
    ("no_workspace", M.MSSM_ERR_WORKSPACE),
    ("small_workspace", M.MSSM_ERR_WORKSPACE),
    ("misaligned_workspace", M.MSSM_ERR_MISALIGNED),
])
def test_scan_validation(case, expect):
    d = small()
    kw = {}
    if case == "null_desc":
        d = None
    elif case == "dim0":
        d = small(dim=0)
    elif case == "neg_batch":
        d = small(batch=-1)
    elif case == "dstate0":
        d = small(dstate=0)
    elif case == "dstate_big":
        d = small(dstate=300, split_state=0)
    elif case == "bad_dtype":
        d = small(io_dtype=7)
    elif case == "flags":
        d = small()
        d.flags = 1
    elif case == "split_state_3":
        d = small(split_state=3)
    elif case == "split_state_too_small":
        d = small(dstate=64, split_state=2)    # 2 lanes x 16 states < 64
    elif case == "split_seq_big":
        d = small(split_seq=5000)
    elif case == "overflow":
        d = small(batch=1 << 40, seqlen=1 << 30)
    elif case == "null_x":
        kw["x"] = None
    elif case == "null_A":
        kw["A"] = None
    elif case == "null_out":
        kw["out"] = None
    elif case == "misaligned_x":
        kw["x"] = BASE + 1
    elif case == "misaligned_A":
        kw["A"] = BASE + 200 * MB + 2
    elif case == "out_aliases_x":
        kw["out"] = BASE + 64
    elif case == "final_aliases_h0":
        kw["h0"] = BASE + 600 * MB
        kw["final"] = BASE + 600 * MB + 256
    elif case in ("no_workspace", "small_workspace", "misaligned_workspace"):
        d = small(seqlen=4096, split_seq=4)
        need = M.lib.mssm_selective_scan_workspace_size(ctypes.byref(d))
        assert need > 0
        if case == "small_workspace":
            kw["ws"], kw["ws_bytes"] = BASE + 700 * MB, need - 1
        elif case == "misaligned_workspace":
            kw["ws"], kw["ws_bytes"] = BASE + 700 * MB + 16, need
    assert _scan_call(d, **kw) == expect


def test_empty_batch_is_a_noop():
    # batch == 0: nothing to do, returns before touching HIP (null pointers allowed)
    d = small(batch=0)
    assert M.lib.mssm_selective_scan_fwd(ctypes.byref(d), None, None, BASE, None, None, None, None, None, None,
                                         None, None, 0, None) == M.MSSM_OK


def test_plan_and_workspace():
    for (b, l, d, n) in [(8, 2048, 1536, 16), (4, 8192, 5120, 16), (1, 1 << 20, 2048, 16), (1, 256, 64, 16)]:
        k, g = M.selective_scan_plan(b, l, d, n)
        assert 1 <= k <= 4096 and g in (1, 2, 4, 8, 16)
        ws = M.selective_scan_workspace_size(b, l, d, n)
        assert (ws == 0) == (k == 1)
    # the long sequence must be split to fill the chip
    assert M.selective_scan_plan(1, 1 << 20, 2048, 16)[0] > 1
    # bf16 at dstate 16: one lane per channel, the chunk count that fills the resident waves (2048 / 32 and
    # 2048 / 320 chunks of 64 channels), and the 130M layer unsplit on one state per lane
    assert M.selective_scan_plan(1, 1 << 20, 2048, 16, M.MSSM_BF16) == (64, 1)
    assert M.selective_scan_plan(4, 8192, 5120, 16, M.MSSM_BF16) == (6, 1)
    assert M.selective_scan_plan(8, 2048, 1536, 16, M.MSSM_BF16) == (1, 16)
    # forced plans are honoured
    assert M.selective_scan_plan(2, 1000, 64, 16, split_seq=3, split_state=4) == (3, 4)
    assert M.selective_scan_plan(1, 10, 64, 16, split_seq=64)[0] == 10   # never more chunks than steps
    # a launch grid counts its work-items in 32 bits: 2048 x 2^20 channels fit only with one lane per
    # channel and no split (2^31 items), 4096 x 2^20 (2^32 items) in no plan at all
    assert M.selective_scan_plan(2048, 1, 1 << 20, 16) == (1, 1)
    with pytest.raises(M.MssmError) as e:
        M.selective_scan_plan(4096, 1, 1 << 20, 16)
    assert e.value.status == M.MSSM_ERR_UNSUPPORTED


def _ssd_call(desc, x=BASE, delta=BASE + 100 * MB, A=BASE + 200 * MB, B=BASE + 300 * MB, C=BASE + 400 * MB,
              out=BASE + 500 * MB):
    return M.lib.mssm_ssd_fwd(ctypes.byref(desc), x, delta, A, B, C, None, None, None, out, None, None, 0, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(io_dtype=7), M.MSSM_ERR_UNSUPPORTED),
    (dict(nheads=6, ngroups=4), M.MSSM_ERR_UNSUPPORTED),
    (dict(chunk=48), M.MSSM_ERR_UNSUPPORTED),
    (dict(chunk=32), M.MSSM_ERR_UNSUPPORTED),
    (dict(dstate=257), M.MSSM_ERR_UNSUPPORTED),
    (dict(headdim=0), M.MSSM_ERR_INVALID_ARG),
    (dict(batch=-2), M.MSSM_ERR_INVALID_ARG),
])
def test_ssd_validation(kw, expect):
    a = dict(batch=2, seqlen=128, nheads=4, headdim=64, dstate=64, ngroups=1, chunk=64, io_dtype=M.MSSM_BF16)
    a.update(kw)
    assert _ssd_call(M.ssd_desc(**a)) == expect


# Shapes and dtypes the matrix-core block kernel does not take: accepted, and run through the recurrent
# update kernel. A null x proves the descriptor passed (the pointer checks reject it) without launching.
RECURRENT_SSD = [dict(io_dtype=M.MSSM_F32), dict(headdim=20), dict(headdim=100), dict(dstate=20), dict(dstate=200),
                 dict(dstate=6)]


@pytest.mark.parametrize("kw", RECURRENT_SSD)
def test_ssd_recurrent_shapes_accepted(kw):
    a = dict(batch=2, seqlen=128, nheads=4, headdim=64, dstate=64, ngroups=1, chunk=64, io_dtype=M.MSSM_BF16)
    a.update(kw)
    d = M.ssd_desc(**a)
    assert _ssd_call(d, x=None) == M.MSSM_ERR_INVALID_ARG
    assert M.lib.mssm_ssd_workspace_size(ctypes.byref(d)) == 0


def test_ssd_route():
    block, rec = M.SSD_ROUTE_BLOCK, M.SSD_ROUTE_RECURRENT
    # the workload's shape and the shapes the block kernel takes
    assert M.ssd_plan(8, 4096, 32, 64, 128, 1, 256) == block
    assert M.ssd_plan(1, 1, 3, 128, 48, 3, 0) == block
    for kw in RECURRENT_SSD:
        a = dict(batch=2, seqlen=128, nheads=4, headdim=64, dstate=64, ngroups=1, chunk=64, io_dtype=M.MSSM_BF16)
        a.update(kw)
        assert M.ssd_plan(**a) == rec, kw
    # the block kernel forms every offset in 64 bits: strides of 2^24 elements and more stay on it
    assert M.ssd_plan(1, 8, (1 << 18) - 1, 64, 64, 1) == block
    assert M.ssd_plan(1, 8, 1 << 18, 64, 64, 1) == block                # nheads * headdim = 2^24
    assert M.ssd_plan(1, 8, (1 << 18) + 1, 64, 64, 1) == block
    assert M.ssd_plan(1, 8, 1 << 20, 64, 16, 1 << 20) == block          # ngroups * dstate = 2^24
    # MIMO: the block kernel takes ranks 1, 2, 4, 8 and 16; others run through the update kernel
    for r in (1, 2, 4, 8, 16):
        assert M.ssd_mimo_plan(8, 4096, 32, 64, 128, 1, r) == block
    for r in (3, 5, 32, 64):
        assert M.ssd_mimo_plan(8, 4096, 32, 64, 128, 1, r) == rec
    assert M.ssd_mimo_plan(1, 8, 4, 64, 64, 1, 4, io_dtype=M.MSSM_F32) == rec
    # headdims that are multiples of 8: 64-wide slices, the last one cut at headdim
    for pd in (8, 24, 48, 96, 136):
        assert M.ssd_plan(2, 100, 4, pd, 64, 1) == block
        assert M.ssd_mimo_plan(2, 100, 4, pd, 64, 1, 4) == block
    # more than 128 states: the block kernel on two shares of the states, one input per channel only
    for n in (144, 192, 256):
        assert M.ssd_plan(8, 4096, 32, 64, n, 1, 256) == block
        assert M.ssd_mimo_plan(8, 4096, 32, 64, n, 1, 1) == block
        assert M.ssd_mimo_plan(8, 4096, 32, 64, n, 1, 2) == rec
    # its workspace holds the two shares in fp32; up to 128 states none is needed
    d = M.ssd_desc(2, 100, 3, 128, 256, 1)
    assert M.lib.mssm_ssd_workspace_size(ctypes.byref(d)) == (2 * 4 * 2 * 100 * 3 * 128 + 255) // 256 * 256
    assert M.lib.mssm_ssd_workspace_size(ctypes.byref(M.ssd_desc(2, 100, 3, 128, 128, 1))) == 0
    for r, st in ((0, M.MSSM_ERR_INVALID_ARG), (-1, M.MSSM_ERR_INVALID_ARG), (65, M.MSSM_ERR_UNSUPPORTED)):
        with pytest.raises(M.MssmError) as e:
            M.ssd_mimo_plan(1, 8, 4, 64, 64, 1, r)
        assert e.value.status == st
    with pytest.raises(M.MssmError):
        M.ssd_plan(1, 8, 6, 64, 64, 4)                                  # nheads % ngroups != 0
    d = M.ssd_desc(1, 8, 4, 64, 64, 1)
    assert M.lib.mssm_ssd_plan(ctypes.byref(d), None) == M.MSSM_ERR_INVALID_ARG


def test_ssd_pointer_checks():
    d = M.ssd_desc(2, 128, 4, 64, 64, 1, 64)
    assert _ssd_call(d, x=None) == M.MSSM_ERR_INVALID_ARG
    assert _ssd_call(d, x=BASE + 8) == M.MSSM_ERR_MISALIGNED
    assert _ssd_call(d, out=BASE + 16) == M.MSSM_ERR_INVALID_ARG


def test_ssd_shares_workspace_checks():
    # above 128 states the block kernel needs its workspace: missing, short, misaligned, or overlapping
    d = M.ssd_desc(2, 128, 4, 64, 256, 1, 64)
    need = M.lib.mssm_ssd_workspace_size(ctypes.byref(d))
    assert need == 2 * 4 * 2 * 128 * 4 * 64

    def call(ws, nbytes, out=BASE + 500 * MB):
        return M.lib.mssm_ssd_fwd(ctypes.byref(d), BASE, BASE + 100 * MB, BASE + 200 * MB, BASE + 300 * MB,
                                  BASE + 400 * MB, None, None, None, out, None, ws, nbytes, None)
    assert call(None, 0) == M.MSSM_ERR_WORKSPACE
    assert call(BASE + 600 * MB, need - 1) == M.MSSM_ERR_WORKSPACE
    assert call(BASE + 600 * MB + 16, need) == M.MSSM_ERR_MISALIGNED
    assert call(BASE + 400 * MB, need) == M.MSSM_ERR_INVALID_ARG       # overlaps C
    assert call(BASE + 600 * MB, need, out=BASE + 600 * MB + need - 64) == M.MSSM_ERR_INVALID_ARG


def _ssd3_call(desc, x=BASE, delta=BASE + 100 * MB, lam=BASE + 150 * MB, A=BASE + 200 * MB, B=BASE + 300 * MB,
               C=BASE + 400 * MB, out=BASE + 500 * MB):
    return M.lib.mssm_ssd_trapezoidal_fwd(ctypes.byref(desc), x, delta, lam, A, B, C, None, None, None, out, None,
                                          None, 0, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(io_dtype=7), M.MSSM_ERR_UNSUPPORTED),
    (dict(dstate=300), M.MSSM_ERR_UNSUPPORTED),
    (dict(batch=-2), M.MSSM_ERR_INVALID_ARG),
])
def test_ssd_trapezoidal_validation(kw, expect):
    """The Mamba-3 entry point shares the SSD descriptor rules."""
    a = dict(batch=2, seqlen=128, nheads=4, headdim=64, dstate=64, ngroups=1, chunk=64, io_dtype=M.MSSM_BF16)
    a.update(kw)
    assert _ssd3_call(M.ssd_desc(**a)) == expect


@pytest.mark.parametrize("kw", RECURRENT_SSD)
def test_ssd_trapezoidal_recurrent_shapes_accepted(kw):
    a = dict(batch=2, seqlen=128, nheads=4, headdim=64, dstate=64, ngroups=1, chunk=64, io_dtype=M.MSSM_BF16)
    a.update(kw)
    d = M.ssd_desc(**a)
    assert _ssd3_call(d, x=None) == M.MSSM_ERR_INVALID_ARG
    assert _ssd3_call(d, lam=None) == M.MSSM_ERR_INVALID_ARG


def test_ssd_trapezoidal_pointer_checks():
    d = M.ssd_desc(2, 128, 4, 64, 64, 1, 64)
    assert _ssd3_call(d, lam=None) == M.MSSM_ERR_INVALID_ARG            # lam is required
    assert _ssd3_call(d, lam=BASE + 150 * MB + 1) == M.MSSM_ERR_MISALIGNED
    assert _ssd3_call(d, out=BASE + 150 * MB - 64) == M.MSSM_ERR_INVALID_ARG   # out overlaps lam
    assert _ssd3_call(d, x=None) == M.MSSM_ERR_INVALID_ARG
    # nothing to do: no batch rows
    assert _ssd3_call(M.ssd_desc(0, 128, 4, 64, 64, 1, 64), lam=None) == M.MSSM_OK


def _upd_call(desc, state=BASE + 600 * MB, x=BASE, delta=BASE + 100 * MB, A=BASE + 200 * MB, B=BASE + 300 * MB,
              C=BASE + 400 * MB, D=None, z=None, out=BASE + 500 * MB):
    return M.lib.mssm_selective_state_update(ctypes.byref(desc) if desc is not None else None, state, x, delta, A,
                                             B, C, D, z, out, None)


@pytest.mark.parametrize("case,expect", [
    ("null_desc", M.MSSM_ERR_INVALID_ARG),
    ("null_state", M.MSSM_ERR_INVALID_ARG),
    ("null_x", M.MSSM_ERR_INVALID_ARG),
    ("misaligned_state", M.MSSM_ERR_MISALIGNED),
    ("misaligned_x", M.MSSM_ERR_MISALIGNED),
    ("state_aliases_x", M.MSSM_ERR_INVALID_ARG),
    ("out_aliases_state", M.MSSM_ERR_INVALID_ARG),
    ("bad_dtype", M.MSSM_ERR_UNSUPPORTED),
    ("dstate_big", M.MSSM_ERR_UNSUPPORTED),
])
def test_state_update_validation(case, expect):
    d = small(seqlen=1)
    kw = {}
    if case == "null_desc":
        d = None
    elif case == "null_state":
        kw["state"] = None
    elif case == "null_x":
        kw["x"] = None
    elif case == "misaligned_state":
        kw["state"] = BASE + 600 * MB + 2
    elif case == "misaligned_x":
        kw["x"] = BASE + 1
    elif case == "state_aliases_x":
        kw["state"] = BASE + 32
    elif case == "out_aliases_state":
        kw["out"] = BASE + 600 * MB + 8
    elif case == "bad_dtype":
        d = small(seqlen=1, io_dtype=5)
    elif case == "dstate_big":
        d = small(seqlen=1, dstate=300, split_state=0)
    assert _upd_call(d, **kw) == expect


def test_state_update_empty_is_a_noop():
    # no tokens, or no batch: nothing to do, returns before touching HIP (null pointers allowed)
    for d in (small(seqlen=0), small(batch=0)):
        assert M.lib.mssm_selective_state_update(ctypes.byref(d), None, None, None, None, None, None, None, None,
                                                 None, None) == M.MSSM_OK
    s = M.ssd_desc(2, 0, 4, 64, 64, 1, 0)
    assert M.lib.mssm_ssd_state_update(ctypes.byref(s), None, None, None, None, None, None, None, None, None,
                                       None) == M.MSSM_OK


@pytest.mark.parametrize("kw,expect", [
    (dict(nheads=6, ngroups=4), M.MSSM_ERR_UNSUPPORTED),
    (dict(dstate=300), M.MSSM_ERR_UNSUPPORTED),
    (dict(io_dtype=7), M.MSSM_ERR_UNSUPPORTED),
    (dict(headdim=0), M.MSSM_ERR_INVALID_ARG),
    (dict(batch=-1), M.MSSM_ERR_INVALID_ARG),
])
def test_ssd_state_update_validation(kw, expect):
    a = dict(batch=2, seqlen=1, nheads=4, headdim=64, dstate=64, ngroups=1, chunk=0, io_dtype=M.MSSM_BF16)
    a.update(kw)
    d = M.ssd_desc(**a)
    assert M.lib.mssm_ssd_state_update(ctypes.byref(d), BASE + 600 * MB, BASE, BASE + 100 * MB, BASE + 200 * MB,
                                       BASE + 300 * MB, BASE + 400 * MB, None, None, BASE + 500 * MB, None) == expect


def test_ssd_state_update_pointer_checks():
    d = M.ssd_desc(2, 1, 4, 64, 64, 1, 0)
    args = [BASE + 600 * MB, BASE, BASE + 100 * MB, BASE + 200 * MB, BASE + 300 * MB, BASE + 400 * MB, None, None,
            BASE + 500 * MB, None]
    call = lambda a: M.lib.mssm_ssd_state_update(ctypes.byref(d), *a)
    bad = list(args); bad[0] = None
    assert call(bad) == M.MSSM_ERR_INVALID_ARG              # state missing
    bad = list(args); bad[0] = BASE + 600 * MB + 1
    assert call(bad) == M.MSSM_ERR_MISALIGNED
    bad = list(args); bad[8] = BASE + 600 * MB
    assert call(bad) == M.MSSM_ERR_INVALID_ARG              # out aliases state


def test_ssd_trapezoidal_state_update_checks():
    """The Mamba-3 decode step: the SSD update's rules, plus lam required and the previous token's x and B
    optional, aligned and not overlapping the outputs."""
    d = M.ssd_desc(2, 1, 4, 64, 64, 1, 0)
    # state, x_prev, B_prev, x, delta, lam, A, B, C, D, z, out
    args = [BASE + 600 * MB, BASE + 700 * MB, BASE + 800 * MB, BASE, BASE + 100 * MB, BASE + 150 * MB,
            BASE + 200 * MB, BASE + 300 * MB, BASE + 400 * MB, None, None, BASE + 500 * MB]
    call = lambda a, dd=d: M.lib.mssm_ssd_trapezoidal_state_update(ctypes.byref(dd), *a, None)
    bad = list(args); bad[5] = None
    assert call(bad) == M.MSSM_ERR_INVALID_ARG              # lam missing
    bad = list(args); bad[2] = BASE + 800 * MB + 1
    assert call(bad) == M.MSSM_ERR_MISALIGNED               # B_prev misaligned
    bad = list(args); bad[11] = BASE + 700 * MB
    assert call(bad) == M.MSSM_ERR_INVALID_ARG              # out overlaps x_prev
    bad = list(args); bad[0] = BASE + 800 * MB
    assert call(bad) == M.MSSM_ERR_INVALID_ARG              # state overlaps B_prev
    for kw, expect in ((dict(dstate=300), M.MSSM_ERR_UNSUPPORTED), (dict(batch=-1), M.MSSM_ERR_INVALID_ARG)):
        a = dict(batch=2, seqlen=1, nheads=4, headdim=64, dstate=64, ngroups=1, chunk=0, io_dtype=M.MSSM_BF16)
        a.update(kw)
        assert call(args, M.ssd_desc(**a)) == expect
    # no tokens: nothing to do, null pointers allowed
    s = M.ssd_desc(2, 0, 4, 64, 64, 1, 0)
    assert call([None] * 12, s) == M.MSSM_OK


def test_mamba3_siso_update_checks():
    """The complex-state update: the trapezoidal update's rules, plus omega required, aligned, not
    overlapping the outputs, and an even dstate."""
    d = M.ssd_desc(2, 1, 4, 64, 64, 1, 0)
    # state, x_prev, B_prev, x, delta, lam, A, omega, B, C, D, z, out
    args = [BASE + 600 * MB, BASE + 700 * MB, BASE + 800 * MB, BASE, BASE + 100 * MB, BASE + 150 * MB,
            BASE + 200 * MB, BASE + 250 * MB, BASE + 300 * MB, BASE + 400 * MB, None, None, BASE + 500 * MB]
    call = lambda a, dd=d: M.lib.mssm_mamba3_siso_update(ctypes.byref(dd), *a, None)
    bad = list(args); bad[7] = None
    assert call(bad) == M.MSSM_ERR_INVALID_ARG              # omega missing
    bad = list(args); bad[5] = None
    assert call(bad) == M.MSSM_ERR_INVALID_ARG              # lam missing
    bad = list(args); bad[7] = BASE + 250 * MB + 2
    assert call(bad) == M.MSSM_ERR_MISALIGNED
    bad = list(args); bad[0] = BASE + 250 * MB
    assert call(bad) == M.MSSM_ERR_INVALID_ARG              # state overlaps omega
    odd = M.ssd_desc(2, 1, 4, 64, 63, 1, 0)
    assert call(args, odd) == M.MSSM_ERR_UNSUPPORTED        # the state pairs need an even dstate
    assert call([None] * 13, M.ssd_desc(2, 0, 4, 64, 64, 1, 0)) == M.MSSM_OK   # no tokens


def _bwd_call(desc, ws=BASE + 2000 * MB, ws_bytes=None, **kw):
    a = dict(x=BASE, delta=BASE + 100 * MB, A=BASE + 200 * MB, B=BASE + 300 * MB, C=BASE + 400 * MB, D=None,
             z=None, h0=None, dout=BASE + 500 * MB, dfinal=None, dx=BASE + 600 * MB, ddelta=BASE + 700 * MB,
             dA=BASE + 800 * MB, dB=BASE + 900 * MB, dC=BASE + 1000 * MB, dD=None, dz=None, dh0=None, ck=None)
    a.update(kw)
    if ws_bytes is None:
        ws_bytes = M.lib.mssm_selective_scan_bwd_workspace_size(ctypes.byref(desc)) if desc is not None else 0
    return M.lib.mssm_selective_scan_bwd(ctypes.byref(desc) if desc is not None else None, a["x"], a["delta"],
                                         a["A"], a["B"], a["C"], a["D"], a["z"], a["h0"], a["dout"], a["dfinal"],
                                         a["dx"], a["ddelta"], a["dA"], a["dB"], a["dC"], a["dD"], a["dz"], a["dh0"],
                                         a["ck"], ws, ws_bytes, None)


@pytest.mark.parametrize("case,expect", [
    ("null_desc", M.MSSM_ERR_INVALID_ARG),
    ("dstate_257", M.MSSM_ERR_UNSUPPORTED),
    ("bad_dtype", M.MSSM_ERR_UNSUPPORTED),
    ("null_dout", M.MSSM_ERR_INVALID_ARG),
    ("null_dA", M.MSSM_ERR_INVALID_ARG),
    ("z_without_dz", M.MSSM_ERR_INVALID_ARG),
    ("D_without_dD", M.MSSM_ERR_INVALID_ARG),
    ("misaligned_dx", M.MSSM_ERR_MISALIGNED),
    ("misaligned_dB", M.MSSM_ERR_MISALIGNED),
    ("dx_aliases_x", M.MSSM_ERR_INVALID_ARG),
    ("dB_aliases_dC", M.MSSM_ERR_INVALID_ARG),
    ("workspace_aliases_dx", M.MSSM_ERR_INVALID_ARG),
    ("checkpoints_dstate8", M.MSSM_ERR_UNSUPPORTED),
    ("dx_aliases_checkpoints", M.MSSM_ERR_INVALID_ARG),
    ("no_workspace", M.MSSM_ERR_WORKSPACE),
    ("small_workspace", M.MSSM_ERR_WORKSPACE),
    ("misaligned_workspace", M.MSSM_ERR_MISALIGNED),
])
def test_scan_bwd_validation(case, expect):
    d = small()
    kw = {}
    if case == "null_desc":
        d = None
    elif case == "dstate_257":
        d = small(dstate=257, split_state=0)
    elif case == "bad_dtype":
        d = small(io_dtype=3)
    elif case == "null_dout":
        kw["dout"] = None
    elif case == "null_dA":
        kw["dA"] = None
    elif case == "z_without_dz":
        kw["z"] = BASE + 1100 * MB
    elif case == "D_without_dD":
        kw["D"] = BASE + 1100 * MB
    elif case == "misaligned_dx":
        kw["dx"] = BASE + 600 * MB + 1
    elif case == "misaligned_dB":
        kw["dB"] = BASE + 900 * MB + 2
    elif case == "dx_aliases_x":
        kw["dx"] = BASE + 64
    elif case == "dB_aliases_dC":
        kw["dB"] = BASE + 1000 * MB + 16
    elif case == "workspace_aliases_dx":
        kw["ws"] = BASE + 600 * MB
    elif case == "checkpoints_dstate8":
        d = small(dstate=8, split_state=0)
        kw["ck"] = BASE + 1200 * MB
    elif case == "dx_aliases_checkpoints":
        kw["ck"] = BASE + 600 * MB + 64
    elif case == "no_workspace":
        kw["ws"] = None
    elif case == "small_workspace":
        kw["ws_bytes"] = M.lib.mssm_selective_scan_bwd_workspace_size(ctypes.byref(d)) - 1
    elif case == "misaligned_workspace":
        kw["ws"] = BASE + 2000 * MB + 16
    assert _bwd_call(d, **kw) == expect


def test_scan_bwd_workspace_size():
    # checkpoints every 16 steps, per-16-channel-block dB/dC partials, per-row dA/dD partials (256-byte aligned)
    d = small(batch=2, seqlen=64, dim=32, dstate=16)
    al = lambda v: (v + 255) // 256 * 256
    want = al(4 * 2 * 4 * 32 * 16) + 2 * al(4 * 2 * 2 * 64 * 16) + al(4 * 2 * 32 * 16) + al(4 * 2 * 32)
    assert M.lib.mssm_selective_scan_bwd_workspace_size(ctypes.byref(d)) == want
    # 40 states: three slices of 16, and the slices' partial sums of the three per-(b, t, c) state sums
    d = small(batch=2, seqlen=64, dim=32, dstate=40, split_state=0)
    want = al(4 * 2 * 4 * 32 * 48) + 2 * al(4 * 2 * 2 * 64 * 48) + al(4 * 2 * 32 * 48) + al(4 * 2 * 32) + \
        3 * al(4 * 3 * 2 * 64 * 32)
    assert M.lib.mssm_selective_scan_bwd_workspace_size(ctypes.byref(d)) == want
    assert M.lib.mssm_selective_scan_bwd_workspace_size(ctypes.byref(small(dstate=257, split_state=0))) == 0


def _conv_call(desc, width=4, ws=None, ws_bytes=0, **kw):
    a = dict(xin=BASE, w=BASE + 100 * MB, bias=None, init=None, delta=BASE + 200 * MB, A=BASE + 300 * MB,
             B=BASE + 400 * MB, C=BASE + 500 * MB, D=None, z=None, h0=None, out=BASE + 600 * MB, final=None)
    a.update(kw)
    return M.lib.mssm_selective_scan_conv_fwd(ctypes.byref(desc) if desc is not None else None, width, a["xin"],
                                              a["w"], a["bias"], a["init"], a["delta"], a["A"], a["B"], a["C"],
                                              a["D"], a["z"], a["h0"], a["out"], a["final"], ws, ws_bytes, None)


@pytest.mark.parametrize("case,expect", [
    ("null_desc", M.MSSM_ERR_INVALID_ARG),
    ("width0", M.MSSM_ERR_UNSUPPORTED),
    ("width5", M.MSSM_ERR_UNSUPPORTED),
    # the fused kernel does not take these: they run through the recurrent kernel, so the descriptor
    # passes and (with a null xin) the pointer checks answer, before anything is launched
    ("dstate8", M.MSSM_ERR_INVALID_ARG),
    ("split_state4", M.MSSM_ERR_INVALID_ARG),
    ("dim_not_16_bytes", M.MSSM_ERR_INVALID_ARG),
    ("null_taps", M.MSSM_ERR_INVALID_ARG),
    ("null_xin", M.MSSM_ERR_INVALID_ARG),
    ("xin_misaligned", M.MSSM_ERR_MISALIGNED),
    ("init_misaligned", M.MSSM_ERR_MISALIGNED),
    ("out_aliases_init", M.MSSM_ERR_INVALID_ARG),
    ("out_aliases_taps", M.MSSM_ERR_INVALID_ARG),
])
def test_conv_validation(case, expect):
    d = small(split_state=0)
    kw = {}
    width = 4
    if case == "null_desc":
        d = None
    elif case == "width0":
        width = 0
    elif case == "width5":
        width = 5
    elif case == "dstate8":
        d, kw["xin"] = small(dstate=8, split_state=0), None
    elif case == "split_state4":
        d, kw["xin"] = small(split_state=4), None
    elif case == "dim_not_16_bytes":
        d, kw["xin"] = small(dim=36, split_state=0), None
    elif case == "null_taps":
        kw["w"] = None
    elif case == "null_xin":
        kw["xin"] = None
    elif case == "xin_misaligned":     # not even element-aligned: refused on either route
        kw["xin"] = BASE + 1
    elif case == "init_misaligned":
        kw["init"] = BASE + 700 * MB + 1
    elif case == "out_aliases_init":
        kw["init"] = BASE + 600 * MB + 64
    elif case == "out_aliases_taps":
        kw["w"] = BASE + 600 * MB + 64
    assert _conv_call(d, width, **kw) == expect


def test_conv_workspace_size():
    # the convolution path plans with 16 lanes per channel; a single chunk needs no workspace
    d = small(split_seq=1, split_state=0)
    assert M.lib.mssm_selective_scan_conv_workspace_size(ctypes.byref(d)) == 0
    d = M.scan_desc(1, 4096, 64, 16, M.MSSM_BF16, 4, 16)
    assert M.lib.mssm_selective_scan_conv_workspace_size(ctypes.byref(d)) == \
        M.lib.mssm_selective_scan_workspace_size(ctypes.byref(d)) > 0
    assert M.lib.mssm_selective_scan_conv_workspace_size(ctypes.byref(small(dstate=8, split_state=0))) == 0


def _ck_call(desc, ws=None, ws_bytes=0, **kw):
    a = dict(x=BASE, delta=BASE + 100 * MB, A=BASE + 200 * MB, B=BASE + 300 * MB, C=BASE + 400 * MB, D=None,
             z=None, h0=None, out=BASE + 500 * MB, final=None, ck=BASE + 600 * MB)
    a.update(kw)
    return M.lib.mssm_selective_scan_fwd_ckpt(ctypes.byref(desc) if desc is not None else None, a["x"], a["delta"],
                                              a["A"], a["B"], a["C"], a["D"], a["z"], a["h0"], a["out"], a["final"],
                                              a["ck"], ws, ws_bytes, None)


@pytest.mark.parametrize("case,expect", [
    ("null_desc", M.MSSM_ERR_INVALID_ARG),
    ("dstate8", M.MSSM_ERR_UNSUPPORTED),
    ("split_state4", M.MSSM_ERR_UNSUPPORTED),
    ("null_checkpoints", M.MSSM_ERR_INVALID_ARG),
    ("misaligned_checkpoints", M.MSSM_ERR_MISALIGNED),
    ("x_not_16_aligned", M.MSSM_ERR_MISALIGNED),
    ("checkpoints_alias_out", M.MSSM_ERR_INVALID_ARG),
    ("checkpoints_alias_x", M.MSSM_ERR_INVALID_ARG),
])
def test_fwd_ckpt_validation(case, expect):
    d = small(split_state=0)
    kw = {}
    if case == "null_desc":
        d = None
    elif case == "dstate8":
        d = small(dstate=8, split_state=0)
    elif case == "split_state4":
        d = small(split_state=4)
    elif case == "null_checkpoints":
        kw["ck"] = None
    elif case == "misaligned_checkpoints":
        kw["ck"] = BASE + 600 * MB + 2
    elif case == "x_not_16_aligned":
        kw["x"] = BASE + 8
    elif case == "checkpoints_alias_out":
        kw["ck"] = BASE + 500 * MB + 64
    elif case == "checkpoints_alias_x":
        kw["ck"] = BASE + 64
    assert _ck_call(d, **kw) == expect


def test_checkpoint_size():
    d = small(batch=2, seqlen=40, dim=24, dstate=16, split_state=0)
    assert M.lib.mssm_selective_scan_checkpoint_size(ctypes.byref(d)) == 2 * 3 * 32 * 16 * 4
    assert M.lib.mssm_selective_scan_checkpoint_size(ctypes.byref(small(dstate=8, split_state=0))) == 0


@pytest.mark.parametrize("case,expect", [
    ("width0", M.MSSM_ERR_UNSUPPORTED),
    ("width5", M.MSSM_ERR_UNSUPPORTED),
    ("null_window", M.MSSM_ERR_INVALID_ARG),
    ("null_taps", M.MSSM_ERR_INVALID_ARG),
    ("misaligned_window", M.MSSM_ERR_MISALIGNED),
    ("window_aliases_out", M.MSSM_ERR_INVALID_ARG),
    ("window_aliases_state", M.MSSM_ERR_INVALID_ARG),
])
def test_state_update_conv_validation(case, expect):
    d = small(seqlen=1)
    a = dict(width=4, state=BASE + 600 * MB, cs=BASE + 700 * MB, xin=BASE, w=BASE + 800 * MB, bias=None,
             delta=BASE + 100 * MB, A=BASE + 200 * MB, B=BASE + 300 * MB, C=BASE + 400 * MB, out=BASE + 500 * MB)
    if case == "width0":
        a["width"] = 0
    elif case == "width5":
        a["width"] = 5
    elif case == "null_window":
        a["cs"] = None
    elif case == "null_taps":
        a["w"] = None
    elif case == "misaligned_window":
        a["cs"] = BASE + 700 * MB + 1
    elif case == "window_aliases_out":
        a["cs"] = BASE + 500 * MB + 16
    elif case == "window_aliases_state":
        a["cs"] = BASE + 600 * MB + 16
    assert M.lib.mssm_selective_state_update_conv(ctypes.byref(d), a["width"], a["state"], a["cs"], a["xin"], a["w"],
                                                  a["bias"], a["delta"], a["A"], a["B"], a["C"], None, None,
                                                  a["out"], None) == expect


def _noalloc_call(desc, x=BASE, delta=BASE + 100 * MB, A=BASE + 200 * MB, B=BASE + 300 * MB, C=BASE + 400 * MB,
                  out=BASE + 500 * MB, final=None):
    return M.lib.mssm_selective_scan_fwd_noalloc(ctypes.byref(desc) if desc is not None else None, x, delta, A,
                                                 B, C, None, None, None, out, final, None)


def test_noalloc_validation():
    """The entry point without workspace rejects bad arguments on the host, before it would look up its
    scratch: the same checks as the forward, and a forced split whose aggregates exceed the scratch."""
    assert _noalloc_call(None) == M.MSSM_ERR_INVALID_ARG
    assert _noalloc_call(small(dstate=0)) == M.MSSM_ERR_INVALID_ARG
    assert _noalloc_call(small(), x=None) == M.MSSM_ERR_INVALID_ARG
    assert _noalloc_call(small(), x=BASE + 1) == M.MSSM_ERR_MISALIGNED
    assert _noalloc_call(small(), out=BASE + 2) == M.MSSM_ERR_INVALID_ARG       # out overlaps x
    # 4096 chunks x 2048 channels x 17 floats x 2 segments is far beyond 32 MiB
    big = M.scan_desc(1, 1 << 20, 2048, 16, M.MSSM_BF16, 4096, 1)
    assert M.selective_scan_workspace_size(1, 1 << 20, 2048, 16, M.MSSM_BF16, 4096, 1) > M.SCRATCH_BYTES
    GB = 1 << 30   # the 2^20 x 2048 bf16 tensors take 4 GiB each: fake addresses 8 GiB apart
    assert _noalloc_call(big, x=BASE, delta=BASE + 8 * GB, A=BASE + 16 * GB, B=BASE + 17 * GB, C=BASE + 18 * GB,
                         out=BASE + 24 * GB) == M.MSSM_ERR_WORKSPACE
    d = small(batch=0)
    assert M.lib.mssm_selective_scan_fwd_noalloc(ctypes.byref(d), None, None, BASE, None, None, None, None, None,
                                                 None, None, None) == M.MSSM_OK


def _mimo_call(desc, rank, x=BASE, delta=BASE + 100 * MB, lam=BASE + 150 * MB, A=BASE + 200 * MB, B=BASE + 300 * MB,
               C=BASE + 400 * MB, D=None, z=None, h0=None, out=BASE + 500 * MB, fin=None):
    return M.lib.mssm_ssd_mimo_fwd(ctypes.byref(desc), rank, x, delta, lam, A, B, C, D, z, h0, out, fin, None, 0,
                                   None)


def test_ssd_mimo_fwd_checks():
    """Mamba-3 MIMO forward: the rank is checked, and every pointer rule of the SSD forward holds with x, z,
    out spanning rank * headdim per head and B, C rank * dstate per group (nothing here reaches a kernel)."""
    d = M.ssd_desc(2, 128, 4, 64, 64, 1, 64)
    for r, st in ((0, M.MSSM_ERR_INVALID_ARG), (-3, M.MSSM_ERR_INVALID_ARG), (65, M.MSSM_ERR_UNSUPPORTED)):
        assert _mimo_call(d, r) == st, r
    assert _mimo_call(d, 4, x=None) == M.MSSM_ERR_INVALID_ARG
    assert _mimo_call(d, 4, A=None) == M.MSSM_ERR_INVALID_ARG
    assert _mimo_call(d, 4, x=BASE + 8) == M.MSSM_ERR_MISALIGNED
    assert _mimo_call(d, 4, lam=BASE + 150 * MB + 1) == M.MSSM_ERR_MISALIGNED
    assert _mimo_call(d, 4, h0=BASE + 600 * MB + 4) == M.MSSM_ERR_MISALIGNED
    # x spans 2 * 128 * 4 * 4 * 64 bf16 = 512 KiB at rank 4: an output 256 KiB in overlaps it
    assert _mimo_call(d, 4, out=BASE + 256 * 1024) == M.MSSM_ERR_INVALID_ARG
    # B spans 2 * 128 * 1 * 4 * 64 bf16 = 128 KiB at rank 4: a final state 64 KiB in overlaps it
    assert _mimo_call(d, 4, fin=BASE + 300 * MB + 64 * 1024) == M.MSSM_ERR_INVALID_ARG
    for kw, st in ((dict(io_dtype=7), M.MSSM_ERR_UNSUPPORTED), (dict(dstate=300), M.MSSM_ERR_UNSUPPORTED),
                   (dict(batch=-1), M.MSSM_ERR_INVALID_ARG), (dict(nheads=6, ngroups=4), M.MSSM_ERR_UNSUPPORTED)):
        a = dict(batch=2, seqlen=128, nheads=4, headdim=64, dstate=64, ngroups=1, chunk=64, io_dtype=M.MSSM_BF16)
        a.update(kw)
        assert _mimo_call(M.ssd_desc(**a), 4) == st, kw
    # no batch rows: nothing to do, null pointers allowed
    assert _mimo_call(M.ssd_desc(0, 128, 4, 64, 64, 1, 64), 4, x=None, delta=None, lam=None, B=None, C=None,
                      out=None) == M.MSSM_OK


def test_ssd_mimo_state_update_checks():
    """Mamba-3 MIMO decode step: rank, state and aliasing rules (nothing here reaches a kernel)."""
    d = M.ssd_desc(2, 1, 4, 64, 64, 1, 0)
    # state, x_prev, B_prev, x, delta, lam, A, B, C, D, z, out
    args = [BASE + 600 * MB, BASE + 700 * MB, BASE + 800 * MB, BASE, BASE + 100 * MB, BASE + 150 * MB,
            BASE + 200 * MB, BASE + 300 * MB, BASE + 400 * MB, None, None, BASE + 500 * MB]
    call = lambda a, r=4, dd=d: M.lib.mssm_ssd_mimo_state_update(ctypes.byref(dd), r, *a, None)
    for r, st in ((0, M.MSSM_ERR_INVALID_ARG), (-1, M.MSSM_ERR_INVALID_ARG), (65, M.MSSM_ERR_UNSUPPORTED)):
        assert call(args, r) == st, r
    bad = list(args); bad[0] = None
    assert call(bad) == M.MSSM_ERR_INVALID_ARG              # state missing
    bad = list(args); bad[0] = BASE + 600 * MB + 2
    assert call(bad) == M.MSSM_ERR_MISALIGNED               # state misaligned
    bad = list(args); bad[11] = BASE + 600 * MB
    assert call(bad) == M.MSSM_ERR_INVALID_ARG              # out aliases the state
    bad = list(args); bad[11] = BASE + 1024
    assert call(bad) == M.MSSM_ERR_INVALID_ARG              # out overlaps x (rank-4 rows span 4 KiB)
    bad = list(args); bad[2] = BASE + 800 * MB + 1
    assert call(bad) == M.MSSM_ERR_MISALIGNED               # B_prev misaligned
    # no tokens: nothing to do, null pointers allowed
    assert call([None] * 12, 4, M.ssd_desc(2, 0, 4, 64, 64, 1, 0)) == M.MSSM_OK
