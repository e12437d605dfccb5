"""MI355X (gfx950) selective scan: thin Python binding of libmssm.so.

Every step of the computation runs in the library's HIP kernels; this module
only checks tensors, allocates outputs and workspace with torch (device memory
and streams are all torch is used for) and forwards raw pointers through the C
ABI declared in include/mssm.h.  There is no fallback path: if the library is
missing, importing this package raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmssm.so")

MSSM_OK = 0
MSSM_ERR_INVALID_ARG = -1
MSSM_ERR_UNSUPPORTED = -2
MSSM_ERR_MISALIGNED = -3
MSSM_ERR_WORKSPACE = -4
MSSM_ERR_HIP = -5
MSSM_F32 = 0
MSSM_BF16 = 1


class ScanDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("dim", ctypes.c_int64),
                ("dstate", ctypes.c_int64), ("io_dtype", ctypes.c_int32), ("split_seq", ctypes.c_int32),
                ("split_state", ctypes.c_int32), ("flags", ctypes.c_uint32)]


class SSDDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("nheads", ctypes.c_int64),
                ("headdim", ctypes.c_int64), ("dstate", ctypes.c_int64), ("ngroups", ctypes.c_int64),
                ("chunk", ctypes.c_int64), ("io_dtype", ctypes.c_int32), ("flags", ctypes.c_uint32)]


# every exported symbol and its ctypes signature (checked against include/mssm.h by the tests)
_P, _SZ, _I = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
SIGNATURES = {
    "mssm_selective_scan_fwd": (_I, [ctypes.POINTER(ScanDesc)] + [_P] * 10 + [_P, _SZ, _P]),
    "mssm_selective_scan_workspace_size": (_SZ, [ctypes.POINTER(ScanDesc)]),
    "mssm_selective_scan_fwd_noalloc": (_I, [ctypes.POINTER(ScanDesc)] + [_P] * 10 + [_P]),
    "mssm_selective_scan_plan": (_I, [ctypes.POINTER(ScanDesc), ctypes.POINTER(ctypes.c_int32),
                                      ctypes.POINTER(ctypes.c_int32)]),
    "mssm_ssd_fwd": (_I, [ctypes.POINTER(SSDDesc)] + [_P] * 10 + [_P, _SZ, _P]),
    "mssm_ssd_workspace_size": (_SZ, [ctypes.POINTER(SSDDesc)]),
    "mssm_ssd_plan": (_I, [ctypes.POINTER(SSDDesc), ctypes.POINTER(ctypes.c_int32)]),
    "mssm_ssd_mimo_plan": (_I, [ctypes.POINTER(SSDDesc), ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)]),
    "mssm_ssd_mimo_fwd": (_I, [ctypes.POINTER(SSDDesc), ctypes.c_int32] + [_P] * 11 + [_P, _SZ, _P]),
    "mssm_ssd_mimo_state_update": (_I, [ctypes.POINTER(SSDDesc), ctypes.c_int32] + [_P] * 13),
    "mssm_ssd_trapezoidal_fwd": (_I, [ctypes.POINTER(SSDDesc)] + [_P] * 11 + [_P, _SZ, _P]),
    "mssm_selective_state_update": (_I, [ctypes.POINTER(ScanDesc)] + [_P] * 10),
    "mssm_ssd_state_update": (_I, [ctypes.POINTER(SSDDesc)] + [_P] * 10),
    "mssm_ssd_trapezoidal_state_update": (_I, [ctypes.POINTER(SSDDesc)] + [_P] * 13),
    "mssm_mamba3_siso_update": (_I, [ctypes.POINTER(SSDDesc)] + [_P] * 14),
    "mssm_selective_state_update_conv": (_I, [ctypes.POINTER(ScanDesc), ctypes.c_int32] + [_P] * 13),
    "mssm_selective_scan_conv_fwd": (_I, [ctypes.POINTER(ScanDesc), ctypes.c_int32] + [_P] * 13 + [_P, _SZ, _P]),
    "mssm_selective_scan_conv_workspace_size": (_SZ, [ctypes.POINTER(ScanDesc)]),
    "mssm_selective_scan_bwd": (_I, [ctypes.POINTER(ScanDesc)] + [_P] * 19 + [_P, _SZ, _P]),
    "mssm_selective_scan_fwd_ckpt": (_I, [ctypes.POINTER(ScanDesc)] + [_P] * 11 + [_P, _SZ, _P]),
    "mssm_selective_scan_fwd_ckpt_workspace_size": (_SZ, [ctypes.POINTER(ScanDesc)]),
    "mssm_selective_scan_checkpoint_size": (_SZ, [ctypes.POINTER(ScanDesc)]),
    "mssm_selective_scan_bwd_workspace_size": (_SZ, [ctypes.POINTER(ScanDesc)]),
    "mssm_status_string": (ctypes.c_char_p, [_I]),
    "mssm_last_error_detail": (ctypes.c_char_p, []),
    "mssm_abi_version": (_I, []),
}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python selective_state_space_17_amd/build.py` "
                          "(or __graft_entry__.build()) first")
    # The library's HIP runtime dependency must resolve to the copy torch ships:
    # two HIP runtimes in one process leave the second without a device.  Load
    # torch first so libamdhip64 is already present when the library is opened.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


class MssmError(RuntimeError):
    def __init__(self, status: int, what: str):
        detail = lib.mssm_last_error_detail().decode() if status == MSSM_ERR_HIP else ""
        msg = f"{what}: {lib.mssm_status_string(status).decode()} ({status})"
        super().__init__(msg + (f": {detail}" if detail else ""))
        self.status = status


def abi_version() -> int:
    return lib.mssm_abi_version()


_TORCH = None


def _torch():
    global _TORCH
    if _TORCH is None:
        import torch
        _TORCH = torch
    return _TORCH


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _check_gpu(name, t, dtype, shape, cur):
    # Every check here runs on each call, so each uses the cheapest accessor (a decode step's
    # call is otherwise dominated by them): cur is the current device, looked up once per call,
    # get_device() is an int (-1 off the GPU), and a torch.Size compares equal to a tuple of
    # the same sizes.
    if t is None:
        return
    where = t.get_device()
    if where != cur:
        if where < 0:
            raise ValueError(f"{name} must be a GPU tensor")
        # the kernels run on the current device: a pointer into another GPU's memory would fault there
        raise ValueError(f"{name} is on {t.device}, but the current device is cuda:{cur} "
                         "(use torch.cuda.device(...) around the call)")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.shape != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _io_code(dtype) -> int:
    torch = _torch()
    if dtype == torch.float32:
        return MSSM_F32
    if dtype == torch.bfloat16:
        return MSSM_BF16
    raise TypeError(f"io dtype must be float32 or bfloat16, got {dtype}")


def _stream_handle(stream) -> int:
    torch = _torch()
    if stream is None:
        # the current stream of the current device (under graph capture: the capturing stream), as
        # its raw handle, without building a Stream object
        return torch._C._cuda_getCurrentRawStream(torch.cuda.current_device())
    if stream.device.index != torch.cuda.current_device():
        raise ValueError(f"stream belongs to {stream.device}, but the current device is "
                         f"cuda:{torch.cuda.current_device()}")
    return stream.cuda_stream


def scan_desc(batch, seqlen, dim, dstate, io_dtype, split_seq=0, split_state=0) -> ScanDesc:
    return ScanDesc(batch, seqlen, dim, dstate, io_dtype, split_seq, split_state, 0)


def selective_scan_plan(batch: int, seqlen: int, dim: int, dstate: int, io_dtype: int = MSSM_BF16,
                        split_seq: int = 0, split_state: int = 0) -> Tuple[int, int]:
    """(sequence chunks, lanes per channel) the library picks for this problem."""
    d = scan_desc(batch, seqlen, dim, dstate, io_dtype, split_seq, split_state)
    k, g = ctypes.c_int32(0), ctypes.c_int32(0)
    st = lib.mssm_selective_scan_plan(ctypes.byref(d), ctypes.byref(k), ctypes.byref(g))
    if st != MSSM_OK:
        raise MssmError(st, "mssm_selective_scan_plan")
    return k.value, g.value


def selective_scan_workspace_size(batch, seqlen, dim, dstate, io_dtype=MSSM_BF16, split_seq=0, split_state=0) -> int:
    d = scan_desc(batch, seqlen, dim, dstate, io_dtype, split_seq, split_state)
    return lib.mssm_selective_scan_workspace_size(ctypes.byref(d))


def selective_scan_fwd(x, delta, A, B, C, D=None, z=None, h0=None, return_final_state: bool = False,
                       split_seq: int = 0, split_state: int = 0, out=None, final_state=None, workspace=None,
                       stream=None):
    """Mamba-1 selective scan forward (mssm_selective_scan_fwd).

    x, delta, z: [batch, seqlen, dim]; B, C: [batch, seqlen, dstate] (float32 or bfloat16, all alike);
    A: [dim, dstate] float32; D: [dim] float32; h0: [batch, dim, dstate] float32.
    Returns out (and final_state [batch, dim, dstate] float32 when requested).
    """
    torch = _torch()
    if x.dim() != 3:
        raise ValueError("x must be [batch, seqlen, dim]")
    bsz, L, dm = x.shape
    if A.dim() != 2 or A.shape[0] != dm:
        raise ValueError("A must be [dim, dstate]")
    N = A.shape[1]
    io = _io_code(x.dtype)
    cur = _torch().cuda.current_device()
    for name, t, shape in (("x", x, (bsz, L, dm)), ("delta", delta, (bsz, L, dm)), ("z", z, (bsz, L, dm)),
                           ("B", B, (bsz, L, N)), ("C", C, (bsz, L, N))):
        _check_gpu(name, t, x.dtype, shape, cur)
    _check_gpu("A", A, torch.float32, (dm, N), cur)
    _check_gpu("D", D, torch.float32, (dm,), cur)
    _check_gpu("h0", h0, torch.float32, (bsz, dm, N), cur)
    if out is None:
        out = torch.empty_like(x)
    _check_gpu("out", out, x.dtype, (bsz, L, dm), cur)
    if return_final_state and final_state is None:
        final_state = torch.empty((bsz, dm, N), dtype=torch.float32, device=x.device)
    _check_gpu("final_state", final_state, torch.float32, (bsz, dm, N), cur)
    d = scan_desc(bsz, L, dm, N, io, split_seq, split_state)
    ws_bytes = lib.mssm_selective_scan_workspace_size(ctypes.byref(d))
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=x.device)
    st = lib.mssm_selective_scan_fwd(ctypes.byref(d), _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                     _ptr(z), _ptr(h0), _ptr(out), _ptr(final_state),
                                     _ptr(workspace) if ws_bytes else None,
                                     workspace.numel() if (ws_bytes and workspace is not None) else 0,
                                     _stream_handle(stream))
    if st != MSSM_OK:
        raise MssmError(st, "mssm_selective_scan_fwd")
    return (out, final_state) if return_final_state else out


SCRATCH_BYTES = 32 << 20   # the per-device scratch mssm_selective_scan_fwd_noalloc keeps its chunk aggregates in


def selective_scan_fwd_noalloc(x, delta, A, B, C, D=None, z=None, h0=None, out=None, final_state=None,
                               split_seq: int = 0, split_state: int = 0, stream=None):
    """mssm_selective_scan_fwd_noalloc: the forward with no workspace (a split sequence keeps its chunk
    aggregates in the library's fixed per-device scratch).  ``out`` (and ``final_state``, when wanted)
    must be given, so that nothing is allocated here either; returns out."""
    torch = _torch()
    if x.dim() != 3:
        raise ValueError("x must be [batch, seqlen, dim]")
    if out is None:
        raise ValueError("out must be given: this entry point allocates nothing")
    bsz, L, dm = x.shape
    if A.dim() != 2 or A.shape[0] != dm:
        raise ValueError("A must be [dim, dstate]")
    N = A.shape[1]
    io = _io_code(x.dtype)
    cur = torch.cuda.current_device()
    for name, t, shape in (("x", x, (bsz, L, dm)), ("delta", delta, (bsz, L, dm)), ("z", z, (bsz, L, dm)),
                           ("B", B, (bsz, L, N)), ("C", C, (bsz, L, N)), ("out", out, (bsz, L, dm))):
        _check_gpu(name, t, x.dtype, shape, cur)
    _check_gpu("A", A, torch.float32, (dm, N), cur)
    _check_gpu("D", D, torch.float32, (dm,), cur)
    _check_gpu("h0", h0, torch.float32, (bsz, dm, N), cur)
    _check_gpu("final_state", final_state, torch.float32, (bsz, dm, N), cur)
    d = scan_desc(bsz, L, dm, N, io, split_seq, split_state)
    st = lib.mssm_selective_scan_fwd_noalloc(ctypes.byref(d), _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C),
                                             _ptr(D), _ptr(z), _ptr(h0), _ptr(out), _ptr(final_state),
                                             _stream_handle(stream))
    if st != MSSM_OK:
        raise MssmError(st, "mssm_selective_scan_fwd_noalloc")
    return out


def selective_scan_checkpoint_size(batch, seqlen, dim, dstate=16, io_dtype=MSSM_BF16) -> int:
    d = scan_desc(batch, seqlen, dim, dstate, io_dtype)
    return lib.mssm_selective_scan_checkpoint_size(ctypes.byref(d))


def selective_scan_fwd_ckpt(x, delta, A, B, C, D=None, z=None, h0=None, checkpoints=None,
                            return_final_state: bool = False, split_seq: int = 0, out=None, final_state=None,
                            workspace=None, stream=None):
    """Training-mode forward (mssm_selective_scan_fwd_ckpt): selective_scan_fwd that also stores the state
    entering every 16-step tile into ``checkpoints`` (allocated when None), for selective_scan_bwd.
    Returns (out, checkpoints) or (out, final_state, checkpoints)."""
    torch = _torch()
    if x.dim() != 3:
        raise ValueError("x must be [batch, seqlen, dim]")
    bsz, L, dm = x.shape
    if A.dim() != 2 or A.shape[0] != dm:
        raise ValueError("A must be [dim, dstate]")
    N = A.shape[1]
    io = _io_code(x.dtype)
    cur = _torch().cuda.current_device()
    for name, t, shape in (("x", x, (bsz, L, dm)), ("delta", delta, (bsz, L, dm)), ("z", z, (bsz, L, dm)),
                           ("B", B, (bsz, L, N)), ("C", C, (bsz, L, N))):
        _check_gpu(name, t, x.dtype, shape, cur)
    _check_gpu("A", A, torch.float32, (dm, N), cur)
    _check_gpu("D", D, torch.float32, (dm,), cur)
    _check_gpu("h0", h0, torch.float32, (bsz, dm, N), cur)
    if out is None:
        out = torch.empty_like(x)
    _check_gpu("out", out, x.dtype, (bsz, L, dm), cur)
    if return_final_state and final_state is None:
        final_state = torch.empty((bsz, dm, N), dtype=torch.float32, device=x.device)
    _check_gpu("final_state", final_state, torch.float32, (bsz, dm, N), cur)
    d = scan_desc(bsz, L, dm, N, io, split_seq, 16)
    ck_bytes = lib.mssm_selective_scan_checkpoint_size(ctypes.byref(d))
    if checkpoints is None:
        checkpoints = torch.empty(max(ck_bytes // 4, 1), dtype=torch.float32, device=x.device)
    elif not checkpoints.is_cuda or checkpoints.dtype != torch.float32 or checkpoints.numel() * 4 < ck_bytes:
        raise ValueError(f"checkpoints must be a float32 GPU tensor of at least {ck_bytes} bytes")
    ws_bytes = lib.mssm_selective_scan_fwd_ckpt_workspace_size(ctypes.byref(d))
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=x.device)
    st = lib.mssm_selective_scan_fwd_ckpt(ctypes.byref(d), _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                          _ptr(z), _ptr(h0), _ptr(out), _ptr(final_state), _ptr(checkpoints),
                                          _ptr(workspace) if ws_bytes else None,
                                          workspace.numel() if (ws_bytes and workspace is not None) else 0,
                                          _stream_handle(stream))
    if st != MSSM_OK:
        raise MssmError(st, "mssm_selective_scan_fwd_ckpt")
    return (out, final_state, checkpoints) if return_final_state else (out, checkpoints)


def selective_scan_conv_workspace_size(batch, seqlen, dim, dstate, io_dtype=MSSM_BF16, split_seq=0) -> int:
    d = scan_desc(batch, seqlen, dim, dstate, io_dtype, split_seq, 16)
    return lib.mssm_selective_scan_conv_workspace_size(ctypes.byref(d))


def selective_scan_conv_fwd(xin, conv_w, conv_b, conv_init, delta, A, B, C, D=None, z=None, h0=None,
                            return_final_state: bool = False, split_seq: int = 0, out=None, final_state=None,
                            workspace=None, stream=None):
    """Selective scan with the short causal convolution + SiLU fused in front
    (mssm_selective_scan_conv_fwd): x = silu(conv_b + causal_conv(xin, conv_w)).

    xin, delta, z: [batch, seqlen, dim]; B, C: [batch, seqlen, dstate]; conv_w [dim, W] float32 (W 1..4);
    conv_b [dim] float32 or None; conv_init [batch, W-1, dim] in xin's dtype or None (read only).
    dstate 16 with rows of a multiple of 16 bytes runs on the fused block kernel; any other problem
    (dstate up to 256) on the recurrent kernel, token by token.
    """
    torch = _torch()
    if xin.dim() != 3:
        raise ValueError("xin must be [batch, seqlen, dim]")
    bsz, L, dm = xin.shape
    if A.dim() != 2 or A.shape[0] != dm:
        raise ValueError("A must be [dim, dstate]")
    if conv_w.dim() != 2 or conv_w.shape[0] != dm:
        raise ValueError("conv_w must be [dim, width]")
    N, W = A.shape[1], conv_w.shape[1]
    io = _io_code(xin.dtype)
    cur = _torch().cuda.current_device()
    for name, t, shape in (("xin", xin, (bsz, L, dm)), ("delta", delta, (bsz, L, dm)), ("z", z, (bsz, L, dm)),
                           ("B", B, (bsz, L, N)), ("C", C, (bsz, L, N)), ("conv_init", conv_init, (bsz, W - 1, dm))):
        _check_gpu(name, t, xin.dtype, shape, cur)
    _check_gpu("conv_w", conv_w, torch.float32, (dm, W), cur)
    _check_gpu("conv_b", conv_b, torch.float32, (dm,), cur)
    _check_gpu("A", A, torch.float32, (dm, N), cur)
    _check_gpu("D", D, torch.float32, (dm,), cur)
    _check_gpu("h0", h0, torch.float32, (bsz, dm, N), cur)
    if out is None:
        out = torch.empty_like(xin)
    _check_gpu("out", out, xin.dtype, (bsz, L, dm), cur)
    if return_final_state and final_state is None:
        final_state = torch.empty((bsz, dm, N), dtype=torch.float32, device=xin.device)
    _check_gpu("final_state", final_state, torch.float32, (bsz, dm, N), cur)
    d = scan_desc(bsz, L, dm, N, io, split_seq, 16)
    ws_bytes = lib.mssm_selective_scan_conv_workspace_size(ctypes.byref(d))
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=xin.device)
    st = lib.mssm_selective_scan_conv_fwd(ctypes.byref(d), W, _ptr(xin), _ptr(conv_w), _ptr(conv_b),
                                          _ptr(conv_init), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                          _ptr(h0), _ptr(out), _ptr(final_state),
                                          _ptr(workspace) if ws_bytes else None,
                                          workspace.numel() if (ws_bytes and workspace is not None) else 0,
                                          _stream_handle(stream))
    if st != MSSM_OK:
        raise MssmError(st, "mssm_selective_scan_conv_fwd")
    return (out, final_state) if return_final_state else out


def selective_scan_bwd_workspace_size(batch, seqlen, dim, dstate, io_dtype=MSSM_BF16) -> int:
    d = scan_desc(batch, seqlen, dim, dstate, io_dtype)
    return lib.mssm_selective_scan_bwd_workspace_size(ctypes.byref(d))


def selective_scan_bwd(x, delta, A, B, C, D=None, z=None, h0=None, dout=None, dfinal=None, want_dh0: bool = True,
                       grads=None, checkpoints=None, workspace=None, stream=None):
    """Gradients of the Mamba-1 selective scan (mssm_selective_scan_bwd), for the loss
    sum(out * dout) + sum(final_state * dfinal).

    Inputs as in selective_scan_fwd; dout [batch, seqlen, dim] in the io dtype; dfinal
    [batch, dim, dstate] float32 or None.  Returns a dict: dx, ddelta, dz (io dtype, dz None without z),
    dB, dC [batch, seqlen, dstate] float32, dA [dim, dstate] float32, dD [dim] float32 (None without D),
    dh0 [batch, dim, dstate] float32 (None unless want_dh0).  ``grads`` may hold preallocated outputs
    (a dict with the same keys, as returned by an earlier call) to write into.  ``checkpoints``: the
    array selective_scan_fwd_ckpt filled for these inputs (dstate 16), which spares the kernel its own
    forward walk.
    """
    torch = _torch()
    if x.dim() != 3:
        raise ValueError("x must be [batch, seqlen, dim]")
    bsz, L, dm = x.shape
    if A.dim() != 2 or A.shape[0] != dm:
        raise ValueError("A must be [dim, dstate]")
    N = A.shape[1]
    io = _io_code(x.dtype)
    if dout is None:
        raise ValueError("dout is required")
    cur = _torch().cuda.current_device()
    for name, t, shape in (("x", x, (bsz, L, dm)), ("delta", delta, (bsz, L, dm)), ("z", z, (bsz, L, dm)),
                           ("B", B, (bsz, L, N)), ("C", C, (bsz, L, N)), ("dout", dout, (bsz, L, dm))):
        _check_gpu(name, t, x.dtype, shape, cur)
    _check_gpu("A", A, torch.float32, (dm, N), cur)
    _check_gpu("D", D, torch.float32, (dm,), cur)
    _check_gpu("h0", h0, torch.float32, (bsz, dm, N), cur)
    _check_gpu("dfinal", dfinal, torch.float32, (bsz, dm, N), cur)
    if checkpoints is not None:
        d0 = scan_desc(bsz, L, dm, N, io)
        need = lib.mssm_selective_scan_checkpoint_size(ctypes.byref(d0))
        if not checkpoints.is_cuda or checkpoints.dtype != torch.float32 or checkpoints.numel() * 4 < need:
            raise ValueError(f"checkpoints must be a float32 GPU tensor of at least {need} bytes")
    dev = x.device
    g = grads if grads is not None else {
        "dx": torch.empty_like(x), "ddelta": torch.empty_like(x),
        "dz": torch.empty_like(x) if z is not None else None,
        "dB": torch.empty((bsz, L, N), dtype=torch.float32, device=dev),
        "dC": torch.empty((bsz, L, N), dtype=torch.float32, device=dev),
        "dA": torch.empty((dm, N), dtype=torch.float32, device=dev),
        "dD": torch.empty((dm,), dtype=torch.float32, device=dev) if D is not None else None,
        "dh0": torch.empty((bsz, dm, N), dtype=torch.float32, device=dev) if want_dh0 else None,
    }
    if grads is not None:
        for name, dt, shape in (("dx", x.dtype, (bsz, L, dm)), ("ddelta", x.dtype, (bsz, L, dm)),
                                ("dz", x.dtype, (bsz, L, dm)), ("dB", torch.float32, (bsz, L, N)),
                                ("dC", torch.float32, (bsz, L, N)), ("dA", torch.float32, (dm, N)),
                                ("dD", torch.float32, (dm,)), ("dh0", torch.float32, (bsz, dm, N))):
            _check_gpu(name, g.get(name), dt, shape, cur)
    d = scan_desc(bsz, L, dm, N, io)
    ws_bytes = lib.mssm_selective_scan_bwd_workspace_size(ctypes.byref(d))
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    st = lib.mssm_selective_scan_bwd(
        ctypes.byref(d), _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0), _ptr(dout),
        _ptr(dfinal), _ptr(g["dx"]), _ptr(g["ddelta"]), _ptr(g["dA"]), _ptr(g["dB"]), _ptr(g["dC"]), _ptr(g["dD"]),
        _ptr(g["dz"]), _ptr(g["dh0"]), _ptr(checkpoints), _ptr(workspace) if ws_bytes else None,
        workspace.numel() if (ws_bytes and workspace is not None) else 0, _stream_handle(stream))
    if st != MSSM_OK:
        raise MssmError(st, "mssm_selective_scan_bwd")
    return g


def ssd_desc(batch, seqlen, nheads, headdim, dstate, ngroups, chunk=0, io_dtype=MSSM_BF16) -> SSDDesc:
    return SSDDesc(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, io_dtype, 0)


SSD_ROUTE_BLOCK = 0       # the matrix-core block kernel
SSD_ROUTE_RECURRENT = 1   # token by token through the update kernel


def ssd_plan(batch, seqlen, nheads, headdim, dstate, ngroups, chunk=0, io_dtype=MSSM_BF16) -> int:
    """Which kernel the multi-head forward runs this problem on (SSD_ROUTE_BLOCK or SSD_ROUTE_RECURRENT)."""
    d = ssd_desc(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, io_dtype)
    r = ctypes.c_int32(-1)
    st = lib.mssm_ssd_plan(ctypes.byref(d), ctypes.byref(r))
    if st != MSSM_OK:
        raise MssmError(st, "mssm_ssd_plan")
    return r.value


def ssd_workspace_size(batch, seqlen, nheads, headdim, dstate, ngroups, chunk=0) -> int:
    d = ssd_desc(batch, seqlen, nheads, headdim, dstate, ngroups, chunk)
    return lib.mssm_ssd_workspace_size(ctypes.byref(d))


def ssd_fwd(x, delta, A, B, C, D=None, z=None, h0=None, chunk: int = 0, return_final_state: bool = False,
            out=None, final_state=None, workspace=None, stream=None):
    """Mamba-2 scalar-A multi-head forward (mssm_ssd_fwd).

    x, z: [batch, seqlen, nheads, headdim]; delta: [batch, seqlen, nheads]; B, C: [batch, seqlen,
    ngroups, dstate], all bfloat16 or all float32; A, D: [nheads] float32; h0: [batch, nheads, headdim,
    dstate] float32.  bfloat16 with headdim a multiple of 8 and dstate a multiple of 16 up to 256 runs
    on the matrix-core block kernel (above 128 states as two shares of the states, with a workspace);
    anything else (float32, other headdims, other dstate up to 256) on the recurrent kernel, token by
    token.
    """
    return _ssd_call("mssm_ssd_fwd", x, delta, None, A, B, C, D, z, h0, chunk, return_final_state, out,
                     final_state, workspace, stream)


def ssd_trapezoidal_fwd(x, delta, lam, A, B, C, D=None, z=None, h0=None, chunk: int = 0,
                        return_final_state: bool = False, out=None, final_state=None, workspace=None, stream=None):
    """Mamba-3 SISO recurrence, exponential-trapezoidal input rule (mssm_ssd_trapezoidal_fwd).

    As ``ssd_fwd`` plus lam: [batch, seqlen, nheads] in the I/O dtype, the weight of each step's own input (1 - lam
    goes to the previous step's input, carried through the step's decay).  lam = 1 gives ``ssd_fwd``.
    """
    return _ssd_call("mssm_ssd_trapezoidal_fwd", x, delta, lam, A, B, C, D, z, h0, chunk, return_final_state,
                     out, final_state, workspace, stream)


def ssd_mimo_plan(batch, seqlen, nheads, headdim, dstate, ngroups, rank, chunk=0, io_dtype=MSSM_BF16) -> int:
    """Which kernel mssm_ssd_mimo_fwd runs this problem on (SSD_ROUTE_BLOCK or SSD_ROUTE_RECURRENT)."""
    d = ssd_desc(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, io_dtype)
    r = ctypes.c_int32(-1)
    st = lib.mssm_ssd_mimo_plan(ctypes.byref(d), rank, ctypes.byref(r))
    if st != MSSM_OK:
        raise MssmError(st, "mssm_ssd_mimo_plan")
    return r.value


def ssd_mimo_fwd(x, delta, lam, A, B, C, D=None, z=None, h0=None, chunk: int = 0, return_final_state: bool = False,
                 out=None, final_state=None, workspace=None, stream=None):
    """Mamba-3 MIMO (mssm_ssd_mimo_fwd): x, z [batch, seqlen, nheads, rank, headdim]; B, C [batch, seqlen,
    ngroups, rank, dstate]; delta, lam [batch, seqlen, nheads] (lam None: the Mamba-2 rule); A, D [nheads];
    h0 [batch, nheads, headdim, dstate].  Returns out (and the final state when asked)."""
    torch = _torch()
    if x.dim() != 5 or B.dim() != 5:
        raise ValueError("x must be [batch, seqlen, nheads, rank, headdim] and B [batch, seqlen, ngroups, rank, dstate]")
    bsz, L, H, R, P = x.shape
    G, N = B.shape[2], B.shape[4]
    io = _io_code(x.dtype)
    cur = torch.cuda.current_device()
    for name, t, shape in (("x", x, (bsz, L, H, R, P)), ("z", z, (bsz, L, H, R, P)), ("delta", delta, (bsz, L, H)),
                           ("lam", lam, (bsz, L, H)), ("B", B, (bsz, L, G, R, N)), ("C", C, (bsz, L, G, R, N))):
        _check_gpu(name, t, x.dtype, shape, cur)
    _check_gpu("A", A, torch.float32, (H,), cur)
    _check_gpu("D", D, torch.float32, (H,), cur)
    _check_gpu("h0", h0, torch.float32, (bsz, H, P, N), cur)
    if out is None:
        out = torch.empty_like(x)
    _check_gpu("out", out, x.dtype, (bsz, L, H, R, P), cur)
    if return_final_state and final_state is None:
        final_state = torch.empty((bsz, H, P, N), dtype=torch.float32, device=x.device)
    _check_gpu("final_state", final_state, torch.float32, (bsz, H, P, N), cur)
    d = ssd_desc(bsz, L, H, P, N, G, chunk, io)
    ws_bytes = lib.mssm_ssd_workspace_size(ctypes.byref(d))
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=x.device)
    st = lib.mssm_ssd_mimo_fwd(ctypes.byref(d), R, _ptr(x), _ptr(delta), _ptr(lam), _ptr(A), _ptr(B), _ptr(C),
                               _ptr(D), _ptr(z), _ptr(h0), _ptr(out), _ptr(final_state),
                               _ptr(workspace) if ws_bytes else None,
                               workspace.numel() if (ws_bytes and workspace is not None) else 0,
                               _stream_handle(stream))
    if st != MSSM_OK:
        raise MssmError(st, "mssm_ssd_mimo_fwd")
    return (out, final_state) if return_final_state else out


def ssd_mimo_state_update(state, x, delta, lam, A, B, C, D=None, z=None, x_prev=None, B_prev=None, out=None,
                          stream=None):
    """Advance a multi-head state by seqlen tokens in place under Mamba-3 MIMO (mssm_ssd_mimo_state_update).
    x, z [batch, seqlen, nheads, rank, headdim]; B, C [batch, seqlen, ngroups, rank, dstate]; lam None: the
    Mamba-2 rule; x_prev [batch, nheads, rank, headdim], B_prev [batch, ngroups, rank, dstate] (None: no
    previous token).  Returns out."""
    torch = _torch()
    if x.dim() != 5 or B.dim() != 5:
        raise ValueError("x must be [batch, seqlen, nheads, rank, headdim] and B [batch, seqlen, ngroups, rank, dstate]")
    bsz, L, H, R, P = x.shape
    G, N = B.shape[2], B.shape[4]
    io = _io_code(x.dtype)
    cur = torch.cuda.current_device()
    for name, t, shape in (("x", x, (bsz, L, H, R, P)), ("z", z, (bsz, L, H, R, P)), ("delta", delta, (bsz, L, H)),
                           ("lam", lam, (bsz, L, H)), ("B", B, (bsz, L, G, R, N)), ("C", C, (bsz, L, G, R, N)),
                           ("x_prev", x_prev, (bsz, H, R, P)), ("B_prev", B_prev, (bsz, G, R, N))):
        _check_gpu(name, t, x.dtype, shape, cur)
    _check_gpu("A", A, torch.float32, (H,), cur)
    _check_gpu("D", D, torch.float32, (H,), cur)
    _check_gpu("state", state, torch.float32, (bsz, H, P, N), cur)
    if out is None:
        out = torch.empty_like(x)
    _check_gpu("out", out, x.dtype, (bsz, L, H, R, P), cur)
    d = ssd_desc(bsz, L, H, P, N, G, 0, io)
    st = lib.mssm_ssd_mimo_state_update(ctypes.byref(d), R, _ptr(state), _ptr(x_prev), _ptr(B_prev), _ptr(x),
                                        _ptr(delta), _ptr(lam), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                        _ptr(out), _stream_handle(stream))
    if st != MSSM_OK:
        raise MssmError(st, "mssm_ssd_mimo_state_update")
    return out


def _ssd_call(fn, x, delta, lam, A, B, C, D, z, h0, chunk, return_final_state, out, final_state, workspace,
              stream):
    torch = _torch()
    if x.dim() != 4 or B.dim() != 4:
        raise ValueError("x must be [batch, seqlen, nheads, headdim] and B [batch, seqlen, ngroups, dstate]")
    bsz, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    io = _io_code(x.dtype)
    trap = fn == "mssm_ssd_trapezoidal_fwd"
    if trap and lam is None:
        raise ValueError("lam is required")
    cur = _torch().cuda.current_device()
    for name, t, shape in (("x", x, (bsz, L, H, P)), ("z", z, (bsz, L, H, P)), ("delta", delta, (bsz, L, H)),
                           ("lam", lam, (bsz, L, H)), ("B", B, (bsz, L, G, N)), ("C", C, (bsz, L, G, N))):
        _check_gpu(name, t, x.dtype, shape, cur)
    _check_gpu("A", A, torch.float32, (H,), cur)
    _check_gpu("D", D, torch.float32, (H,), cur)
    _check_gpu("h0", h0, torch.float32, (bsz, H, P, N), cur)
    if out is None:
        out = torch.empty_like(x)
    _check_gpu("out", out, x.dtype, (bsz, L, H, P), cur)
    if return_final_state and final_state is None:
        final_state = torch.empty((bsz, H, P, N), dtype=torch.float32, device=x.device)
    _check_gpu("final_state", final_state, torch.float32, (bsz, H, P, N), cur)
    d = ssd_desc(bsz, L, H, P, N, G, chunk, io)
    ws_bytes = lib.mssm_ssd_workspace_size(ctypes.byref(d))
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=x.device)
    ws = (_ptr(workspace) if ws_bytes else None,
          workspace.numel() if (ws_bytes and workspace is not None) else 0, _stream_handle(stream))
    if trap:
        st = lib.mssm_ssd_trapezoidal_fwd(ctypes.byref(d), _ptr(x), _ptr(delta), _ptr(lam), _ptr(A), _ptr(B),
                                          _ptr(C), _ptr(D), _ptr(z), _ptr(h0), _ptr(out), _ptr(final_state), *ws)
    else:
        st = lib.mssm_ssd_fwd(ctypes.byref(d), _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                              _ptr(h0), _ptr(out), _ptr(final_state), *ws)
    if st != MSSM_OK:
        raise MssmError(st, fn)
    return (out, final_state) if return_final_state else out


def selective_state_update(state, x, delta, A, B, C, D=None, z=None, out=None, stream=None):
    """Advance a Mamba-1 state by seqlen tokens in place (mssm_selective_state_update).

    state: [batch, dim, dstate] float32 (overwritten); x, delta, z: [batch, seqlen, dim];
    B, C: [batch, seqlen, dstate] (float32 or bfloat16, all alike); A: [dim, dstate]; D: [dim].
    Returns out [batch, seqlen, dim].
    """
    torch = _torch()
    if x.dim() != 3:
        raise ValueError("x must be [batch, seqlen, dim]")
    bsz, L, dm = x.shape
    if A.dim() != 2 or A.shape[0] != dm:
        raise ValueError("A must be [dim, dstate]")
    N = A.shape[1]
    io = _io_code(x.dtype)
    cur = _torch().cuda.current_device()
    for name, t, shape in (("x", x, (bsz, L, dm)), ("delta", delta, (bsz, L, dm)), ("z", z, (bsz, L, dm)),
                           ("B", B, (bsz, L, N)), ("C", C, (bsz, L, N))):
        _check_gpu(name, t, x.dtype, shape, cur)
    _check_gpu("A", A, torch.float32, (dm, N), cur)
    _check_gpu("D", D, torch.float32, (dm,), cur)
    _check_gpu("state", state, torch.float32, (bsz, dm, N), cur)
    if out is None:
        out = torch.empty_like(x)
    _check_gpu("out", out, x.dtype, (bsz, L, dm), cur)
    d = scan_desc(bsz, L, dm, N, io)
    st = lib.mssm_selective_state_update(ctypes.byref(d), _ptr(state), _ptr(x), _ptr(delta), _ptr(A), _ptr(B),
                                         _ptr(C), _ptr(D), _ptr(z), _ptr(out), _stream_handle(stream))
    if st != MSSM_OK:
        raise MssmError(st, "mssm_selective_state_update")
    return out


def selective_state_update_conv(state, conv_state, xin, conv_w, conv_b, delta, A, B, C, D=None, z=None, out=None,
                                stream=None):
    """Token-by-token update with the short causal convolution in front (mssm_selective_state_update_conv).

    state [batch, dim, dstate] float32 and conv_state [batch, W-1, dim] (xin's dtype; None when W == 1) are
    advanced in place; xin, delta, z: [batch, T, dim]; conv_w [dim, W] float32; conv_b [dim] or None.
    Returns out [batch, T, dim]."""
    torch = _torch()
    if xin.dim() != 3:
        raise ValueError("xin must be [batch, tokens, dim]")
    bsz, T, dm = xin.shape
    N = A.shape[1]
    W = conv_w.shape[1]
    io = _io_code(xin.dtype)
    cur = _torch().cuda.current_device()
    for name, t, shape in (("xin", xin, (bsz, T, dm)), ("delta", delta, (bsz, T, dm)), ("z", z, (bsz, T, dm)),
                           ("B", B, (bsz, T, N)), ("C", C, (bsz, T, N)),
                           ("conv_state", conv_state, (bsz, W - 1, dm))):
        _check_gpu(name, t, xin.dtype, shape, cur)
    _check_gpu("state", state, torch.float32, (bsz, dm, N), cur)
    _check_gpu("conv_w", conv_w, torch.float32, (dm, W), cur)
    _check_gpu("conv_b", conv_b, torch.float32, (dm,), cur)
    _check_gpu("A", A, torch.float32, (dm, N), cur)
    _check_gpu("D", D, torch.float32, (dm,), cur)
    if out is None:
        out = torch.empty_like(xin)
    _check_gpu("out", out, xin.dtype, (bsz, T, dm), cur)
    d = scan_desc(bsz, T, dm, N, io)
    st = lib.mssm_selective_state_update_conv(ctypes.byref(d), W, _ptr(state), _ptr(conv_state), _ptr(xin),
                                              _ptr(conv_w), _ptr(conv_b), _ptr(delta), _ptr(A), _ptr(B), _ptr(C),
                                              _ptr(D), _ptr(z), _ptr(out), _stream_handle(stream))
    if st != MSSM_OK:
        raise MssmError(st, "mssm_selective_state_update_conv")
    return out


def ssd_state_update(state, x, delta, A, B, C, D=None, z=None, out=None, stream=None):
    """Advance a multi-head (scalar A) state by seqlen tokens in place (mssm_ssd_state_update).

    state: [batch, nheads, headdim, dstate] float32 (overwritten); x, z: [batch, seqlen, nheads, headdim];
    delta: [batch, seqlen, nheads]; B, C: [batch, seqlen, ngroups, dstate]; A, D: [nheads].
    Returns out [batch, seqlen, nheads, headdim].
    """
    return _ssd_update_call("mssm_ssd_state_update", state, None, None, x, delta, None, A, B, C, D, z, out, stream)


def ssd_trapezoidal_state_update(state, x, delta, lam, A, B, C, D=None, z=None, x_prev=None, B_prev=None,
                                 out=None, stream=None):
    """Advance a multi-head state by seqlen tokens in place under the Mamba-3 SISO rule
    (mssm_ssd_trapezoidal_state_update).

    As ``ssd_state_update`` plus lam [batch, seqlen, nheads] and the previous token's x_prev
    [batch, nheads, headdim] and B_prev [batch, ngroups, dstate] (None: no previous token).
    """
    return _ssd_update_call("mssm_ssd_trapezoidal_state_update", state, x_prev, B_prev, x, delta, lam, A, B, C, D,
                            z, out, stream)


def mamba3_siso_update(state, x, delta, lam, A, omega, B, C, D=None, z=None, x_prev=None, B_prev=None, out=None,
                       stream=None):
    """Advance a multi-head state by seqlen tokens in place under the Mamba-3 SISO recurrence with a
    complex-valued state (mssm_mamba3_siso_update): the exponential-trapezoidal rule, each state pair
    rotated by delta * omega per step.

    As ``ssd_trapezoidal_state_update`` plus omega [nheads, dstate / 2] float32; dstate must be even.
    With seqlen = L it is also the sequence form (state in: h0; state out: the final state).
    """
    return _ssd_update_call("mssm_mamba3_siso_update", state, x_prev, B_prev, x, delta, lam, A, B, C, D, z, out,
                            stream, omega=omega)


def _ssd_update_call(fn, state, x_prev, B_prev, x, delta, lam, A, B, C, D, z, out, stream, omega=None):
    torch = _torch()
    if x.dim() != 4:
        raise ValueError("x must be [batch, seqlen, nheads, headdim]")
    bsz, L, H, P = x.shape
    if B.dim() != 4:
        raise ValueError("B must be [batch, seqlen, ngroups, dstate]")
    G, N = B.shape[2], B.shape[3]
    io = _io_code(x.dtype)
    trap = fn in ("mssm_ssd_trapezoidal_state_update", "mssm_mamba3_siso_update")
    if trap and lam is None:
        raise ValueError("lam is required")
    if fn == "mssm_mamba3_siso_update" and omega is None:
        raise ValueError("omega is required")
    cur = _torch().cuda.current_device()
    for name, t, shape in (("x", x, (bsz, L, H, P)), ("z", z, (bsz, L, H, P)), ("delta", delta, (bsz, L, H)),
                           ("lam", lam, (bsz, L, H)), ("B", B, (bsz, L, G, N)), ("C", C, (bsz, L, G, N)),
                           ("x_prev", x_prev, (bsz, H, P)), ("B_prev", B_prev, (bsz, G, N))):
        _check_gpu(name, t, x.dtype, shape, cur)
    _check_gpu("A", A, torch.float32, (H,), cur)
    _check_gpu("D", D, torch.float32, (H,), cur)
    _check_gpu("state", state, torch.float32, (bsz, H, P, N), cur)
    _check_gpu("omega", omega, torch.float32, (H, N // 2), cur)
    if out is None:
        out = torch.empty_like(x)
    _check_gpu("out", out, x.dtype, (bsz, L, H, P), cur)
    d = ssd_desc(bsz, L, H, P, N, G, 0, io)
    if fn == "mssm_mamba3_siso_update":
        st = lib.mssm_mamba3_siso_update(ctypes.byref(d), _ptr(state), _ptr(x_prev), _ptr(B_prev), _ptr(x),
                                         _ptr(delta), _ptr(lam), _ptr(A), _ptr(omega), _ptr(B), _ptr(C), _ptr(D),
                                         _ptr(z), _ptr(out), _stream_handle(stream))
    elif trap:
        st = lib.mssm_ssd_trapezoidal_state_update(ctypes.byref(d), _ptr(state), _ptr(x_prev), _ptr(B_prev), _ptr(x),
                                                   _ptr(delta), _ptr(lam), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                                   _ptr(z), _ptr(out), _stream_handle(stream))
    else:
        st = lib.mssm_ssd_state_update(ctypes.byref(d), _ptr(state), _ptr(x), _ptr(delta), _ptr(A), _ptr(B),
                                       _ptr(C), _ptr(D), _ptr(z), _ptr(out), _stream_handle(stream))
    if st != MSSM_OK:
        raise MssmError(st, fn)
    return out
