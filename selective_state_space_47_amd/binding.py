"""Thin ctypes binding over the C ABI in include/mamba_scan.h.

Argument marshalling only: checks dtypes, shapes and devices, allocates outputs and workspace with
torch, passes raw device pointers and torch's current HIP stream to the library.  Every step of
the computation runs in the library's kernels.  There is no fallback: if the native library is
missing the first call raises.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import threading

import torch

from . import _build

MAMBA_F32 = 0
MAMBA_BF16 = 1
DSTATE = 16

_lock = threading.Lock()
_LIB = None


class mamba_block_dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64),
                ("d_model", ctypes.c_int64), ("d_inner", ctypes.c_int64),
                ("dstate", ctypes.c_int64), ("dt_rank", ctypes.c_int64),
                ("conv_width", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class mamba_dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("dim", ctypes.c_int64), ("dstate", ctypes.c_int64),
                ("seqlen", ctypes.c_int64), ("io_dtype", ctypes.c_int32),
                ("chunk_len", ctypes.c_int32)]


EXPORTS = ("mamba_scan_fwd", "mamba_scan_fwd_noalloc", "mamba_scan_fwd_conv", "mamba_state_update",
           "mamba_scan_workspace_bytes",
           "mamba_scan_bwd", "mamba_scan_bwd_workspace_bytes", "mamba_gemm_bf16",
           "mamba_block_fwd", "mamba_block_workspace_bytes", "mamba_status_string",
           "mamba_abi_version")


def library_path() -> str:
    return _build.LIB_PATH


def lib():
    """The loaded native library (raises RuntimeError if it has not been built)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    with _lock:
        if _LIB is None:
            path = library_path()
            if not os.path.exists(path):
                raise RuntimeError(
                    f"native library {path} is missing: build it with "
                    "`python -c 'import __graft_entry__ as g; g.build()'` (hipcc, gfx950)")
            L = ctypes.CDLL(path)
            vp, fp = ctypes.c_void_p, ctypes.c_void_p
            dp = ctypes.POINTER(mamba_dims)
            L.mamba_scan_fwd.argtypes = [vp, vp, fp, vp, vp, fp, vp, fp, ctypes.c_int, vp, fp, dp,
                                         vp, ctypes.c_size_t, vp]
            L.mamba_scan_fwd.restype = ctypes.c_int
            L.mamba_scan_fwd_noalloc.argtypes = [vp, vp, fp, vp, vp, fp, vp, fp, ctypes.c_int, vp,
                                                 fp, dp, vp]
            L.mamba_scan_fwd_noalloc.restype = ctypes.c_int
            L.mamba_scan_fwd_conv.argtypes = [vp, fp, fp, ctypes.c_int, vp, fp, vp, vp, fp, vp,
                                              fp, ctypes.c_int, vp, fp, vp, dp, vp,
                                              ctypes.c_size_t, vp]
            L.mamba_scan_fwd_conv.restype = ctypes.c_int
            L.mamba_state_update.argtypes = [fp, vp, vp, fp, vp, vp, fp, vp, fp, ctypes.c_int, vp,
                                             dp, vp]
            L.mamba_state_update.restype = ctypes.c_int
            L.mamba_scan_workspace_bytes.argtypes = [dp]
            L.mamba_scan_workspace_bytes.restype = ctypes.c_size_t
            L.mamba_scan_bwd.argtypes = [vp, vp, fp, vp, vp, fp, vp, fp, ctypes.c_int, vp, fp,
                                         vp, vp, fp, vp, vp, fp, vp, fp, dp, vp,
                                         ctypes.c_size_t, vp]
            L.mamba_scan_bwd.restype = ctypes.c_int
            L.mamba_scan_bwd_workspace_bytes.argtypes = [dp]
            L.mamba_scan_bwd_workspace_bytes.restype = ctypes.c_size_t
            i64 = ctypes.c_int64
            L.mamba_gemm_bf16.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, i64,
                                          i64, ctypes.c_int, ctypes.c_int, vp]
            L.mamba_gemm_bf16.restype = ctypes.c_int
            bp = ctypes.POINTER(mamba_block_dims)
            L.mamba_block_fwd.argtypes = [vp, vp, fp, fp, vp, vp, fp, fp, fp, vp, vp, bp, vp,
                                          ctypes.c_size_t, vp]
            L.mamba_block_fwd.restype = ctypes.c_int
            L.mamba_block_workspace_bytes.argtypes = [bp]
            L.mamba_block_workspace_bytes.restype = ctypes.c_size_t
            L.mamba_status_string.argtypes = [ctypes.c_int]
            L.mamba_status_string.restype = ctypes.c_char_p
            L.mamba_abi_version.argtypes = []
            L.mamba_abi_version.restype = ctypes.c_int
            _LIB = L
    return _LIB


def mamba_status_string(status: int) -> str:
    return lib().mamba_status_string(int(status)).decode()


def mamba_abi_version() -> int:
    return int(lib().mamba_abi_version())


def _io_code(dtype) -> int:
    if dtype == torch.float32:
        return MAMBA_F32
    if dtype == torch.bfloat16:
        return MAMBA_BF16
    raise ValueError(f"unsupported io dtype {dtype}; use float32 or bfloat16")


def make_dims(batch, dim, seqlen, io_dtype, dstate=DSTATE, chunk_len=0) -> mamba_dims:
    return mamba_dims(int(batch), int(dim), int(dstate), int(seqlen), int(io_dtype),
                      int(chunk_len))


def mamba_scan_workspace_bytes(batch, dim, seqlen, io_dtype=torch.float32, dstate=DSTATE,
                               chunk_len=0) -> int:
    code = io_dtype if isinstance(io_dtype, int) else _io_code(io_dtype)
    dm = make_dims(batch, dim, seqlen, code, dstate, chunk_len)
    return int(lib().mamba_scan_workspace_bytes(ctypes.byref(dm)))


def _ptr(t):
    # a plain int: the c_void_p argtypes convert it, which is cheaper than a c_void_p object
    return None if t is None else t.data_ptr()


# torch's own accessor of the current stream's raw handle (one C call); the public path builds a
# Stream object per call, which costs more host time than a short scan's kernel
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(dev):
    """Raw handle of the current stream on `dev`, as an int."""
    if _raw_stream is not None:
        return _raw_stream(dev.index)
    return torch.cuda.current_stream(dev).cuda_stream


# dims structs (read-only for the library) and the forward's workspace size, per shape; short
# sequences are called at a high rate with the same shape
_FWD_CACHE = {}


def _fwd_dims(batch, dim, L, code, chunk_len):
    key = (batch, dim, L, code, chunk_len)
    hit = _FWD_CACHE.get(key)
    if hit is None:
        dm = make_dims(batch, dim, L, code, DSTATE, chunk_len)
        hit = (dm, int(lib().mamba_scan_workspace_bytes(ctypes.byref(dm))))
        if len(_FWD_CACHE) >= 1024:
            _FWD_CACHE.clear()
        _FWD_CACHE[key] = hit
    return hit


def _check(t, name, shape, dtype, device):
    if t is None:
        return
    # fast path: one combined test for a well-formed tensor (the per-call host overhead matters
    # for short sequences); anything else goes through the detailed checks below
    if (type(t) is torch.Tensor and t.dtype is dtype and t.shape == shape
            and t.get_device() == device.index and t.is_contiguous()):
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_group(tensors, shape, dtype, device):
    """_check for several (tensor, name) pairs of one shape and dtype; the common case (all
    well-formed) costs one Python call instead of one per tensor."""
    idx = device.index
    for t, name in tensors:
        if t is not None and not (type(t) is torch.Tensor and t.dtype is dtype
                                  and t.shape == shape and t.get_device() == idx
                                  and t.is_contiguous()):
            _check(t, name, shape, dtype, device)


_NO_SWITCH = contextlib.nullcontext()


def _on(dev):
    """Context making `dev` current for a call; nothing to switch when it already is."""
    return _NO_SWITCH if torch.cuda.current_device() == dev.index else torch.cuda.device(dev)


def _raise(status):
    if status != 0:
        raise ValueError(f"mamba library error {status}: {mamba_status_string(status)}")


def _workspace(workspace, need, dev, min_bytes=0):
    """The caller's workspace, checked, or a new one of `need` bytes (at least min_bytes).
    Returns (tensor or None, its size in bytes)."""
    if workspace is None:
        n = max(need, min_bytes)
        if n == 0:
            return None, 0
        workspace = torch.empty(n, dtype=torch.uint8, device=dev)
    if not isinstance(workspace, torch.Tensor):
        raise TypeError("workspace must be a torch.Tensor")
    if workspace.device != dev or not workspace.is_contiguous():
        raise ValueError(f"workspace must be a contiguous tensor on {dev}")
    return workspace, workspace.numel() * workspace.element_size()


def mamba_scan_fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=False,
                   return_last_state=False, chunk_len=0, out=None, last_state=None,
                   workspace=None):
    """Selective-scan forward (see mamba_scan_fwd in include/mamba_scan.h).

    u, delta, z: (batch, dim, L); B, C: (batch, 16, L) -- all float32 or all bfloat16;
    A: (dim, 16) float32; D, delta_bias: (dim,) float32.  Returns out, or (out, last_state).
    """
    if u.dim() != 3:
        raise ValueError("u must be (batch, dim, seqlen)")
    batch, dim, L = u.shape
    dev = u.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a HIP device")
    io = u.dtype
    code = _io_code(io)
    if out is None:
        out = torch.empty((batch, dim, L), dtype=io, device=dev)
    if return_last_state and last_state is None:
        last_state = torch.empty((batch, dim, DSTATE), dtype=torch.float32, device=dev)
    _check_group(((u, "u"), (delta, "delta"), (z, "z"), (out, "out")), (batch, dim, L), io, dev)
    _check_group(((B, "B"), (C, "C")), (batch, DSTATE, L), io, dev)
    _check(A, "A", (dim, DSTATE), torch.float32, dev)
    _check_group(((D, "D"), (delta_bias, "delta_bias")), (dim,), torch.float32, dev)
    _check(last_state, "last_state", (batch, dim, DSTATE), torch.float32, dev)
    dm, ws_bytes = _fwd_dims(batch, dim, L, code, chunk_len)
    L_ = lib()
    workspace, ws_len = _workspace(workspace, ws_bytes, dev)
    with _on(dev):
        stream = _stream(dev)
        st = L_.mamba_scan_fwd(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                               _ptr(z), _ptr(delta_bias), int(bool(delta_softplus)), _ptr(out),
                               _ptr(last_state), ctypes.byref(dm), _ptr(workspace), ws_len,
                               stream)
    _raise(st)
    return (out, last_state) if return_last_state else out


def mamba_scan_fwd_noalloc(u, delta, A, B, C, D=None, z=None, delta_bias=None,
                           delta_softplus=False, return_last_state=False, chunk_len=0, out=None,
                           last_state=None):
    """mamba_scan_fwd_noalloc of include/mamba_scan.h: the forward with its chunk records in the
    library's fixed per-GPU scratch array (no workspace).  Arguments and results as for
    mamba_scan_fwd; outputs are allocated here only when not passed in."""
    if u.dim() != 3:
        raise ValueError("u must be (batch, dim, seqlen)")
    batch, dim, L = u.shape
    dev = u.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a HIP device")
    io = u.dtype
    code = _io_code(io)
    for t, name, shape, dt in ((u, "u", (batch, dim, L), io), (delta, "delta", (batch, dim, L), io),
                               (z, "z", (batch, dim, L), io), (B, "B", (batch, DSTATE, L), io),
                               (C, "C", (batch, DSTATE, L), io),
                               (A, "A", (dim, DSTATE), torch.float32),
                               (D, "D", (dim,), torch.float32),
                               (delta_bias, "delta_bias", (dim,), torch.float32)):
        _check(t, name, shape, dt, dev)
    if out is None:
        out = torch.empty((batch, dim, L), dtype=io, device=dev)
    _check(out, "out", (batch, dim, L), io, dev)
    if return_last_state and last_state is None:
        last_state = torch.empty((batch, dim, DSTATE), dtype=torch.float32, device=dev)
    _check(last_state, "last_state", (batch, dim, DSTATE), torch.float32, dev)
    dm = _fwd_dims(batch, dim, L, code, chunk_len)[0]
    with _on(dev):
        stream = _stream(dev)
        st = lib().mamba_scan_fwd_noalloc(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C),
                                          _ptr(D), _ptr(z), _ptr(delta_bias),
                                          int(bool(delta_softplus)), _ptr(out), _ptr(last_state),
                                          ctypes.byref(dm), stream)
    _raise(st)
    return (out, last_state) if return_last_state else out


def mamba_scan_fwd_conv(x, conv_weight, delta, A, B, C, D=None, z=None, delta_bias=None,
                        delta_softplus=False, conv_bias=None, return_last_state=False,
                        return_u=False, chunk_len=0, out=None, last_state=None, u_out=None,
                        workspace=None):
    """Forward with the causal conv1d + SiLU fused into the load stage (mamba_scan_fwd_conv in
    include/mamba_scan.h).  x: (batch, dim, L) like u of mamba_scan_fwd; conv_weight: (dim, W)
    float32, W in 1..4; conv_bias: (dim,) float32 or None.  Returns out, plus last_state and/or
    u when requested, in that order."""
    if x.dim() != 3:
        raise ValueError("x must be (batch, dim, seqlen)")
    batch, dim, L = x.shape
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a HIP device")
    io = x.dtype
    code = _io_code(io)
    if conv_weight is None or conv_weight.dim() != 2:
        raise ValueError("conv_weight must be (dim, width)")
    width = conv_weight.shape[1]
    _check(x, "x", (batch, dim, L), io, dev)
    _check(conv_weight, "conv_weight", (dim, width), torch.float32, dev)
    _check(conv_bias, "conv_bias", (dim,), torch.float32, dev)
    _check(delta, "delta", (batch, dim, L), io, dev)
    _check(z, "z", (batch, dim, L), io, dev)
    _check(B, "B", (batch, DSTATE, L), io, dev)
    _check(C, "C", (batch, DSTATE, L), io, dev)
    _check(A, "A", (dim, DSTATE), torch.float32, dev)
    _check(D, "D", (dim,), torch.float32, dev)
    _check(delta_bias, "delta_bias", (dim,), torch.float32, dev)
    if out is None:
        out = torch.empty((batch, dim, L), dtype=io, device=dev)
    _check(out, "out", (batch, dim, L), io, dev)
    if return_last_state and last_state is None:
        last_state = torch.empty((batch, dim, DSTATE), dtype=torch.float32, device=dev)
    _check(last_state, "last_state", (batch, dim, DSTATE), torch.float32, dev)
    if return_u and u_out is None:
        u_out = torch.empty((batch, dim, L), dtype=io, device=dev)
    _check(u_out, "u_out", (batch, dim, L), io, dev)
    dm = make_dims(batch, dim, L, code, DSTATE, chunk_len)
    L_ = lib()
    ws_bytes = int(L_.mamba_scan_workspace_bytes(ctypes.byref(dm)))
    workspace, ws_len = _workspace(workspace, ws_bytes, dev)
    with _on(dev):
        stream = _stream(dev)
        st = L_.mamba_scan_fwd_conv(_ptr(x), _ptr(conv_weight), _ptr(conv_bias), int(width),
                                    _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                    _ptr(delta_bias), int(bool(delta_softplus)), _ptr(out),
                                    _ptr(last_state), _ptr(u_out), ctypes.byref(dm),
                                    _ptr(workspace), ws_len, stream)
    _raise(st)
    res = [out]
    if return_last_state:
        res.append(last_state)
    if return_u:
        res.append(u_out)
    return res[0] if len(res) == 1 else tuple(res)


def mamba_state_update(state, u, delta, A, B, C, D=None, z=None, delta_bias=None,
                       delta_softplus=False, out=None):
    """One generation step (see mamba_state_update in include/mamba_scan.h).

    state: (batch, dim, 16) float32, updated in place; u, delta, z: (batch, dim);
    B, C: (batch, 16); A: (dim, 16) float32; D, delta_bias: (dim,) float32.  Returns out.
    """
    if state.dim() != 3:
        raise ValueError("state must be (batch, dim, 16)")
    batch, dim, _ = state.shape
    dev = state.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a HIP device")
    io = u.dtype
    code = _io_code(io)
    _check(state, "state", (batch, dim, DSTATE), torch.float32, dev)
    _check(u, "u", (batch, dim), io, dev)
    _check(delta, "delta", (batch, dim), io, dev)
    _check(z, "z", (batch, dim), io, dev)
    _check(B, "B", (batch, DSTATE), io, dev)
    _check(C, "C", (batch, DSTATE), io, dev)
    _check(A, "A", (dim, DSTATE), torch.float32, dev)
    _check(D, "D", (dim,), torch.float32, dev)
    _check(delta_bias, "delta_bias", (dim,), torch.float32, dev)
    if out is None:
        out = torch.empty((batch, dim), dtype=io, device=dev)
    _check(out, "out", (batch, dim), io, dev)
    dm = _fwd_dims(batch, dim, 1, code, 0)[0]
    with _on(dev):
        stream = _stream(dev)
        st = lib().mamba_state_update(_ptr(state), _ptr(u), _ptr(delta), _ptr(A), _ptr(B),
                                      _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
                                      int(bool(delta_softplus)), _ptr(out), ctypes.byref(dm),
                                      stream)
    _raise(st)
    return out


def mamba_scan_bwd_workspace_bytes(batch, dim, seqlen, io_dtype=torch.float32, dstate=DSTATE,
                                   chunk_len=0) -> int:
    code = io_dtype if isinstance(io_dtype, int) else _io_code(io_dtype)
    dm = make_dims(batch, dim, seqlen, code, dstate, chunk_len)
    return int(lib().mamba_scan_bwd_workspace_bytes(ctypes.byref(dm)))


def mamba_scan_bwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=False,
                   dout=None, dlast=None, chunk_len=0, workspace=None, grads=None):
    """Gradients of mamba_scan_fwd (see mamba_scan_bwd in include/mamba_scan.h).

    Same inputs as mamba_scan_fwd plus dout (batch, dim, L) in the io dtype and optionally dlast
    (batch, dim, 16) float32.  Returns a dict with du, ddelta, dz (io dtype, dz None without z),
    dB, dC (io dtype), dA, dD, ddelta_bias (float32; dD / ddelta_bias None when D / delta_bias is
    None).  `grads` may hold preallocated output tensors under the same keys.
    """
    if u.dim() != 3:
        raise ValueError("u must be (batch, dim, seqlen)")
    batch, dim, L = u.shape
    dev = u.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a HIP device")
    io = u.dtype
    code = _io_code(io)
    if dout is None:
        raise ValueError("dout is required")
    for t, name, shape in ((u, "u", (batch, dim, L)), (delta, "delta", (batch, dim, L)),
                           (z, "z", (batch, dim, L)), (dout, "dout", (batch, dim, L)),
                           (B, "B", (batch, DSTATE, L)), (C, "C", (batch, DSTATE, L))):
        _check(t, name, shape, io, dev)
    _check(A, "A", (dim, DSTATE), torch.float32, dev)
    _check(D, "D", (dim,), torch.float32, dev)
    _check(delta_bias, "delta_bias", (dim,), torch.float32, dev)
    _check(dlast, "dlast", (batch, dim, DSTATE), torch.float32, dev)
    g = dict(grads or {})
    spec = {"du": ((batch, dim, L), io), "ddelta": ((batch, dim, L), io),
            "dB": ((batch, DSTATE, L), io), "dC": ((batch, DSTATE, L), io),
            "dA": ((dim, DSTATE), torch.float32)}
    if z is not None:
        spec["dz"] = ((batch, dim, L), io)
    if D is not None:
        spec["dD"] = ((dim,), torch.float32)
    if delta_bias is not None:
        spec["ddelta_bias"] = ((dim,), torch.float32)
    for k, (shape, dt) in spec.items():
        if g.get(k) is None:
            g[k] = torch.empty(shape, dtype=dt, device=dev)
        _check(g[k], k, shape, dt, dev)
    for k in ("dz", "dD", "ddelta_bias"):
        if k not in spec:
            g[k] = None
    dm = make_dims(batch, dim, L, code, DSTATE, chunk_len)
    L_ = lib()
    ws_bytes = int(L_.mamba_scan_bwd_workspace_bytes(ctypes.byref(dm)))
    workspace, ws_len = _workspace(workspace, ws_bytes, dev, min_bytes=1)
    with _on(dev):
        stream = _stream(dev)
        st = L_.mamba_scan_bwd(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                               _ptr(z), _ptr(delta_bias), int(bool(delta_softplus)), _ptr(dout),
                               _ptr(dlast), _ptr(g["du"]), _ptr(g["ddelta"]), _ptr(g["dA"]),
                               _ptr(g["dB"]), _ptr(g["dC"]), _ptr(g["dD"]), _ptr(g["dz"]),
                               _ptr(g["ddelta_bias"]), ctypes.byref(dm), _ptr(workspace),
                               ws_len, stream)
    _raise(st)
    return {k: g[k] for k in ("du", "ddelta", "dz", "dA", "dB", "dC", "dD", "ddelta_bias")}


def mamba_gemm_bf16(A, B, b_kcontig=True, c_trans=False, out=None):
    """Batched bf16 GEMM on the matrix cores (mamba_gemm_bf16 in include/mamba_scan.h).

    A: (M, K) bfloat16.  B: (batch, N, K) when b_kcontig (element (k, n) = B[b, n, k]), else
    (batch, K, N).  Returns C: (batch, M, N), or (batch, N, M) when c_trans, bfloat16.
    """
    if A.dim() != 2 or B.dim() != 3:
        raise ValueError("A must be (M, K) and B (batch, N, K) or (batch, K, N)")
    M, K = A.shape
    batch = B.shape[0]
    N = B.shape[1] if b_kcontig else B.shape[2]
    dev = A.device
    _check(A, "A", (M, K), torch.bfloat16, dev)
    _check(B, "B", (batch, N, K) if b_kcontig else (batch, K, N), torch.bfloat16, dev)
    shape = (batch, N, M) if c_trans else (batch, M, N)
    if out is None:
        out = torch.empty(shape, dtype=torch.bfloat16, device=dev)
    _check(out, "out", shape, torch.bfloat16, dev)
    ldb = K if b_kcontig else N
    ldc = M if c_trans else N
    with _on(dev):
        stream = _stream(dev)
        st = lib().mamba_gemm_bf16(_ptr(A), _ptr(B), _ptr(out), M, N, K, batch, K, ldb, N * K,
                                   ldc, M * N, int(bool(b_kcontig)), int(bool(c_trans)), stream)
    _raise(st)
    return out


def block_dims(hidden, w_in, w_x, w_dt, conv_weight, dstate=DSTATE) -> mamba_block_dims:
    batch, L, d_model = hidden.shape
    E = w_in.shape[0] // 2
    R = w_dt.shape[1]
    return mamba_block_dims(int(batch), int(L), int(d_model), int(E), int(dstate), int(R),
                            int(conv_weight.shape[1]), 0)


def mamba_block_workspace_bytes(dims: mamba_block_dims) -> int:
    return int(lib().mamba_block_workspace_bytes(ctypes.byref(dims)))


def mamba_block_fwd(hidden, w_in, conv_weight, conv_bias, w_x, w_dt, dt_bias, A, D, w_out,
                    out=None, workspace=None):
    """A Mamba block forward (mamba_block_fwd in include/mamba_scan.h).

    hidden: (batch, L, d_model) bf16; w_in (2E, d_model), w_x (R + 32, E), w_dt (E, R),
    w_out (d_model, E) bf16; conv_weight (E, W), conv_bias (E,), dt_bias (E,), A (E, 16), D (E,)
    float32 (conv_bias, dt_bias, D may be None).  Returns out (batch, L, d_model) bf16.
    """
    if hidden.dim() != 3:
        raise ValueError("hidden must be (batch, seqlen, d_model)")
    batch, L, d_model = hidden.shape
    dev = hidden.device
    E = w_in.shape[0] // 2
    R = w_dt.shape[1] if w_dt.dim() == 2 else -1
    bf, f32 = torch.bfloat16, torch.float32
    _check(hidden, "hidden", (batch, L, d_model), bf, dev)
    _check(w_in, "w_in", (2 * E, d_model), bf, dev)
    _check(w_x, "w_x", (R + 2 * DSTATE, E), bf, dev)
    _check(w_dt, "w_dt", (E, R), bf, dev)
    _check(w_out, "w_out", (d_model, E), bf, dev)
    if conv_weight is None or conv_weight.dim() != 2:
        raise ValueError("conv_weight must be (d_inner, width)")
    _check(conv_weight, "conv_weight", (E, conv_weight.shape[1]), f32, dev)
    _check(conv_bias, "conv_bias", (E,), f32, dev)
    _check(dt_bias, "dt_bias", (E,), f32, dev)
    _check(A, "A", (E, DSTATE), f32, dev)
    _check(D, "D", (E,), f32, dev)
    if out is None:
        out = torch.empty((batch, L, d_model), dtype=bf, device=dev)
    _check(out, "out", (batch, L, d_model), bf, dev)
    dm = block_dims(hidden, w_in, w_x, w_dt, conv_weight)
    L_ = lib()
    ws_bytes = int(L_.mamba_block_workspace_bytes(ctypes.byref(dm)))
    workspace, ws_len = _workspace(workspace, ws_bytes, dev, min_bytes=1)
    with _on(dev):
        stream = _stream(dev)
        st = L_.mamba_block_fwd(_ptr(hidden), _ptr(w_in), _ptr(conv_weight), _ptr(conv_bias),
                                _ptr(w_x), _ptr(w_dt), _ptr(dt_bias), _ptr(A), _ptr(D),
                                _ptr(w_out), _ptr(out), ctypes.byref(dm), _ptr(workspace),
                                ws_len, stream)
    _raise(st)
    return out
