"""fp64 CPU oracle for Mamba's selective scan and single-token state update.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the benchmark's CPU-baseline
leg may import this package.  It shares no code with the GPU library and never imports it; the
only module both sides use is the seeded input generator, which holds none of the method's
arithmetic.

The arithmetic lives in ``mamba_oracle.c`` (plain sequential recurrence in double precision, see
that file's header for the page passages it follows).  This wrapper builds it with gcc, converts
inputs to float64 (exact for fp32 and bf16 values) and calls it through ctypes.

Every function here is pinned by tests against values the pages print, closed forms, brute force
and library special cases; see the oracle pin tests.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mamba_oracle.c")
_BUILD_DIR = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_BUILD_DIR, "libmamba_oracle.so")
_lock = threading.Lock()
_lib = None


def build_oracle(force: bool = True) -> str:
    """Compile the C oracle into a shared library (gcc, -O2, OpenMP). Returns its path."""
    os.makedirs(_BUILD_DIR, exist_ok=True)
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
               "-ffp-contract=off", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                build_oracle(force=False)
            lib = ctypes.CDLL(_LIB_PATH)
            dp = ctypes.POINTER(ctypes.c_double)
            i64 = ctypes.c_int64
            lib.ref_scan_fwd_f64.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp, ctypes.c_int,
                                             i64, i64, i64, i64, dp, dp]
            lib.ref_scan_fwd_f64.restype = None
            lib.ref_state_update_f64.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp, dp, ctypes.c_int,
                                                 i64, i64, i64, dp]
            lib.ref_state_update_f64.restype = None
            lib.ref_scan_bwd_f64.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp, ctypes.c_int, dp,
                                             dp, i64, i64, i64, i64, dp, dp, dp, dp, dp, dp, dp,
                                             dp]
            lib.ref_scan_bwd_f64.restype = None
            lib.ref_causal_conv1d_silu_f64.argtypes = [dp, dp, dp, i64, i64, i64, i64, dp]
            lib.ref_causal_conv1d_silu_f64.restype = None
            lib.ref_affine_scan_f64.argtypes = [dp, dp, i64, ctypes.c_double, dp]
            lib.ref_affine_scan_f64.restype = None
            lib.ref_softplus_f64.argtypes = [ctypes.c_double]
            lib.ref_softplus_f64.restype = ctypes.c_double
            lib.ref_silu_f64.argtypes = [ctypes.c_double]
            lib.ref_silu_f64.restype = ctypes.c_double
            lib.ref_set_threads.argtypes = [ctypes.c_int]
            lib.ref_set_threads.restype = None
            lib.ref_max_threads.argtypes = []
            lib.ref_max_threads.restype = ctypes.c_int
            _lib = lib
    return _lib


def _f64(x):
    """Contiguous float64 copy (or view) of an array-like; None stays None."""
    if x is None:
        return None
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(x):
    if x is None:
        return None
    return x.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def set_threads(n: int) -> None:
    """Set the OpenMP thread count the oracle uses (n <= 0 leaves it unchanged)."""
    _load().ref_set_threads(int(n))


def max_threads() -> int:
    return int(_load().ref_max_threads())


def scan_ref(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=False):
    """Selective-scan forward from a zero state, in float64.

    Shapes: u, delta, z (batch, dim, L); A (dim, N); B, C (batch, N, L); D, delta_bias (dim,).
    Returns (out (batch, dim, L), last_state (batch, dim, N)), both float64.
    """
    u, delta, A, B, C = (_f64(v) for v in (u, delta, A, B, C))
    D, z, delta_bias = _f64(D), _f64(z), _f64(delta_bias)
    batch, dim, L = u.shape
    N = A.shape[1]
    assert delta.shape == u.shape and A.shape == (dim, N)
    assert B.shape == (batch, N, L) and C.shape == (batch, N, L)
    assert z is None or z.shape == u.shape
    assert D is None or D.shape == (dim,)
    assert delta_bias is None or delta_bias.shape == (dim,)
    out = np.empty((batch, dim, L), dtype=np.float64)
    last = np.empty((batch, dim, N), dtype=np.float64)
    _load().ref_scan_fwd_f64(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                             _ptr(delta_bias), int(bool(delta_softplus)), batch, dim, N, L,
                             _ptr(out), _ptr(last))
    return out, last


def state_update_ref(state, u, delta, A, B, C, D=None, z=None, delta_bias=None,
                     delta_softplus=False):
    """One generation step. state (batch, dim, N); u, delta, z (batch, dim); B, C (batch, N).

    Returns (out (batch, dim), new_state (batch, dim, N)) in float64; the input is not modified.
    """
    st = np.array(state, dtype=np.float64, copy=True, order="C")
    u, delta, A, B, C = (_f64(v) for v in (u, delta, A, B, C))
    D, z, delta_bias = _f64(D), _f64(z), _f64(delta_bias)
    batch, dim, N = st.shape
    assert u.shape == (batch, dim) and delta.shape == (batch, dim)
    assert A.shape == (dim, N) and B.shape == (batch, N) and C.shape == (batch, N)
    out = np.empty((batch, dim), dtype=np.float64)
    _load().ref_state_update_f64(_ptr(st), _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C),
                                 _ptr(D), _ptr(z), _ptr(delta_bias), int(bool(delta_softplus)),
                                 batch, dim, N, _ptr(out))
    return out, st


def state_update_ref_inplace(state, u, delta, A, B, C, D=None, z=None, delta_bias=None,
                             delta_softplus=False):
    """state_update_ref that updates `state` (a C-contiguous float64 array (batch, dim, N)) in
    place instead of copying it; returns out (batch, dim) in float64."""
    assert isinstance(state, np.ndarray) and state.dtype == np.float64
    assert state.flags["C_CONTIGUOUS"] and state.ndim == 3
    u, delta, A, B, C = (_f64(v) for v in (u, delta, A, B, C))
    D, z, delta_bias = _f64(D), _f64(z), _f64(delta_bias)
    batch, dim, N = state.shape
    assert u.shape == (batch, dim) and delta.shape == (batch, dim)
    assert A.shape == (dim, N) and B.shape == (batch, N) and C.shape == (batch, N)
    out = np.empty((batch, dim), dtype=np.float64)
    _load().ref_state_update_f64(_ptr(state), _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C),
                                 _ptr(D), _ptr(z), _ptr(delta_bias), int(bool(delta_softplus)),
                                 batch, dim, N, _ptr(out))
    return out


def scan_bwd_ref(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=False,
                 dout=None, dlast=None):
    """Gradients of sum(out * dout) + sum(last_state * dlast) by the hand-written adjoint
    recurrence in float64 (``ref_scan_bwd_f64``).

    Returns a dict of float64 arrays du, ddelta (w.r.t. the raw delta), dA, dB, dC, dD,
    ddelta_bias and dz (None without a gate).  dD and ddelta_bias are the gradients for a zero skip
    or bias when D or delta_bias is None.  dlast=None means zero.
    """
    u, delta, A, B, C = (_f64(v) for v in (u, delta, A, B, C))
    D, z, delta_bias, dout, dlast = (_f64(v) for v in (D, z, delta_bias, dout, dlast))
    batch, dim, L = u.shape
    N = A.shape[1]
    assert dout is not None and dout.shape == u.shape
    assert dlast is None or dlast.shape == (batch, dim, N)
    assert B.shape == (batch, N, L) and C.shape == (batch, N, L)
    res = {k: np.empty(s, dtype=np.float64) for k, s in (
        ("du", u.shape), ("ddelta", u.shape), ("dA", (dim, N)), ("dB", B.shape),
        ("dC", C.shape), ("dD", (dim,)), ("ddelta_bias", (dim,)))}
    res["dz"] = np.empty(u.shape, dtype=np.float64) if z is not None else None
    _load().ref_scan_bwd_f64(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                             _ptr(delta_bias), int(bool(delta_softplus)), _ptr(dout),
                             _ptr(dlast), batch, dim, N, L, _ptr(res["du"]),
                             _ptr(res["ddelta"]), _ptr(res["dA"]), _ptr(res["dB"]),
                             _ptr(res["dC"]), _ptr(res["dD"]), _ptr(res["dz"]),
                             _ptr(res["ddelta_bias"]))
    return res


def conv_silu_ref(x, w, bias=None):
    """u = silu(causal depthwise conv1d(x) + bias) in float64 (``ref_causal_conv1d_silu_f64``).

    x (batch, dim, L); w (dim, W); bias (dim,) or None.  The newest token multiplies w[:, W-1];
    tokens before the start are zero.
    """
    x, w, bias = _f64(x), _f64(w), _f64(bias)
    batch, dim, L = x.shape
    assert w.ndim == 2 and w.shape[0] == dim and w.shape[1] >= 1
    assert bias is None or bias.shape == (dim,)
    u = np.empty_like(x)
    _load().ref_causal_conv1d_silu_f64(_ptr(x), _ptr(w), _ptr(bias), w.shape[1], batch, dim, L,
                                       _ptr(u))
    return u


def scan_conv_ref(x, conv_w, conv_b, delta, A, B, C, D=None, z=None, delta_bias=None,
                  delta_softplus=False):
    """The fused forward's definition: u = conv_silu_ref(x, conv_w, conv_b), then scan_ref.
    Returns (out, last_state, u)."""
    u = conv_silu_ref(x, conv_w, conv_b)
    out, last = scan_ref(u, delta, A, B, C, D, z, delta_bias, delta_softplus)
    return out, last, u


def affine_scan_ref(a, b, h0=0.0):
    """h_t = a_t*h_{t-1} + b_t from h_{-1} = h0; returns every h_t (float64)."""
    a, b = _f64(a), _f64(b)
    assert a.shape == b.shape and a.ndim == 1
    h = np.empty_like(a)
    _load().ref_affine_scan_f64(_ptr(a), _ptr(b), a.shape[0], float(h0), _ptr(h))
    return h


def softplus_ref(x: float) -> float:
    return float(_load().ref_softplus_f64(float(x)))


def silu_ref(x: float) -> float:
    return float(_load().ref_silu_f64(float(x)))
