"""fp64 reference of a whole Mamba block forward (test infrastructure only).

The block, by page title and section: "Mamba" (elemedex), "How it works" (linear projection,
short convolution, selective SSM, multiplicative gate); "State Spaces, Selectively -- Mamba"
(papermap), ch.02 (Delta, B and C computed from the token); "Mamba" (visual-learn),
"Simplifications and limits" (trained linear maps around the SSM, a brief convolution ahead of
it and gating behind it).  Per sequence, with E = d_inner, R = dt_rank, N = 16:

    [x; z] = W_in h^T,   u = silu(causal_conv1d(x) + conv_b),   [dlow; B; C] = W_x u,
    Delta_raw = W_dt dlow,   y = scan(u, Delta_raw, A, B, C, D, z, dt_bias, softplus),
    out = (W_out y)^T.

The matrix products are numpy matmuls (BLAS, float64); the convolution and the scan are this
package's C oracle.  round_bf16=True stores each intermediate (x, z, u, dlow, B, C, Delta_raw, y)
as the nearest bf16 value (``nearest_bf16``), the storage points of the GPU block; False is the
block in exact arithmetic.
Pinned by the oracle block tests against an independent torch-module implementation.
"""
from __future__ import annotations

import numpy as np

from . import conv_silu_ref, scan_ref


def nearest_bf16(x):
    """Nearest bf16 value of float64 data, ties to even, returned as float64.

    Rounds the float64 value directly (no float32 step, so no double rounding).  A finite value
    x = m * 2^e (0.5 <= |m| < 1) is rounded to a multiple of the bf16 quantum 2^(max(e-1, -126) - 7)
    with numpy's round-half-to-even; the clamp at -126 gives bf16's subnormal spacing.  Results of
    magnitude 2^128 or more (past bf16's largest finite value) become infinities of the same sign;
    infinities, signed zeros and NaNs pass through unchanged.
    """
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    fin = np.isfinite(x) & (x != 0)
    if np.any(fin):
        v = x[fin]
        _, e = np.frexp(v)
        k = np.maximum(e - 1, -126) - 7
        r = np.ldexp(np.round(np.ldexp(v, -k)), k)
        r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, v), r)
        out[fin] = r
    return out


def block_ref(hidden, w_in, conv_w, conv_b, w_x, w_dt, dt_bias, A, D, w_out, dstate=16,
              round_bf16=True):
    """Returns out (batch, L, d_model) in float64."""
    f = lambda a: None if a is None else np.asarray(a, dtype=np.float64)
    h, w_in, w_x, w_dt, w_out = f(hidden), f(w_in), f(w_x), f(w_dt), f(w_out)
    rb = nearest_bf16 if round_bf16 else (lambda a: a)
    E = w_in.shape[0] // 2
    R = w_dt.shape[1]
    N = dstate
    # (W h^T) per sequence as BLAS matrix products in float64
    xz = np.matmul(w_in[None], np.swapaxes(h, 1, 2))
    x, z = rb(xz[:, :E]), rb(xz[:, E:])
    u = rb(conv_silu_ref(x, conv_w, conv_b))
    dbc = np.matmul(w_x[None], u)
    dlow, B, C = rb(dbc[:, :R]), rb(dbc[:, R:R + N]), rb(dbc[:, R + N:R + 2 * N])
    draw = rb(np.matmul(w_dt[None], dlow))
    y, _ = scan_ref(u, draw, A, B, C, D, z, dt_bias, True)
    y = rb(y)
    return np.swapaxes(np.matmul(w_out[None], y), 1, 2)
