"""fp64 reference gradients of the selective-scan forward (test infrastructure only).

The forward recurrence is written out as plain PyTorch CPU operations in float64, one token at a
time, with the same readings as the C oracle (Delta = softplus(raw + bias), Abar = exp(Delta*A),
Bbar*x = Delta*B*u, h from zero, readout after the update, skip, silu gate).  The gradients are
torch.autograd's derivatives of that definition: the backward pass that "activation
recomputation" refers to in "State Spaces, Selectively -- Mamba" (papermap), chapter 01/02, is
the exact derivative of the forward, so autograd of the plain loop is its definition.

Pinned by the oracle backward tests: its forward equals the C oracle, and its gradients equal
central finite differences of the C oracle's forward.
"""
from __future__ import annotations

import numpy as np
import torch


def _t(x):
    return None if x is None else torch.as_tensor(np.asarray(x, dtype=np.float64))


def forward_torch(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=False,
                  h0=None):
    """(out, last_state) as float64 torch tensors (differentiable)."""
    batch, dim, L = u.shape
    N = A.shape[1]
    h = torch.zeros(batch, dim, N, dtype=torch.float64) if h0 is None else h0
    ys = []
    for t in range(L):
        dt = delta[:, :, t]
        if delta_bias is not None:
            dt = dt + delta_bias[None, :]
        if delta_softplus:
            # threshold raised: log1p(exp(x)) everywhere, derivative sigmoid(x)
            dt = torch.nn.functional.softplus(dt, threshold=1000.0)
        abar = torch.exp(dt[:, :, None] * A[None, :, :])
        h = abar * h + (dt * u[:, :, t])[:, :, None] * B[:, None, :, t]
        y = (h * C[:, None, :, t]).sum(-1)
        if D is not None:
            y = y + D[None, :] * u[:, :, t]
        if z is not None:
            y = y * torch.nn.functional.silu(z[:, :, t])
        ys.append(y)
    return torch.stack(ys, dim=-1), h


def scan_bwd_ref(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=False,
                 dout=None, dlast=None):
    """Gradients of sum(out * dout) + sum(last_state * dlast) with respect to every input.

    Returns a dict of float64 numpy arrays: du, ddelta (w.r.t. the raw delta), dz, dA, dB, dC,
    dD, ddelta_bias; entries for absent optional inputs are None.
    """
    names = ["u", "delta", "A", "B", "C", "D", "z", "delta_bias"]
    vals = [u, delta, A, B, C, D, z, delta_bias]
    ts = {n: (_t(v).requires_grad_(True) if v is not None else None) for n, v in zip(names, vals)}
    out, last = forward_torch(ts["u"], ts["delta"], ts["A"], ts["B"], ts["C"], ts["D"], ts["z"],
                              ts["delta_bias"], delta_softplus)
    loss = (out * _t(dout)).sum()
    if dlast is not None:
        loss = loss + (last * _t(dlast)).sum()
    inputs = [ts[n] for n in names if ts[n] is not None]
    grads = torch.autograd.grad(loss, inputs, allow_unused=True)
    res = {}
    it = iter(grads)
    for n in names:
        if ts[n] is None:
            res["d" + n] = None
        else:
            g = next(it)
            res["d" + n] = (torch.zeros_like(ts[n]) if g is None else g).detach().numpy()
    return res
