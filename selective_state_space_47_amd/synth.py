"""Seeded synthetic inputs for the selective scan and the state update.

This module is the only code that both the GPU path's tests and the fp64 oracle consume.  It draws
random numbers and rounds them to the storage precision; it holds none of the scan's arithmetic.

Recipe (every workload):
  * A[d, n] = -(n + 1) in fp32, D[d] = 1, delta_bias[d] = log(expm1(U[lo, hi])) computed in fp64
    and stored as fp32 (so softplus(delta_bias) is uniform on [lo, hi]).
  * u, raw delta, z ~ N(0, 1) and B, C ~ N(0, 1), drawn in fp32 with numpy's PCG64.
  * bf16 workloads round each fp32 draw once to bf16 (round to nearest, ties to even); both the
    oracle and the GPU then consume exactly those bf16 values.
  * Large tensors are drawn in independent blocks of rows so generation can run on several threads
    and any subset of channels can be regenerated alone: block j of tensor k of a workload with
    seed s comes from ``Generator(PCG64(SeedSequence([s, k, j])))``.  Rows are the leading
    (batch*dim) channel rows for (batch, dim, L) tensors, (batch*dstate) rows for B and C, and
    one generation step per block for the per-step token tensors.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

BLOCK_ROWS = 64

# tensor ids used in the seed sequences
_T_BIAS, _T_U, _T_DELTA, _T_Z, _T_B, _T_C, _T_STATE = 0, 1, 2, 3, 4, 5, 6
_T_DOUT, _T_DLAST = 8, 9  # (7 is the selective-copying stream)
_T_CONV = 10
_T_BLOCK = 11


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    dim: int
    dstate: int
    seqlen: int
    io_dtype: str          # "f32" or "bf16": storage of u, delta, z, B, C and out
    bias_lo: float
    bias_hi: float
    seed: int
    steps: int = 0         # >0: generation-step workload (state update repeated `steps` times)
    tol: float = 1e-4      # parity bound of the GPU tests for this workload
    tol_kind: str = "rel"  # "rel": max|err|/max(|ref|, rms(ref)); "rms": max|err|/rms(ref)

    @property
    def channels(self) -> int:
        return self.batch * self.dim

    @property
    def channel_steps(self) -> int:
        return self.batch * self.dim * max(self.seqlen, 1) * max(self.steps, 1)


WORKLOADS = {
    "tiny": Workload("tiny", 1, 64, 16, 256, "f32", 1e-3, 1e-1, 4700, tol=1e-4),
    "130m_layer": Workload("130m_layer", 2, 1536, 16, 2048, "f32", 1e-3, 1e-1, 4701, tol=1e-4),
    "2p8b_layer": Workload("2p8b_layer", 8, 5120, 16, 2048, "bf16", 1e-3, 1e-1, 4702, tol=1e-2),
    "1m_steps": Workload("1m_steps", 1, 1536, 16, 1 << 20, "f32", 1e-4, 1e-2, 4703, tol=1e-3,
                         tol_kind="rms"),
    "gen_step": Workload("gen_step", 256, 5120, 16, 1, "bf16", 1e-3, 1e-1, 4704, steps=1000,
                         tol=1e-2),
}


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> nearest bf16 value (ties to even), returned as fp32 holding that exact value."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    # finite inputs only: the sum stays below 2**32 for every finite fp32 bit pattern
    r = bits + np.uint32(0x7FFF) + ((bits >> np.uint32(16)) & np.uint32(1))
    r &= np.uint32(0xFFFF0000)
    return r.view(np.float32)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _rng(seed: int, tensor: int, block: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tensor, block])))


def _normal_rows(seed: int, tensor: int, nrows: int, rowlen: int, rows=None, bf16=False):
    """Standard-normal fp32 matrix (len(rows) or nrows, rowlen) drawn block-wise."""
    if rows is None:
        rows = np.arange(nrows)
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((rows.shape[0], rowlen), dtype=np.float32)
    blocks = np.unique(rows // BLOCK_ROWS)

    def work(j):
        lo = int(j) * BLOCK_ROWS
        n = min(BLOCK_ROWS, nrows - lo)
        blk = _rng(seed, tensor, int(j)).standard_normal((n, rowlen), dtype=np.float32)
        if bf16:
            blk = round_to_bf16(blk)
        sel = np.nonzero((rows >= lo) & (rows < lo + n))[0]
        out[sel] = blk[rows[sel] - lo]

    if len(blocks) == 1:
        work(blocks[0])
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, blocks))
    return out


def params(w: Workload):
    """A (dim, N), D (dim,), delta_bias (dim,) as fp32."""
    A = -np.broadcast_to(np.arange(1, w.dstate + 1, dtype=np.float32), (w.dim, w.dstate)).copy()
    D = np.ones(w.dim, dtype=np.float32)
    U = _rng(w.seed, _T_BIAS, 0).uniform(w.bias_lo, w.bias_hi, size=w.dim)  # fp64
    bias = np.log(np.expm1(U)).astype(np.float32)
    return A, D, bias


def scan_inputs(w: Workload, channels=None):
    """Inputs of a whole-sequence workload.

    channels: optional 1-D array of flat channel indices (b*dim + d) to generate only those rows of
    u, delta and z (then shaped (len(channels), L)); B and C are always complete.
    Returns a dict of fp32 arrays holding the exact stored values.
    """
    bf = w.io_dtype == "bf16"
    A, D, bias = params(w)
    L = w.seqlen
    nrows = w.batch * w.dim
    shape = (w.batch, w.dim, L) if channels is None else (len(channels), L)
    u = _normal_rows(w.seed, _T_U, nrows, L, channels, bf).reshape(shape)
    delta = _normal_rows(w.seed, _T_DELTA, nrows, L, channels, bf).reshape(shape)
    z = _normal_rows(w.seed, _T_Z, nrows, L, channels, bf).reshape(shape)
    B = _normal_rows(w.seed, _T_B, w.batch * w.dstate, L, None, bf).reshape(w.batch, w.dstate, L)
    C = _normal_rows(w.seed, _T_C, w.batch * w.dstate, L, None, bf).reshape(w.batch, w.dstate, L)
    return dict(u=u, delta=delta, z=z, B=B, C=C, A=A, D=D, delta_bias=bias)


def grad_inputs(w: Workload, channels=None):
    """Output gradients for the backward pass of a whole-sequence workload: dout (batch, dim, L)
    ~ N(0, 1) in the workload's storage precision and dlast (batch, dim, N) ~ N(0, 1) fp32.
    channels: as for scan_inputs (rows of dout and dlast only)."""
    bf = w.io_dtype == "bf16"
    nrows = w.batch * w.dim
    dshape = (w.batch, w.dim, w.seqlen) if channels is None else (len(channels), w.seqlen)
    lshape = (w.batch, w.dim, w.dstate) if channels is None else (len(channels), w.dstate)
    dout = _normal_rows(w.seed, _T_DOUT, nrows, w.seqlen, channels, bf).reshape(dshape)
    dlast = _normal_rows(w.seed, _T_DLAST, nrows, w.dstate, channels, False).reshape(lshape)
    return dict(dout=dout, dlast=dlast)


def conv_params(w: Workload, width: int = 4):
    """Depthwise causal-conv taps (dim, width) and bias (dim,), fp32, uniform in
    [-1/sqrt(width), 1/sqrt(width)] (the usual fan-in scaling of a depthwise convolution)."""
    r = _rng(w.seed, _T_CONV, width)
    bound = 1.0 / np.sqrt(width)
    taps = r.uniform(-bound, bound, size=(w.dim, width)).astype(np.float32)
    bias = r.uniform(-bound, bound, size=w.dim).astype(np.float32)
    return taps, bias


def step_inputs(w: Workload, steps=None, channels=None):
    """Inputs of the generation-step workload.

    Returns dict with state0 (batch, dim, N) fp32 ~ N(0,1); per-step tokens u, delta, z
    (steps, batch, dim) and B, C (steps, batch, N), rounded to bf16 values when io_dtype is bf16;
    and A, D, delta_bias.  channels: optional flat channel indices to generate only those columns
    of the token tensors and rows of state0 (shapes (steps, len(channels)) and (len, N)).
    """
    bf = w.io_dtype == "bf16"
    A, D, bias = params(w)
    S = w.steps if steps is None else steps
    nch = w.batch * w.dim
    st = _normal_rows(w.seed, _T_STATE, nch, w.dstate, channels, False)
    if channels is None:
        st = st.reshape(w.batch, w.dim, w.dstate)

    def per_step(tensor, width, cols=None):
        # one block per step: row s of the (S, width) matrix comes from SeedSequence([seed, k, s])
        out = np.empty((S, width if cols is None else len(cols)), dtype=np.float32)

        def work(s):
            v = _rng(w.seed, tensor, s).standard_normal(width, dtype=np.float32)
            if bf:
                v = round_to_bf16(v)
            out[s] = v if cols is None else v[cols]

        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(S)))
        return out

    u = per_step(_T_U, nch, channels)
    delta = per_step(_T_DELTA, nch, channels)
    z = per_step(_T_Z, nch, channels)
    B = per_step(_T_B, w.batch * w.dstate).reshape(S, w.batch, w.dstate)
    C = per_step(_T_C, w.batch * w.dstate).reshape(S, w.batch, w.dstate)
    if channels is None:
        u, delta, z = (x.reshape(S, w.batch, w.dim) for x in (u, delta, z))
    return dict(state0=st, u=u, delta=delta, z=z, B=B, C=C, A=A, D=D, delta_bias=bias)


def random_case(seed, batch, dim, L, dstate=16, bias_lo=1e-3, bias_hi=1e-1, bf16=False):
    """Small seeded case of arbitrary shape (edge-shape and flag-toggle tests)."""
    w = Workload("case", batch, dim, dstate, L, "bf16" if bf16 else "f32", bias_lo, bias_hi, seed)
    return scan_inputs(w)


def selective_copy_values(gap: int, n_seq: int = 400, seed: int = 4705):
    """Values of the selective-copying experiment: n_seq sequences, each a target scalar followed
    by `gap` distractors, all N(0, 1) fp32; returns an (n_seq, 1 + gap) array (column 0 is the
    target).  One generator per gap: SeedSequence([seed, 7, gap])."""
    return _rng(seed, 7, gap).standard_normal((n_seq, 1 + gap), dtype=np.float32)


@dataclass(frozen=True)
class BlockWorkload:
    """A Mamba block forward: hidden (batch, seqlen, d_model) -> out (batch, seqlen, d_model)."""
    name: str
    batch: int
    seqlen: int
    d_model: int
    d_inner: int
    dt_rank: int
    conv_width: int
    seed: int
    dstate: int = 16


BLOCK_WORKLOADS = {
    # Mamba-2.8B layer sizes: d_model 2560, expand 2 (d_inner 5120), dt_rank ceil(2560/16) = 160
    "block_2p8b": BlockWorkload("block_2p8b", 8, 2048, 2560, 5120, 160, 4, 4706),
}


def block_inputs(w: BlockWorkload, seqlen=None):
    """Seeded hidden states and random weights of a block, all fp32 arrays holding the stored
    values: hidden and the four projection matrices rounded to bf16; conv taps/bias, dt_bias, A,
    D in fp32.  Projection weights ~ N(0, 1/fan_in); conv taps and bias as conv_params; dt_bias,
    A and D as params() with the workloads' bias range [1e-3, 1e-1].  seqlen: optional shorter
    prefix of the same hidden states (the draws of the first tokens do not depend on it)."""
    E, R, N, Dm = w.d_inner, w.dt_rank, w.dstate, w.d_model
    L = w.seqlen if seqlen is None else seqlen
    r = _rng(w.seed, _T_BLOCK, 0)
    w_in = round_to_bf16((r.standard_normal((2 * E, Dm)) / np.sqrt(Dm)).astype(np.float32))
    w_x = round_to_bf16((r.standard_normal((R + 2 * N, E)) / np.sqrt(E)).astype(np.float32))
    w_dt = round_to_bf16((r.standard_normal((E, R)) / np.sqrt(R)).astype(np.float32))
    w_out = round_to_bf16((r.standard_normal((Dm, E)) / np.sqrt(E)).astype(np.float32))
    sw = Workload(w.name, w.batch, E, N, L, "bf16", 1e-3, 1e-1, w.seed)
    A, D, bias = params(sw)
    conv_w, conv_b = conv_params(sw, w.conv_width)
    # hidden: one block of rows per (sequence, token) row of d_model values
    hid = _normal_rows(w.seed, _T_BLOCK + 1, w.batch * w.seqlen, Dm, None, True)
    hid = hid.reshape(w.batch, w.seqlen, Dm)[:, :L]
    return dict(hidden=np.ascontiguousarray(hid), w_in=w_in, conv_w=conv_w, conv_b=conv_b,
                w_x=w_x, w_dt=w_dt, dt_bias=bias, A=A, D=D, w_out=w_out)
