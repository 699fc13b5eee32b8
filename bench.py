"""Benchmark of the selective-scan forward on one MI355X.

One step = one selective-scan forward (Delta/discretization/recurrence/readout/skip/gate) over
the whole 2.8B-layer-shaped workload: batch 8, 5120 channels, 16 states, 2048 tokens, bf16
u/Delta/z/B/C/out, fp32 A/D/bias/state, fp32 arithmetic -- 83,886,080 channel-steps.  Inputs are
seeded synthetic data resident in HBM before timing starts.  The single-token state update of
the generation workload (256 x 5120 x 16 fp32 states, bf16 tokens) is timed in the same run and
reported in its own field.

Prints one JSON line.  Roofline: `roofline` is the HBM roofline the metric names (algorithmic
bytes per launch over the scan kernel's mean HIP-event time, against 8 TB/s); the scan is bound
by VALU issue on gfx950, and the ALU fraction (ALU_PEAK_LANE_OPS, ALU_OPS_PER_CHANNEL_STEP below)
sits beside it.  Before timing, launches run for --settle-seconds so the clocks are settled
whatever --warmup says.  `parity` compares the timed run's outputs with the fp64 oracle outputs
that the CPU-baseline leg computes on the same inputs; the run fails if they differ beyond the
workload's bound.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "scan_fwd_2p8b_layer_counters.json")
HBM_PEAK_GBS = 8000.0
# VALU peak of the chip in lane-ops/s: 256 CUs x 4 SIMD x 16 lanes x 2.4 GHz (non-packed fp32;
# one lane-op per lane-cycle; a transcendental counts 2 lane-ops, its issue cost on gfx950).
ALU_PEAK_LANE_OPS = 256 * 4 * 16 * 2.4e9
# Algorithmic lane-ops per channel-step at N = 16:
#   per state: Delta*A' (1), exp2 (2), Delta*u*B (1), h fma (1), C*h fma (1)  -> 6 x 16 = 96
#   per channel-step: bias add 1, softplus (mul 1, exp2 2, log 2, mul 1, max/add 2) 9,
#   Delta*u 1, skip fma 1, silu (mul 1, exp2 2, add 1, rcp 2, mul 1) 7, gate mul 1  -> 19
ALU_OPS_PER_CHANNEL_STEP = 96 + 19
# Backward (gradients of the scan with one recomputation of the forward), per channel-step:
#   per state, recompute 6 (as above); adjoint: lam = dy*C + carry (1), carry = Abar*lam (1),
#   Abar*h_prev (1), *lam (1), dA fma (1), sum lam*Abar*h*A fma (1), sum lam*B fma (1),
#   dB term lam*Delta*u (1) and its sum over channels (1), dC term dy*h (1) and its sum (1)
#   -> 17 x 16 = 272
#   per channel-step: softplus 9, bias add 1, Delta*u 1, skip fma 1, gate: sigmoid 6, dy 2,
#   dz 5, softplus' (sigmoid 6, product 1) 7, dDelta fma 1, du 2, dD 1, dbias 1  -> 37
BWD_OPS_PER_CHANNEL_STEP = 272 + 37
# Forward with the fused causal conv (width 4) + SiLU: the forward's 115 plus 4 fma (taps + bias
# as the first fma's addend) and silu 7 -> 126
CONV_OPS_PER_CHANNEL_STEP = ALU_OPS_PER_CHANNEL_STEP + 4 + 7


# Sources of the forward scan and state-update kernels (the counters in profiles/ are tied to them)
FWD_KERNEL_SOURCES = ("mamba_common.h", "mamba_scan.hip")


def _code_only(text: str) -> str:
    """The source without comments and with whitespace collapsed: an edit of a comment leaves
    the kernel, and so the counters recorded for it, unchanged."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return " ".join(text.split())


def kernel_source_hash(files=FWD_KERNEL_SOURCES) -> str:
    h = hashlib.sha256()
    for name in files:
        with open(os.path.join(ROOT, "selective_state_space_47_amd", "csrc", name)) as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def scan_alg_bytes(batch, dim, L, N, s_in, s_out):
    """Bytes the method must move: u, Delta, z read and out written per channel-step; B and C
    per (sequence, token); last_state written; A, D, bias read."""
    return (batch * L * dim * (3 * s_in + s_out) + batch * L * 2 * N * s_in + batch * dim * N * 4
            + dim * N * 4 + 2 * dim * 4)


def step_alg_bytes(batch, dim, N, s_in, s_out):
    """State read + write, u/Delta/z read and out written per channel; B, C per sequence."""
    return batch * dim * (2 * N * 4 + 3 * s_in + s_out) + batch * 2 * N * s_in + dim * (N + 2) * 4


def parse_counters(fetch_csv, write_csv, out_json, alg_bytes, kernel_filter, label):
    """Turn two rocprofv3 --pmc CSVs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch) into HBM bytes per
    dispatch of every kernel whose name contains `kernel_filter`, each scaled by the same counter
    on a plain device copy of 1 GiB in the same run (--calib-copy).  alg_bytes: algorithmic bytes
    of one call of the workload (all of its kernels); the record compares their sum with it."""
    import csv

    def read(path, counter):
        per = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if r.get("Counter_Name") != counter:
                    continue
                name = r.get("Kernel_Name", "")
                per.setdefault(name, []).append(float(r["Counter_Value"]))
        return per

    kernels = {}
    scale = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        per = read(path, counter)
        # the calibration copy: torch.mul(a, 1.0, out=b) over 1 GiB; its largest dispatches
        # (smaller ones of the same kernel come from torch's own setup)
        copy_k = [k for k in per if "MulFunctor<float>" in k and "AUnaryFunctor" in k]
        copy = sorted(per[copy_k[0]])[-3:] if copy_k else []
        sel = {k: v for k, v in per.items() if kernel_filter in k}
        if not sel or not copy:
            raise SystemExit(f"{counter}: kernel '{kernel_filter}' or the copy not found in {path}")
        copy_kib = sorted(copy)[len(copy) // 2]
        factor = (1 << 30) / (copy_kib * 1024.0)
        scale[counter] = dict(copy_kib_per_dispatch=copy_kib, copy_bytes=1 << 30, scale=factor)
        for k, v in sel.items():
            kib = sorted(v)[len(v) // 2]
            kernels.setdefault(k, {})[counter] = dict(kib_per_dispatch=kib, dispatches=len(v),
                                                      bytes_scaled=kib * 1024.0 * factor)
    for k, v in kernels.items():
        v["traffic_bytes"] = sum(v[c]["bytes_scaled"] for c in ("FETCH_SIZE", "WRITE_SIZE")
                                 if c in v)
    total = sum(v["traffic_bytes"] for v in kernels.values())
    doc = dict(workload=label, kernel_filter=kernel_filter, source_hash=kernel_source_hash(),
               calibration=scale, kernels=kernels, traffic_bytes_per_call=total,
               algorithmic_bytes_per_call=alg_bytes, traffic_over_algorithmic=total / alg_bytes,
               note="per-call traffic sums one dispatch of each listed kernel")
    if out_json:
        with open(out_json, "w") as f:
            json.dump(doc, f, indent=1)
    print(json.dumps(doc, indent=1))


def cpu_baseline(x, w, target_cpu_s):
    """The fp64 oracle, as it stands, on a bounded sample of the same workload: whole sequences
    (all channels of one sequence per call) in order, repeating the workload if needed, until
    about `target_cpu_s` seconds of CPU work (wall time x threads) have been spent."""
    import oracle
    threads = oracle.max_threads()
    cores = min(threads, w.dim)
    L = w.seqlen
    done = 0
    spent = 0.0
    passes = 0
    refs = {}
    while spent * cores < target_cpu_s:
        for b in range(w.batch):
            t0 = time.perf_counter()
            ref = oracle.scan_ref(x["u"][b:b + 1], x["delta"][b:b + 1], x["A"], x["B"][b:b + 1],
                                  x["C"][b:b + 1], x["D"], x["z"][b:b + 1], x["delta_bias"],
                                  True)
            spent += time.perf_counter() - t0
            if b not in refs:
                refs[b] = ref
            done += w.dim * L
            if spent * cores >= target_cpu_s:
                break
        passes += 1
    seqs = done // (w.dim * L)
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return refs, dict(value=done / spent, unit="channel-steps/s", cores=cores, kind="oracle",
                cpu_model=model, usable_cores=len(os.sched_getaffinity(0)),
                sample=f"{seqs} sequences ({passes} pass(es) over the {w.batch} sequences) x "
                       f"{w.dim} channels x {L} tokens of the {w.name} workload ({done} "
                       f"channel-steps, {spent:.1f} s wall x {cores} threads = "
                       f"{spent * cores:.0f} s of CPU work, fp64, OpenMP over channels; input "
                       f"conversion to fp64 not timed)")


def timed_output_parity(out_h, last_h, refs, bound):
    """Error of the timed run's out and last_state against the oracle outputs of the sequences
    the CPU baseline computed: R15's max relative error (floor rms of the reference) and
    max|err| / rms(ref), over every compared element."""
    import numpy as np
    seqs = sorted(refs)
    if not seqs:
        return None
    ro = np.concatenate([refs[b][0] for b in seqs])
    rl = np.concatenate([refs[b][1] for b in seqs])
    go = np.asarray(out_h[seqs], dtype=np.float64)
    gl = np.asarray(last_h[seqs], dtype=np.float64)
    res = {}
    for key, g, r in (("out", go, ro), ("last_state", gl, rl)):
        rms = float(np.sqrt(np.mean(r * r)))
        err = np.abs(g - r)
        res[f"max_rel_err_{key}"] = float(np.max(err / np.maximum(np.abs(r), rms)))
        res[f"err_rms_ratio_{key}"] = float(np.max(err)) / rms
    res["bound"] = bound
    res["ok"] = bool(res["max_rel_err_out"] <= bound and res["max_rel_err_last_state"] <= bound)
    res["compared"] = f"sequences {seqs[0]}..{seqs[-1]} ({len(seqs)} of {out_h.shape[0]}), all " \
                      f"channels and tokens, against the fp64 oracle on the same inputs"
    return res


def calib_copy(torch, dev):
    """Plain streaming copy of a known size for counter calibration: reads 1 GiB, writes 1 GiB
    (an elementwise multiply by one)."""
    a = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(3):
        torch.mul(a, 1.0, out=b)
    torch.cuda.synchronize()
    del a, b


def settle(step, torch, seconds):
    """Untimed launches until `seconds` of wall time have passed, so the clocks reach their
    sustained state whatever --warmup says; returns (seconds spent, launches)."""
    t0 = time.perf_counter()
    n = 0
    while True:
        for _ in range(10):
            step()
        n += 10
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        if el >= seconds:
            return el, n


def bench_state_update(steps, torch, binding, synth, dev):
    w = synth.WORKLOADS["gen_step"]
    x = synth.step_inputs(w, steps=steps)
    st = torch.from_numpy(x["state0"]).to(dev)
    A, D, bias = (torch.from_numpy(x[k]).to(dev) for k in ("A", "D", "delta_bias"))
    tok = {k: torch.from_numpy(x[k]).to(dev).to(torch.bfloat16)
           for k in ("u", "delta", "z", "B", "C")}
    del x
    out = torch.empty((w.batch, w.dim), dtype=torch.bfloat16, device=dev)
    for s in range(min(10, steps)):
        binding.mamba_state_update(st, tok["u"][s], tok["delta"][s], A, tok["B"][s], tok["C"][s],
                                   D, tok["z"][s], bias, True, out=out)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for s in range(steps):
        binding.mamba_state_update(st, tok["u"][s], tok["delta"][s], A, tok["B"][s], tok["C"][s],
                                   D, tok["z"][s], bias, True, out=out)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    per = ms / steps
    nbytes = step_alg_bytes(w.batch, w.dim, w.dstate, 2, 2)
    return dict(workload="gen_step", batch=w.batch, dim=w.dim, dstate=w.dstate, steps=steps,
                us_per_step=per * 1e3, channel_steps_per_s=w.batch * w.dim / (per * 1e-3),
                effective_GBps=nbytes / (per * 1e-3) / 1e9,
                effective_frac_of_hbm_peak=nbytes / (per * 1e-3) / 1e9 / HBM_PEAK_GBS,
                note="state (80 MiB) is updated in place every step and fits the 256 MB "
                     "Infinity Cache: effective bandwidth, wall time over back-to-back launches")


def device_inputs(w, dev, torch, L=None, seed=0):
    """Seeded on-device inputs of a workload's shape and distributions (timing only: the parity
    tests use the host generator in selective_state_space_47_amd.synth)."""
    from selective_state_space_47_amd import synth
    L = w.seqlen if L is None else L
    io = torch.bfloat16 if w.io_dtype == "bf16" else torch.float32
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed * 1000 + seed)
    shp = (w.batch, w.dim, L)
    t = {k: torch.randn(shp, generator=g, device=dev, dtype=torch.float32).to(io)
         for k in ("u", "delta", "z")}
    for k in ("B", "C"):
        t[k] = torch.randn((w.batch, w.dstate, L), generator=g, device=dev,
                           dtype=torch.float32).to(io)
    A, D, bias = synth.params(w)
    t["A"], t["D"], t["delta_bias"] = (torch.from_numpy(v).to(dev) for v in (A, D, bias))
    return t


def time_forward(t, torch, binding, reps, warm, flush=False, graph=0):
    """HIP-event time of whole mamba_scan_fwd calls (all of its launches) on the current stream;
    returns (median ms, MALL-flushed median ms or None).  flush: also time `reps` calls that each
    follow a 512 MB scratch write (outside the events), so no input is left in the 256 MB
    Infinity Cache."""
    u = t["u"]
    out = torch.empty_like(u)
    last = torch.empty((u.shape[0], u.shape[1], 16), dtype=torch.float32, device=u.device)

    def call():
        binding.mamba_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"],
                               t["delta_bias"], True, return_last_state=True, out=out,
                               last_state=last)
    for _ in range(warm):
        call()
    settle(call, torch, 0.2)
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record(stream)
        call()
        b.record(stream)
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    fl = None
    if graph:
        # per-call time inside a replayed HIP graph of `graph` calls: no host launch overhead
        # between calls (the entry points allocate nothing and issue no memsets, so they capture)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(3):
                call()
        torch.cuda.current_stream().wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(graph):
                call()
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        gms = []
        for _ in range(5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            g.replay()
            b.record(stream)
            torch.cuda.synchronize()
            gms.append(a.elapsed_time(b) / graph)
        del g
        graph_ms = sorted(gms)[len(gms) // 2]
    if flush:
        scratch = torch.empty(1 << 27, dtype=torch.float32, device=u.device)
        fms = []
        for _ in range(reps):
            scratch.fill_(1.0)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            call()
            b.record(stream)
            torch.cuda.synchronize()
            fms.append(a.elapsed_time(b))
        del scratch
        fms.sort()
        fl = fms[len(fms) // 2]
    if graph:
        return ms[len(ms) // 2], fl, graph_ms
    return ms[len(ms) // 2], fl


def bwd_alg_bytes(batch, dim, L, N, s_io):
    """Bytes the backward must move: u, Delta, z, dout read and du, dDelta, dz written per
    channel-step; B, C read and dB, dC written per (sequence, token); dlast read; A, D, bias read
    and dA, dD, dbias written."""
    return (batch * L * dim * 7 * s_io + batch * L * 4 * N * s_io + batch * dim * N * 4
            + 2 * (dim * N * 4 + 2 * dim * 4))


def bench_backward(w, torch, binding, dev, reps, warm):
    """HIP-event time of whole mamba_scan_bwd calls (every pass: checkpoints, adjoint chunk
    summaries when chunked, gradients, reductions) on seeded device inputs."""
    t = device_inputs(w, dev, torch, seed=7)
    io = t["u"].dtype
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed * 1000 + 8)
    dout = torch.randn(t["u"].shape, generator=g, device=dev, dtype=torch.float32).to(io)
    dlast = torch.randn((w.batch, w.dim, w.dstate), generator=g, device=dev)
    ws = torch.empty(binding.mamba_scan_bwd_workspace_bytes(w.batch, w.dim, w.seqlen, io),
                     dtype=torch.uint8, device=dev)
    grads = {}

    def call():
        return binding.mamba_scan_bwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"],
                                      t["delta_bias"], True, dout, dlast, workspace=ws,
                                      grads=grads)
    grads.update(call())
    for _ in range(warm):
        call()
    settle(call, torch, 0.3)
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record(stream)
        call()
        b.record(stream)
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    med = ms[len(ms) // 2]
    chsteps = w.batch * w.dim * w.seqlen
    s = 2 if w.io_dtype == "bf16" else 4
    nbytes = bwd_alg_bytes(w.batch, w.dim, w.seqlen, w.dstate, s)
    ok = all(bool(torch.isfinite(v.float()).all().item()) for v in grads.values()
             if v is not None)
    res = dict(workload=w.name, us=med * 1e3, us_p10=ms[len(ms) // 10] * 1e3,
               us_p90=ms[(len(ms) * 9) // 10] * 1e3, channel_steps_per_s=chsteps / (med * 1e-3),
               alu_achieved=chsteps * BWD_OPS_PER_CHANNEL_STEP / (med * 1e-3) / 1e12,
               alu_frac=chsteps * BWD_OPS_PER_CHANNEL_STEP / (med * 1e-3) / ALU_PEAK_LANE_OPS,
               ops_per_channel_step=BWD_OPS_PER_CHANNEL_STEP,
               alg_GBps=nbytes / (med * 1e-3) / 1e9, algorithmic_bytes=nbytes,
               workspace_bytes=ws.numel(), outputs_finite=ok, reps=reps, warmup=warm,
               note="whole backward call, all passes; ALU roofline counts one recomputation")
    del t, dout, dlast, ws, grads
    torch.cuda.empty_cache()
    return res


def bench_conv(w, torch, binding, synth, dev, reps, warm, plain_us):
    """HIP-event time of whole mamba_scan_fwd_conv calls (width 4, u not stored) on seeded device
    inputs: x takes the place of u, so the HBM bytes equal the plain forward's."""
    t = device_inputs(w, dev, torch, seed=9)
    cw, cb = synth.conv_params(w, 4)
    cw, cb = torch.from_numpy(cw).to(dev), torch.from_numpy(cb).to(dev)
    out = torch.empty_like(t["u"])
    last = torch.empty((w.batch, w.dim, w.dstate), dtype=torch.float32, device=dev)

    def call():
        binding.mamba_scan_fwd_conv(t["u"], cw, t["delta"], t["A"], t["B"], t["C"], t["D"],
                                    t["z"], t["delta_bias"], True, conv_bias=cb,
                                    return_last_state=True, out=out, last_state=last)
    for _ in range(warm):
        call()
    settle(call, torch, 0.3)
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record(stream)
        call()
        b.record(stream)
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    med = ms[len(ms) // 2]
    chsteps = w.batch * w.dim * w.seqlen
    ok = bool(torch.isfinite(out.float()).all().item())
    del t, out, last
    torch.cuda.empty_cache()
    return dict(workload=w.name, conv_width=4, us=med * 1e3, us_p10=ms[len(ms) // 10] * 1e3,
                us_p90=ms[(len(ms) * 9) // 10] * 1e3, channel_steps_per_s=chsteps / (med * 1e-3),
                alu_frac=chsteps * CONV_OPS_PER_CHANNEL_STEP / (med * 1e-3) / ALU_PEAK_LANE_OPS,
                ops_per_channel_step=CONV_OPS_PER_CHANNEL_STEP,
                overhead_vs_plain_forward=med * 1e3 / plain_us - 1.0, outputs_finite=ok,
                reps=reps, warmup=warm)


BF16_MFMA_PEAK = 2.5e15  # dense bf16 MFMA flop/s of the chip


def bench_block(torch, binding, synth, dev, reps, warm):
    """HIP-event time of whole mamba_block_fwd calls at the Mamba-2.8B layer sizes (random
    weights, seeded hidden states); flops are the four projections' 2*M*N*K."""
    w = synth.BLOCK_WORKLOADS["block_2p8b"]
    p = synth.block_inputs(w)
    bf = ("hidden", "w_in", "w_x", "w_dt", "w_out")
    t = {k: torch.from_numpy(v).to(dev) for k, v in p.items()}
    t = {k: (v.to(torch.bfloat16) if k in bf else v) for k, v in t.items()}
    out = torch.empty_like(t["hidden"])
    dm = binding.block_dims(t["hidden"], t["w_in"], t["w_x"], t["w_dt"], t["conv_w"])
    ws = torch.empty(binding.mamba_block_workspace_bytes(dm), dtype=torch.uint8, device=dev)

    def call():
        binding.mamba_block_fwd(t["hidden"], t["w_in"], t["conv_w"], t["conv_b"], t["w_x"],
                                t["w_dt"], t["dt_bias"], t["A"], t["D"], t["w_out"], out=out,
                                workspace=ws)
    for _ in range(warm):
        call()
    settle(call, torch, 0.3)
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record(stream)
        call()
        b.record(stream)
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    med = ms[len(ms) // 2]
    E, R, Dm, L, B = w.d_inner, w.dt_rank, w.d_model, w.seqlen, w.batch
    flops = 2.0 * B * L * (2 * E * Dm + (R + 2 * w.dstate) * E + E * R + Dm * E)
    ok = bool(torch.isfinite(out.float()).all().item())
    del t, out, ws
    torch.cuda.empty_cache()
    return dict(workload=w.name, batch=B, seqlen=L, d_model=Dm, d_inner=E, dt_rank=R,
                conv_width=w.conv_width, us=med * 1e3, us_p10=ms[len(ms) // 10] * 1e3,
                us_p90=ms[(len(ms) * 9) // 10] * 1e3, tokens_per_s=B * L / (med * 1e-3),
                projection_flops=flops, projection_tflops_over_block=flops / (med * 1e-3) / 1e12,
                mfma_frac_over_block=flops / (med * 1e-3) / BF16_MFMA_PEAK, outputs_finite=ok,
                reps=reps, warmup=warm,
                note="whole block (4 GEMMs, conv, scan); per-kernel split in profiles/")


def other_workloads(torch, binding, synth, dev):
    """Every other whole-sequence workload, and the sequence-length sweep (batch 1, 1536
    channels, fp32) for the linear-in-L claim."""
    res = {}
    for name in ("tiny", "130m_layer", "1m_steps"):
        w = synth.WORKLOADS[name]
        t = device_inputs(w, dev, torch)
        reps, warm = (5, 2) if name == "1m_steps" else (30, 20)
        # the 130M-layer inputs (101 MB) fit the Infinity Cache: also timed after a flush; the
        # short workloads also inside a replayed graph of 20 calls (kernel time without the
        # host's per-call overhead, which the event pair around one call includes)
        gr = 0 if name == "1m_steps" else 20
        ms, fl, *gms = time_forward(t, torch, binding, reps, warm, flush=name == "130m_layer",
                                    graph=gr)
        s = 2 if w.io_dtype == "bf16" else 4
        nbytes = scan_alg_bytes(w.batch, w.dim, w.seqlen, w.dstate, s, s)
        ws = binding.mamba_scan_workspace_bytes(w.batch, w.dim, w.seqlen, t["u"].dtype)
        res[name] = dict(batch=w.batch, dim=w.dim, seqlen=w.seqlen, io_dtype=w.io_dtype,
                         us=ms * 1e3, channel_steps_per_s=w.channel_steps / (ms * 1e-3),
                         alg_GBps=nbytes / (ms * 1e-3) / 1e9,
                         alu_frac=w.channel_steps * ALU_OPS_PER_CHANNEL_STEP / (ms * 1e-3)
                         / ALU_PEAK_LANE_OPS,
                         workspace_bytes=ws)
        if gms:
            res[name]["us_in_graph"] = gms[0] * 1e3
        if fl is not None:
            res[name]["us_mall_flushed"] = fl * 1e3
            res[name]["alg_GBps_mall_flushed"] = nbytes / (fl * 1e-3) / 1e9
        del t
        torch.cuda.empty_cache()
    sweep = []
    w = synth.WORKLOADS["1m_steps"]
    for lg in (11, 13, 15, 17, 19, 20):
        L = 1 << lg
        t = device_inputs(w, dev, torch, L=L, seed=lg)
        ms, _ = time_forward(t, torch, binding, 5 if lg >= 19 else 15, 3)
        sweep.append(dict(L=L, us=ms * 1e3, channel_steps_per_s=w.dim * L / (ms * 1e-3)))
        del t
        torch.cuda.empty_cache()
    return res, sweep


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5, help="untimed steps first")
    ap.add_argument("--settle-seconds", type=float, default=0.5,
                    help="then untimed launches for this long, whatever --warmup says (the "
                         "clocks need ~0.1-0.3 s of load to settle)")
    ap.add_argument("--workload", default="2p8b_layer")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--cpu-seconds", type=float, default=16.0,
                    help="CPU work (wall seconds x threads) for the oracle baseline")
    ap.add_argument("--no-step", action="store_true", help="skip the state-update timing")
    ap.add_argument("--no-others", action="store_true",
                    help="skip the other workloads and the sequence-length sweep")
    ap.add_argument("--step-steps", type=int, default=1000)
    ap.add_argument("--no-bwd", action="store_true", help="skip the backward timing")
    ap.add_argument("--no-conv", action="store_true", help="skip the fused-conv forward timing")
    ap.add_argument("--no-block", action="store_true", help="skip the Mamba block timing")
    ap.add_argument("--block-only", action="store_true",
                    help="time only the Mamba block forward (for profiling runs)")
    ap.add_argument("--bwd-steps", type=int, default=10)
    ap.add_argument("--bwd-warmup", type=int, default=60)
    ap.add_argument("--bwd-only", action="store_true",
                    help="time only the backward (for profiling runs)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--parse-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn rocprofv3 FETCH_SIZE / WRITE_SIZE CSVs into per-kernel bytes")
    ap.add_argument("--counter-kernel", default="scan_kernel",
                    help="--parse-counters: kernel-name substring to report")
    ap.add_argument("--counter-json", default=None,
                    help="--parse-counters: output file (default: the headline's profile record "
                             "for the 2p8b_layer scan kernel)")
    ap.add_argument("--counter-alg", choices=("scan", "step", "bwd"), default="scan",
                    help="--parse-counters: algorithmic bytes of which call")
    ap.add_argument("--step-only", action="store_true",
                    help="time only the state update of the generation workload")
    args = ap.parse_args()

    from selective_state_space_47_amd import synth
    w = synth.WORKLOADS[args.workload]
    bf = w.io_dtype == "bf16"
    s_io = 2 if bf else 4
    alg_bytes = scan_alg_bytes(w.batch, w.dim, w.seqlen, w.dstate, s_io, s_io)

    if args.parse_counters:
        if args.counter_alg == "step":
            ws = synth.WORKLOADS["gen_step"]
            nb, label = step_alg_bytes(ws.batch, ws.dim, ws.dstate, 2, 2), "gen_step"
        elif args.counter_alg == "bwd":
            nb, label = bwd_alg_bytes(w.batch, w.dim, w.seqlen, w.dstate, s_io), w.name + " bwd"
        else:
            nb, label = alg_bytes, w.name
        out = args.counter_json
        if out is None and w.name == "2p8b_layer" and args.counter_alg == "scan":
            out = PROFILE_COUNTERS
        parse_counters(args.parse_counters[0], args.parse_counters[1], out, nb,
                       args.counter_kernel, label)
        return 0
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the selective scan runs on a single MI355X here "
              "(channels are independent, so the path would shard over batch or channels). "
              "Run with --gpus 1.", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    from selective_state_space_47_amd import _build, binding
    if not os.path.exists(_build.LIB_PATH):
        _build.build()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.block_only:
        print(json.dumps(bench_block(torch, binding, synth, dev, 10, 5)), flush=True)
        return 0
    if args.step_only:
        print(json.dumps(bench_state_update(args.step_steps, torch, binding, synth, dev)),
              flush=True)
        if args.calib_copy:
            calib_copy(torch, dev)
        return 0
    if args.bwd_only:
        print(json.dumps(bench_backward(w, torch, binding, dev, args.bwd_steps,
                                        args.bwd_warmup)), flush=True)
        if args.calib_copy:
            calib_copy(torch, dev)
        return 0

    io = torch.bfloat16 if bf else torch.float32
    if args.no_cpu:
        # no oracle leg: seeded device-side inputs of the same shape and distributions
        x = None
        t = device_inputs(w, dev, torch)
    else:
        x = synth.scan_inputs(w)
        t = {}
        for k, v in x.items():
            tt = torch.from_numpy(v).to(dev)
            t[k] = tt.to(io) if k in ("u", "delta", "z", "B", "C") else tt
    out = torch.empty((w.batch, w.dim, w.seqlen), dtype=io, device=dev)
    last = torch.empty((w.batch, w.dim, w.dstate), dtype=torch.float32, device=dev)
    ws_bytes = binding.mamba_scan_workspace_bytes(w.batch, w.dim, w.seqlen, io)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)

    def step():
        binding.mamba_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"],
                               t["delta_bias"], True, return_last_state=True, out=out,
                               last_state=last, workspace=ws if ws_bytes else None)

    for _ in range(args.warmup):
        step()
    settle_s, settle_n = settle(step, torch, args.settle_seconds)
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        step()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall = t1 - t0
    kern_ms = [a.elapsed_time(b) for a, b in ev]
    kern_ms.sort()
    kern_avg = sum(kern_ms) / len(kern_ms)
    chsteps = w.batch * w.dim * w.seqlen
    value = args.steps * chsteps / wall
    ok = bool(torch.isfinite(out.float()).all().item())
    # the timed run's outputs, for the comparison with the oracle below
    out_h = out.float().cpu().numpy()
    last_h = last.cpu().numpy()

    if args.calib_copy:
        calib_copy(torch, dev)

    # the same kernel with the last-level cache (MALL, 256 MB) flushed before each launch by a
    # 512 MB scratch write outside the events: the cold-cache kernel time
    scratch = torch.empty(1 << 27, dtype=torch.float32, device=dev)
    flushed = []
    for _ in range(10):
        scratch.fill_(1.0)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        step()
        b.record(stream)
        torch.cuda.synchronize()
        flushed.append(a.elapsed_time(b))
    flushed.sort()
    # streaming-copy bandwidth of this GPU in the same run (reads 1 GiB, writes 1 GiB)
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    copies = []
    for _ in range(5):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        dst.copy_(src)
        b.record(stream)
        torch.cuda.synchronize()
        copies.append(a.elapsed_time(b))
    copy_GBps = 2 * src.numel() * 4 / (sorted(copies)[len(copies) // 2] * 1e-3) / 1e9
    del scratch, src, dst

    alu_achieved = chsteps * ALU_OPS_PER_CHANNEL_STEP / (kern_avg * 1e-3)
    hbm_achieved = alg_bytes / (kern_avg * 1e-3) / 1e9
    traffic = None
    if os.path.exists(PROFILE_COUNTERS):
        with open(PROFILE_COUNTERS) as f:
            prof = json.load(f)
        if prof.get("source_hash") == kernel_source_hash() and args.workload == "2p8b_layer":
            traffic = prof["traffic_bytes_per_call"]

    rec = {
        "metric": "selective-scan B·D·L channel-steps/s + achieved HBM GB/s "
                  "(% of peak), 1 MI355X",
        "value": value,
        "unit": "channel-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",  # arithmetic type; storage of u/Delta/z/B/C/out is bf16 (config)
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "dim": w.dim, "dstate": w.dstate,
                   "seqlen": w.seqlen, "io_dtype": w.io_dtype, "state_dtype": "f32",
                   "softplus": True, "delta_bias": True, "D": True, "z_gate": True,
                   "channel_steps": chsteps, "chunks": 1 if ws_bytes == 0 else "multi"},
        "roofline": {"bound": "hbm", "achieved": hbm_achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": hbm_achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "scan_kernel<bf16, main>",
                     "alu": {"achieved": alu_achieved / 1e12, "peak": ALU_PEAK_LANE_OPS / 1e12,
                             "unit": "T lane-op/s", "frac": alu_achieved / ALU_PEAK_LANE_OPS,
                             "ops_per_channel_step": ALU_OPS_PER_CHANNEL_STEP},
                     "limiter": "VALU issue: 16 exp2 and ~100 other fp32 lane-ops per "
                                "channel-step put the ALU floor above the HBM time; the HBM "
                                "fraction is the metric's, the ALU fraction is what bounds it"},
        "hbm": {"achieved_GBps": hbm_achieved, "peak_GBps": HBM_PEAK_GBS,
                "frac": hbm_achieved / HBM_PEAK_GBS, "algorithmic_bytes": alg_bytes,
                "bytes_per_channel_step": alg_bytes / chsteps,
                "counter_GBps": (traffic / (kern_avg * 1e-3) / 1e9) if traffic else None,
                "copy_GBps": copy_GBps, "frac_of_copy": hbm_achieved / copy_GBps},
        "kernel_us": {"mean": kern_avg * 1e3, "p10": kern_ms[len(kern_ms) // 10] * 1e3,
                      "median": kern_ms[len(kern_ms) // 2] * 1e3,
                      "p90": kern_ms[(len(kern_ms) * 9) // 10] * 1e3},
        "kernel_us_mall_flushed": {"median": flushed[len(flushed) // 2] * 1e3,
                                   "p10": flushed[1] * 1e3, "p90": flushed[-2] * 1e3},
        "outputs_finite": ok,
        "settle_s": settle_s,
        "settle_launches": settle_n,
    }
    if not args.no_conv:
        rec["conv_fused_forward"] = bench_conv(w, torch, binding, synth, dev, 30, 100,
                                               kern_ms[len(kern_ms) // 2] * 1e3)
    if not args.no_bwd:
        rec["backward"] = bench_backward(w, torch, binding, dev, args.bwd_steps, args.bwd_warmup)
    if not args.no_block:
        rec["block_forward"] = bench_block(torch, binding, synth, dev, 10, 5)
    if not args.no_step:
        del t, out
        torch.cuda.empty_cache()
        rec["state_update"] = bench_state_update(args.step_steps, torch, binding, synth, dev)
    if not args.no_others:
        rec["other_workloads"], rec["seqlen_sweep"] = other_workloads(torch, binding, synth, dev)
    parity_ok = True
    if not args.no_cpu:
        refs, rec["cpu_baseline"] = cpu_baseline(x, w, args.cpu_seconds)
        rec["parity"] = timed_output_parity(out_h, last_h, refs, w.tol)
        parity_ok = rec["parity"] is None or rec["parity"]["ok"]
    else:
        rec["cpu_baseline"] = None
        rec["parity"] = None
    print(json.dumps(rec), flush=True)
    if not parity_ok:
        print("timed outputs differ from the oracle beyond the bound", file=sys.stderr)
        return 1
    return 0


if __name__ == "__main__":
    sys.exit(main())
