#!/usr/bin/env python3
"""Benchmark of the chunked SSD forward pass on one MI355X.

One step = one full forward pass (chunk_cb, chunk_state with the cumsum step
inside, state_passing, [seq_final], chunk_scan) over one batch of seeded synthetic
input already resident in HBM.  Prints ONE JSON line:

  value        tokens/s of the headline workload over the K timed steps, each
               step cold: a 1 GiB write and a read of it before the step
               (outside its HIP events) evict L2 and the 256 MB MALL, so every
               input comes from HBM, and leave the caches clean, so no
               write-back of the flush lands in the step; ms_per_step is the
               mean cold step
  warm         the same K steps back to back (wall clock between synchronisations)
  roofline     the dominant kernel's achieved algorithmic bytes/s (or FLOP/s) per
               launch, from HIP events recorded on the launch stream, against
               MI355X's published peak; traffic = its HBM bytes per launch from
               the committed FETCH_SIZE / WRITE_SIZE records (scaled by a plain
               copy's reading), traffic_requests = the same from the per-size
               request counters (null once the kernel sources change)
  step_ms      p10/p50/p90 of single steps between HIP events, cold and warm
  cpu_baseline the fp64 CPU oracle timed on a bounded sample of the same workload
  kernels      per-kernel breakdown of the headline workload (average ms per
               launch, achieved rate, fraction, counter-measured MFMA busy %
               where a record for these sources exists); chunk_cumsum is the
               standalone cumsum step, which ssd_fwd runs inside chunk_state
  workloads    the same forward measurements (cold and warm rates, TFLOP/s,
               per-kernel fractions) for every one of the five workloads
  backward     ssd_bwd on the same workload (all input gradients): time per call,
               and per stage (ssd_bwd_stage_times: HIP events between the
               stages of one call) placed on the roofline; backward_packed the
               same on the packed workload
  decode       the decode step (one token per sequence, state carried) on its own
               seeded workload: time per launch, tokens/s and its HBM roofline
  block        the convolution prologue and the gated forward

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 3]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "SSD fwd tokens/sec on 1 MI355X + % of bf16 MFMA / HBM roofline per kernel"
PEAK = {"bf16_mfma_tflops": 2500.0, "fp32_mfma_tflops": 157.3, "hbm_gbs": 8000.0}
DEFAULT_WORKLOAD = 3   # 16K tokens, N = 256: the configuration the roofline targets are quoted on
CSRC = os.path.join(ROOT, "ssd_chunked_scan_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


def kernel_source_hash():
    """sha256 over the HIP sources (sorted by name): identifies the kernels a
    counter record was taken from."""
    import hashlib
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".hpp", ".h")):
            h.update(name.encode())
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(f.read())
    return h.hexdigest()


def traffic_record(kernel, workload):
    """The committed HBM-traffic counter record of `kernel` on `workload`, or
    None when no record exists or the kernel sources changed since it was taken."""
    import glob
    src = kernel_source_hash()
    for path in sorted(glob.glob(os.path.join(PROFILES, "*hbm_traffic*.md"))):
        with open(path) as f:
            for line in f:
                if not line.startswith("traffic-record: "):
                    continue
                rec = json.loads(line[len("traffic-record: "):])
                if rec["kernel"] == kernel and rec["workload"] == workload and rec["source_sha256"] == src:
                    return rec
    return None


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload`: FETCH_SIZE + WRITE_SIZE,
    each scaled by what it reads for a plain device copy of known size in the
    same run; None without a current record."""
    rec = traffic_record(kernel, workload)
    return None if rec is None else int(rec["fetch_bytes"] + rec["write_bytes"])


def measured_traffic_requests(kernel, workload):
    """The same bytes from the L2-to-fabric request counters by request size
    (read: 32, 64 and 128 B requests; write: 64 B requests and the rest at 32
    B), which need no calibration; None without a current record."""
    rec = traffic_record(kernel, workload)
    return None if rec is None or "read_req_bytes" not in rec else int(rec["read_req_bytes"] + rec["write_req_bytes"])


def measured_mfma(kernel, workload):
    """Counter-measured MFMA busy percentage of `kernel` on `workload` (the
    MfmaUtil metric: MFMA busy cycles over active cycles x SIMDs) from the
    committed counter records, or None when no record exists or the kernels
    changed since."""
    import glob
    src = kernel_source_hash()
    for path in sorted(glob.glob(os.path.join(PROFILES, "*mfma_util*.md"))):
        with open(path) as f:
            for line in f:
                if not line.startswith("mfma-record: "):
                    continue
                rec = json.loads(line[len("mfma-record: "):])
                if rec["kernel"] == kernel and rec["workload"] == workload and rec["source_sha256"] == src:
                    return rec["mfma_busy_pct"]
    return None


def host_cpu():
    """(online CPUs, CPU model name) of this host, for the oracle baseline."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return os.cpu_count(), model


def percentiles(ms):
    v = sorted(ms)
    pick = lambda q: v[min(len(v) - 1, int(round(q * (len(v) - 1))))]
    return {"p10": round(pick(0.1), 5), "p50": round(pick(0.5), 5), "p90": round(pick(0.9), 5)}


def roofline_point(wk, sec, esz):
    """Place one kernel launch on the roofline.  The binding roof follows from the
    kernel's arithmetic intensity: below the ridge point (peak FLOP/s over peak
    bytes/s) HBM bounds it and `frac` is achieved bytes/s over the HBM peak; at or
    above it, achieved FLOP/s over the MFMA peak of the compute dtype.  Both rates
    are returned either way."""
    mfma_peak = PEAK["bf16_mfma_tflops"] if esz == 2 else PEAK["fp32_mfma_tflops"]
    ridge = mfma_peak * 1e12 / (PEAK["hbm_gbs"] * 1e9)
    flops, nbytes = wk.get("flops", 0.0), wk["bytes"]
    e = {"hbm_gbs": round(nbytes / sec / 1e9, 1), "hbm_frac": round(nbytes / sec / 1e9 / PEAK["hbm_gbs"], 4)}
    if flops:
        e.update(tflops=round(flops / sec / 1e12, 2), mfma_frac=round(flops / sec / 1e12 / mfma_peak, 4),
                 flop_per_byte=round(flops / nbytes, 1) if nbytes else None, ridge_flop_per_byte=round(ridge, 1))
    if flops and (not nbytes or flops / nbytes >= ridge):
        e.update(bound="mfma", achieved=e["tflops"], peak=mfma_peak, unit="TFLOP/s", frac=e["mfma_frac"])
    else:
        e.update(bound="hbm", achieved=e["hbm_gbs"], peak=PEAK["hbm_gbs"], unit="GB/s", frac=e["hbm_frac"])
    return e


def algorithmic_work(shape, esz, packed):
    """Per-launch algorithmic FLOPs (multiply-add = 2) and HBM bytes of each kernel.

    FLOPs count only what the method needs (the causal half of each Q x Q
    block); bytes count each tensor a kernel must read or write once."""
    b, T, H, P, N, G, Q = (shape[k] for k in ("batch", "seqlen", "nheads", "headdim", "dstate",
                                             "ngroups", "chunk"))
    nc = (T + Q - 1) // Q
    causal = (Q + 1) / (2.0 * Q)
    st = b * nc * H * P * N * esz            # chunk states (stored in the compute dtype)
    dcs = 2 * b * H * nc * Q * 4             # delta + cs
    cbb = b * nc * G * Q * Q * esz * (Q // 64 + 1) / (2 * (Q // 64))  # lower block triangle
    w = {
        "chunk_cumsum": dict(bytes=b * T * H * esz + H * 4 + dcs),
        "chunk_cb": dict(flops=2.0 * b * nc * Q * G * Q * N * causal,
                         bytes=2 * b * T * G * N * esz + cbb),
        # chunk_state runs the cumsum step too: it reads dt and writes delta and cs
        "chunk_state": dict(flops=2.0 * b * T * H * P * N,
                            bytes=b * T * H * P * esz + b * T * G * N * esz + b * T * H * esz + dcs + st),
        "state_passing": dict(bytes=2 * st + b * H * nc * 4 + 2 * b * H * P * N * 4),
        "chunk_scan": dict(flops=2.0 * b * T * H * P * Q * causal + 2.0 * b * T * H * N * P,
                           bytes=2 * b * T * H * P * esz + b * T * G * N * esz + dcs + st + cbb),
    }
    if packed is not None and packed is not False:
        w["seq_final"] = seq_final_work(shape, esz, packed)
    return w


def backward_stage_work(shape, esz, nseq=0):
    """Algorithmic FLOPs and HBM bytes of each stage of ssd_bwd (the names that
    ssd_bwd_stage_times reports), on the real tokens of the problem.

    The backward runs the forward's scan once more on the time-reversed problem
    (dy in the place of x, B and C swapped, unit step size), which gives the
    gradient states G_c and dx; the rest are products with those.  FLOPs count
    the MFMA work the method needs (causal halves only), bytes each tensor a
    stage must read or write once."""
    b, T, H, P, N, G, Q = (shape[k] for k in ("batch", "seqlen", "nheads", "headdim", "dstate",
                                             "ngroups", "chunk"))
    nc = (T + Q - 1) // Q
    causal = (Q + 1) / (2.0 * Q)
    X = b * T * H * P * esz                  # x, dy, dx
    BC = b * T * G * N * esz                 # B, C, dB, dC
    ST = b * nc * H * P * N * esz            # one set of chunk states
    V4 = b * H * nc * Q * 4                  # one fp32 value per (token, head)
    DT = b * T * H * esz                     # dt, ddt
    CB = b * nc * G * Q * Q * esz * (Q // 64 + 1) / (2 * (Q // 64))   # a lower block triangle
    PN4 = b * H * P * N * 4
    fwd = algorithmic_work(shape, esz, None)
    scan_flops = fwd["chunk_scan"]["flops"]
    w = {
        "chunk_cb": fwd["chunk_cb"], "chunk_state": fwd["chunk_state"], "state_passing": fwd["state_passing"],
        "chunk_cb_rev": fwd["chunk_cb"],
        "chunk_state_grad": dict(flops=2.0 * b * T * H * P * N, bytes=X + BC + V4 + ST),
        "inject_dfinal": dict(bytes=nseq * H * P * N * (4 + esz)),
        "state_passing_rev": dict(bytes=3 * ST + 2 * b * H * nc * 4 + 2 * PN4),
        # y' of the reversed problem; dx = delta y' + D dy; x . (G term), x . y', dy . x
        "chunk_scan_dx": dict(flops=scan_flops, bytes=3 * X + BC + CB + ST + 6 * V4),
        "chunk_scan_dy_hin": dict(flops=2.0 * b * T * H * N * P, bytes=X + BC + ST + 2 * V4),
        # M = sum over the group's heads of (dy x^T) o decay, with its row and column sums
        "m_rows_cols": dict(flops=2.0 * b * nc * H * Q * Q * P * causal, bytes=2 * X + 3 * CB + 4 * V4),
        "dl_ddt_dA_dD": dict(bytes=8 * V4 + 2 * DT),
        "dC": dict(flops=2.0 * b * T * G * N * Q * causal + 2.0 * b * T * H * P * N,
                   bytes=X + ST + CB + 2 * BC + 2 * V4),
        "dB": dict(flops=2.0 * b * T * G * N * Q * causal + 2.0 * b * T * H * P * N,
                   bytes=X + ST + CB + 2 * BC + 2 * V4),
        # the packed stream's chunk map: seq_idx read once, per-segment and per-chunk words written
        "chunk_map": dict(bytes=b * T * 4 + nseq * 16 + nc * 12),
    }
    return w


def seq_final_work(shape, esz, seq_idx):
    """Algorithmic FLOPs and bytes of seq_final on a packed stream (seq_idx: the
    host copy of the int32 ids, nseq taken from shape["nseq"]).  Per sequence
    whose last token t_e lies in chunk c: the rows of c from the later of the
    chunk start and the sequence start through t_e (x, B, and their delta and
    cs), the state entering c when the sequence was already open there, and the
    fp32 final state; every id without a token still gets its zero state
    written."""
    import numpy as np
    ids = np.asarray(seq_idx)
    H, P, N, G, Q = (shape[k] for k in ("nheads", "headdim", "dstate", "ngroups", "chunk"))
    nseq = shape["nseq"]
    flops, nbytes = 0.0, nseq * H * P * N * 4 + len(ids) * 4
    change = np.flatnonzero(np.diff(ids)) + 1
    starts = np.concatenate([[0], change])
    ends = np.concatenate([change - 1, [len(ids) - 1]])
    for st, te in zip(starts, ends):
        t0 = (te // Q) * Q
        rows = te - max(t0, st) + 1
        flops += 2.0 * rows * H * P * N
        nbytes += rows * (H * P * esz + G * N * esz + 2 * H * 4)
        if st < t0:
            nbytes += H * P * N * esz
    return dict(flops=flops, bytes=int(nbytes))


def run_cpu_baseline(inp, budget_s=20.0):
    """Time the fp64 oracle on sampled (batch, head) units of the same workload and
    extrapolate to the whole workload's tokens/s."""
    import numpy as np
    import oracle

    b, T, H, P = inp.x.shape
    units = b * H
    # one unit first, to size the sample to the time budget
    order = np.random.default_rng(0).permutation(units)
    mask = np.zeros(units, bool)
    mask[order[0]] = True
    t0 = time.perf_counter()
    oracle.forward(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, inp.initial_states, inp.seq_idx,
                   inp.nseq or None, inp.dt_softplus, unit_mask=mask.reshape(b, H))
    one = time.perf_counter() - t0
    k = int(max(1, min(units, budget_s / max(one, 1e-3))))
    mask[:] = False
    mask[order[:k]] = True
    times = []
    while True:   # repeat the sample while the budget allows (at most 5 runs); report the median
        t0 = time.perf_counter()
        oracle.forward(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, inp.initial_states, inp.seq_idx,
                       inp.nseq or None, inp.dt_softplus, unit_mask=mask.reshape(b, H))
        times.append(time.perf_counter() - t0)
        if len(times) >= 5 or sum(times) + times[-1] > budget_s:
            break
    dt = sorted(times)[len(times) // 2]
    full_time = dt * units / k
    nproc, model = host_cpu()
    return {"value": inp.real_tokens / full_time, "unit": "tokens/s", "cores": oracle.max_threads(),
            "kind": "oracle", "nproc": nproc, "cpu_model": model,
            "sample": f"{k} of {units} (batch, head) units, all {T} tokens each; median of "
                      f"{len(times)} runs of {dt:.2f} s, extrapolated x{units / k:.1f}",
            "seconds_measured": round(sum(times), 3)}


def run_backward(dev, inp, g, reps, warmup):
    """Time ssd_bwd (every input gradient) on the workload's inputs with a seeded
    dy and dfinal, between HIP events on the launch stream; outputs and workspaces
    preallocated.  Two ways: reading the forward's chunk intermediates from the
    workspace of the forward that produced y (a training step's order), and
    recomputing them inside."""
    import numpy as np
    import torch
    from ssd_chunked_scan_amd import ssd

    nseq = inp.nseq if inp.seq_idx is not None else None
    p = ssd.Problem(g.x, g.dt, g.A, g.B, g.C, inp.chunk, g.D, g.initial_states, g.seq_idx, nseq)
    fws = torch.empty(ssd.workspace_bytes(p), dtype=torch.uint8, device=dev)
    y, _ = ssd.fwd(g.x, g.dt, g.A, g.B, g.C, inp.chunk, D=g.D, initial_states=g.initial_states, seq_idx=g.seq_idx,
                   nseq=nseq, workspace=fws)
    rng = np.random.default_rng(7)
    dy = torch.from_numpy(rng.standard_normal(tuple(inp.x.shape)).astype(np.float32)).to(dev).to(g.x.dtype)
    dfin = torch.from_numpy(rng.standard_normal(p.final_shape()).astype(np.float32)).to(dev)
    ws = torch.empty(ssd.bwd_workspace_bytes(p), dtype=torch.uint8, device=dev)
    kw = dict(D=g.D, initial_states=g.initial_states, dfinal_states=dfin, workspace=ws, seq_idx=g.seq_idx,
              nseq=nseq)
    grads = ssd.bwd(g.x, g.dt, g.A, g.B, g.C, inp.chunk, y, dy, **kw)
    stream = torch.cuda.current_stream(dev)
    recomp = _event_ms(lambda: ssd.bwd(g.x, g.dt, g.A, g.B, g.C, inp.chunk, y, dy, grads=grads, **kw),
                       reps, warmup, stream)
    avg_r = sum(recomp) / len(recomp)
    out = {"workload": inp.name, "real_tokens": inp.real_tokens, "ms_recompute": round(avg_r, 5),
           "step_ms_recompute": percentiles(recomp), "workspace_bytes": int(ws.numel())}
    if nseq is None:
        saved = _event_ms(lambda: ssd.bwd(g.x, g.dt, g.A, g.B, g.C, inp.chunk, y, dy, grads=grads,
                                          fwd_workspace=fws, **kw), reps, warmup, stream)
        avg = sum(saved) / len(saved)
        out.update(ms=round(avg, 5), step_ms=percentiles(saved),
                   tokens_per_s=round(inp.real_tokens / (avg / 1e3), 1),
                   note="all input gradients; ms reads the forward's chunk intermediates from that forward's "
                        "workspace, ms_recompute recomputes them inside")
    else:
        out.update(ms=round(avg_r, 5), tokens_per_s=round(inp.real_tokens / (avg_r / 1e3), 1),
                   note="all input gradients of a packed stream: the stream is laid out again with every "
                        "sequence starting at a chunk start, and the chunk intermediates recomputed there")
    # per stage: HIP events between the stages of the same call (ssd_bwd_stage_times),
    # mean over the reps, each placed on the roofline with its algorithmic work
    kw_st = dict(kw, fwd_workspace=fws if nseq is None else None)
    sums = {}
    for r in range(warmup + reps):
        stages = []
        ssd.bwd(g.x, g.dt, g.A, g.B, g.C, inp.chunk, y, dy, grads=grads, stage_times=stages, **kw_st)
        if r >= warmup:
            for name, ms in stages:
                sums[name] = sums.get(name, 0.0) + ms
    shape = dict(batch=p.b, seqlen=p.T, nheads=p.H, headdim=p.P, dstate=p.N, ngroups=p.G, chunk=p.Q)
    esz = 2 if g.x.dtype == torch.bfloat16 else 4
    work = backward_stage_work(shape, esz, nseq or 0)
    stages_out = {}
    for name, tot in sums.items():
        ms = tot / reps
        e = {"ms": round(ms, 5)}
        if name in work:
            e.update(roofline_point(work[name], ms / 1e3, esz))
        stages_out[name] = e
    out["stages"] = stages_out
    out["stages_note"] = ("events between the stages of one ssd_bwd_stage_times call, mean of the reps; "
                          "the events add a little to the total")
    return out


def run_decode(dev, reps, warmup):
    """Time the decode step (ssd_step) on the seeded decode workload: HIP events
    around each launch on the launch stream, the state carried from launch to
    launch as in serving."""
    import torch
    from ssd_chunked_scan_amd import ssd
    from ssd_chunked_scan_amd import workloads as wl

    s = wl.decode_inputs()
    g = s.to(dev)
    state = g.state.clone()
    y = torch.empty_like(g.x)
    b, H, P = s.x.shape
    G, N = s.B.shape[1], s.B.shape[2]
    esz = 2 if s.x.dtype == torch.bfloat16 else 4
    stream = torch.cuda.current_stream(dev)

    def one():
        ssd.step(g.x, g.dt, g.A, g.B, g.C, state, D=g.D, y=y)

    for _ in range(warmup):
        one()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b_ in ev:
        a.record(stream)
        one()
        b_.record(stream)
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b_) for a, b_ in ev]
    avg = sum(ms) / len(ms)
    # the state is read and written once; x and y once; dt, B and C once
    nbytes = 2 * b * H * P * N * 4 + 2 * b * H * P * esz + b * H * esz + 2 * b * G * N * esz + 2 * H * 4
    ach = nbytes / (avg / 1e3) / 1e9
    return {"workload": s.name, "batch": b, "nheads": H, "headdim": P, "dstate": N, "ngroups": G,
            "ms": round(avg, 5), "step_ms": percentiles(ms), "tokens_per_s": round(b / (avg / 1e3), 1),
            "roofline": {"kernel": "ssd_step", "bound": "hbm", "achieved": round(ach, 1),
                         "peak": PEAK["hbm_gbs"], "unit": "GB/s", "frac": round(ach / PEAK["hbm_gbs"], 4),
                         "traffic": measured_traffic("ssd_step", s.name), "algorithmic_bytes": int(nbytes)}}


def _event_ms(fn, reps, warmup, stream):
    """Per-call times of fn (ms) between HIP events on the launch stream."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b_ in ev:
        a.record(stream)
        fn()
        b_.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b_) for a, b_ in ev]


def run_block(dev, inp, g, reps, warmup):
    """The Mamba-2 block's steps around the SSD on the workload's shape: the
    convolution prologue (ssd_conv1d_silu) and the forward with the SiLU(z) gate
    fused into its last kernel (ssd_fwd_gated), each timed alone and chained,
    beside the plain forward and an unfused gate (torch's y * silu(z)) for
    comparison.  Seeded block inputs; HIP events on the launch stream."""
    import torch
    from ssd_chunked_scan_amd import ssd
    from ssd_chunked_scan_amd import workloads as wl

    blk = wl.block_inputs(inp, seed=4000)
    b, T, H, P = inp.x.shape
    G, N = inp.B.shape[2], inp.B.shape[3]
    nseq = inp.nseq if inp.seq_idx is not None else None
    xbc, wt, bias, z = (t.to(dev) for t in (blk.xbc, blk.weight, blk.bias, blk.z))
    x, Bm, Cm = ssd.conv1d_silu(xbc, wt, H, P, G, N, bias=bias, seq_idx=g.seq_idx)
    p = ssd.Problem(x, g.dt, g.A, Bm, Cm, inp.chunk, g.D, g.initial_states, g.seq_idx, nseq)
    ws = torch.empty(ssd.workspace_bytes(p), dtype=torch.uint8, device=dev)
    y = torch.empty_like(x)
    yg = torch.empty_like(x)
    fin = torch.empty(p.final_shape(), dtype=torch.float32, device=dev)
    kw = dict(D=g.D, initial_states=g.initial_states, seq_idx=g.seq_idx, nseq=nseq, final_states=fin, workspace=ws)
    stream = torch.cuda.current_stream(dev)

    conv = lambda: ssd.conv1d_silu(xbc, wt, H, P, G, N, bias=bias, seq_idx=g.seq_idx, x=x, B=Bm, C=Cm)
    gated = lambda: ssd.fwd_gated(x, g.dt, g.A, Bm, Cm, inp.chunk, z, y=yg, **kw)
    plain = lambda: ssd.fwd(x, g.dt, g.A, Bm, Cm, inp.chunk, y=y, **kw)
    unfused_gate = lambda: torch.mul(y, torch.nn.functional.silu(z), out=yg)

    def chain():
        conv()
        gated()

    ms = {k: sum(v) / len(v) for k, v in (("conv", _event_ms(conv, reps, warmup, stream)),
                                         ("fwd_gated", _event_ms(gated, reps, warmup, stream)),
                                         ("fwd", _event_ms(plain, reps, warmup, stream)),
                                         ("unfused_gate", _event_ms(unfused_gate, reps, warmup, stream)),
                                         ("block", _event_ms(chain, reps, warmup, stream)))}
    esz = 2 if x.dtype == torch.bfloat16 else 4
    CC = H * P + 2 * G * N
    conv_bytes = 2 * b * T * CC * esz + CC * blk.width * 4 + CC * 4 + (T * 4 if nseq else 0)
    ach = conv_bytes / (ms["conv"] / 1e3) / 1e9
    return {"conv_ms": round(ms["conv"], 5), "fwd_gated_ms": round(ms["fwd_gated"], 5),
            "fwd_ms": round(ms["fwd"], 5), "gate_cost_ms": round(ms["fwd_gated"] - ms["fwd"], 5),
            "unfused_gate_ms": round(ms["unfused_gate"], 5), "block_ms": round(ms["block"], 5),
            "block_tokens_per_s": round(inp.real_tokens / (ms["block"] / 1e3), 1), "conv_width": blk.width,
            "conv_roofline": {"kernel": "conv1d_silu", "bound": "hbm", "achieved": round(ach, 1),
                              "peak": PEAK["hbm_gbs"], "unit": "GB/s", "frac": round(ach / PEAK["hbm_gbs"], 4),
                              "traffic": measured_traffic("conv1d_silu", inp.name),
                              "algorithmic_bytes": int(conv_bytes)},
            "note": "block_ms = conv1d_silu + fwd_gated back to back; unfused_gate_ms is torch's "
                    "y * silu(z) on the plain forward's y, for comparison only"}


def progress(msg):
    """One line on stderr per finished phase (stdout carries only the JSON line)."""
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def measure_forward(idx, dev, steps, warmup, kreps, flush):
    """The forward on workload `idx`: K cold steps (each after a cache-evicting
    write, outside its HIP events), K warm steps back to back (wall clock), and
    the per-kernel breakdown through the per-step entry points (HIP events on
    the launch stream around each launch, kernels in ssd_fwd's order so that the
    caches between them are as in a real forward)."""
    import numpy as np
    import torch
    from ssd_chunked_scan_amd import ssd
    from ssd_chunked_scan_amd import workloads as wl

    cfg = wl.WORKLOADS[idx]
    t_start = time.perf_counter()
    inp = wl.workload(idx)
    g = inp.to(dev)
    progress(f"workload {idx} inputs ready ({time.perf_counter() - t_start:.1f} s)")
    nseq = inp.nseq if inp.seq_idx is not None else None
    p = ssd.Problem(g.x, g.dt, g.A, g.B, g.C, inp.chunk, g.D, g.initial_states, g.seq_idx, nseq)
    ws = torch.empty(ssd.workspace_bytes(p), dtype=torch.uint8, device=dev)
    y = torch.empty_like(g.x)
    fin = torch.empty(p.final_shape(), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        ssd.fwd(g.x, g.dt, g.A, g.B, g.C, inp.chunk, D=g.D, initial_states=g.initial_states,
                seq_idx=g.seq_idx, nseq=nseq, y=y, final_states=fin, workspace=ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # cold: K steps, each after a 1 GiB write and a read of the same buffer
    # (outside the events).  The write evicts L2 and the MALL; the read makes
    # the lines left in them clean, so that no write-back of the flush itself
    # falls inside the timed step.
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    sink = torch.empty((), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    for r in range(steps):
        flush.fill_(float(r))
        torch.sum(flush, 0, out=sink)
        pairs[r][0].record(stream)
        step()
        pairs[r][1].record(stream)
    torch.cuda.synchronize()
    cold = [a.elapsed_time(b_) for a, b_ in pairs]
    # warm: K steps back to back, wall clock between synchronisations
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    warm_s = time.perf_counter() - t0
    # warm single steps between events
    wreps = min(steps, 100)
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(wreps)]
    for a, b_ in pairs:
        a.record(stream)
        step()
        b_.record(stream)
    torch.cuda.synchronize()
    warm_ev = [a.elapsed_time(b_) for a, b_ in pairs]

    # per-kernel breakdown
    names = ["chunk_cumsum", "chunk_cb", "chunk_state", "state_passing"]
    if inp.seq_idx is not None:
        names.append("seq_final")
    names.append("chunk_scan")
    delta = torch.empty((p.b, p.H, p.nc, p.Q), dtype=torch.float32, device=dev)
    cs = torch.empty_like(delta)
    cb = torch.empty(p.cb_shape(), dtype=g.x.dtype, device=dev)
    states = torch.empty((p.b, p.nc, p.H, p.P, p.N), dtype=g.x.dtype, device=dev)
    seg_end = torch.empty((max(p.nseq, 1),), dtype=torch.int32, device=dev)
    ybuf = torch.empty_like(g.x)
    calls = {
        "chunk_cumsum": lambda: ssd.chunk_cumsum(p, delta, cs),
        "chunk_cb": lambda: ssd.chunk_cb(p, cb),
        "chunk_state": lambda: ssd.chunk_state(p, delta, cs, cb, states),
        "state_passing": lambda: ssd.state_passing(p, cs, states, None if inp.seq_idx is not None else fin),
        "seq_final": lambda: ssd.seq_final_states(p, delta, cs, states, fin, seg_end),
        "chunk_scan": lambda: ssd.chunk_scan(p, delta, cs, cb, states, ybuf),
    }
    ev = {n: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(kreps)] for n in names}
    for _ in range(2):
        for n in names:
            calls[n]()
    torch.cuda.synchronize()
    for r in range(kreps):
        for n in names:
            ev[n][r][0].record(stream)
            calls[n]()
            ev[n][r][1].record(stream)
    torch.cuda.synchronize()
    kms = {n: sum(a.elapsed_time(b_) for a, b_ in ev[n]) / kreps for n in names}

    esz = 2 if g.x.dtype == torch.bfloat16 else 4
    shape = dict(inp.shape, nseq=nseq or 0)
    work = algorithmic_work(shape, esz, None if inp.seq_idx is None else inp.seq_idx.numpy())
    kernels = {}
    for n in names:
        kernels[n] = dict(ms=round(kms[n], 5), **roofline_point(work[n], kms[n] / 1e3, esz))
        kernels[n]["algorithmic_bytes"] = int(work[n]["bytes"])
        kernels[n]["traffic"] = measured_traffic(n, cfg["name"])
        kernels[n]["traffic_requests"] = measured_traffic_requests(n, cfg["name"])
        if work[n].get("flops"):
            kernels[n]["mfma_busy_pct"] = measured_mfma(n, cfg["name"])
    kernels["chunk_cumsum"]["note"] = "standalone; ssd_fwd runs this step inside chunk_state"
    fwd_names = [n for n in names if n != "chunk_cumsum"]
    total_flops = sum(work[n].get("flops", 0.0) for n in fwd_names)
    cold_ms = sum(cold) / len(cold)
    progress(f"workload {idx} forward measured ({time.perf_counter() - t_start:.1f} s)")
    return {
        "inp": inp, "g": g, "work": work, "names": fwd_names, "kms": kms, "esz": esz,
        "summary": {
            "workload": cfg["name"], "batch": inp.x.shape[0], "seqlen": inp.x.shape[1],
            "real_tokens": inp.real_tokens,
            "cold": {"ms": round(cold_ms, 5), **percentiles(cold),
                     "tokens_per_s": round(inp.real_tokens * len(cold) / (sum(cold) / 1e3), 1),
                     "tflops": round(total_flops / (cold_ms / 1e3) / 1e12, 2)},
            "warm": {"ms": round(warm_s * 1e3 / steps, 5), **percentiles(warm_ev),
                     "tokens_per_s": round(inp.real_tokens * steps / warm_s, 1),
                     "tflops": round(total_flops / (warm_s / steps) / 1e12, 2)},
            "kernels": kernels,
        },
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # a forward is ~0.1 ms: enough steps that clocks and queues settle (still milliseconds)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=DEFAULT_WORKLOAD)
    ap.add_argument("--only-headline", action="store_true", help="skip the other four workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode-step measurement")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward measurement")
    ap.add_argument("--no-block", action="store_true", help="skip the block (conv + gate) measurement")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle work")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first run a plain device copy of this many MiB (3 times), as the "
                         "reference kernel for scaling hardware byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "the multi-GPU path is a design, not code", file=sys.stderr)
        sys.exit(2)

    import torch
    from ssd_chunked_scan_amd import ssd
    from ssd_chunked_scan_amd import workloads as wl

    ssd.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB
    kreps = max(5, min(args.steps, 50))
    head = measure_forward(args.workload, dev, args.steps, args.warmup, kreps, flush)
    inp, g = head["inp"], head["g"]
    cfg = wl.WORKLOADS[args.workload]
    summ = head["summary"]
    kernels = summ["kernels"]
    names = head["names"]
    kms = head["kms"]
    dom = max(names, key=lambda n: kms[n])
    kd = kernels[dom]
    work = head["work"]
    roofline = {"kernel": dom, "bound": kd["bound"], "achieved": kd["achieved"], "peak": kd["peak"],
                "unit": kd["unit"], "frac": kd["frac"], "mfma_frac": kd.get("mfma_frac"),
                "hbm_frac": kd["hbm_frac"], "flop_per_byte": kd.get("flop_per_byte"),
                "traffic": measured_traffic(dom, cfg["name"]), "traffic_unit": "HBM bytes per launch",
                "traffic_requests": measured_traffic_requests(dom, cfg["name"]),
                "algorithmic_bytes": int(work[dom]["bytes"]),
                "mfma_busy_pct": measured_mfma(dom, cfg["name"])}
    workloads = {}
    for idx in sorted(wl.WORKLOADS):
        if idx == args.workload:
            workloads[str(idx)] = summ
        elif not args.only_headline:
            other = measure_forward(idx, dev, args.steps, args.warmup, kreps, flush)
            workloads[str(idx)] = other["summary"]
            del other
            torch.cuda.empty_cache()
    del flush
    torch.cuda.empty_cache()

    decode = None if args.no_decode else run_decode(dev, kreps * 2, 5)
    progress("decode measured")
    backward = None if args.no_backward else run_backward(dev, inp, g, max(5, min(kreps, 20)), 3)
    backward_packed = None
    if not args.no_backward and not args.only_headline and wl.WORKLOADS[args.workload].get("packed") is None:
        pk = wl.workload(4)
        backward_packed = run_backward(dev, pk, pk.to(dev), max(5, min(kreps, 20)), 3)
        del pk
    progress("backward measured")
    block = None if args.no_block else run_block(dev, inp, g, kreps, 3)
    progress("block measured")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = run_cpu_baseline(inp, args.cpu_budget)
        progress("cpu baseline measured")

    b, T, H, P = inp.x.shape
    esz = head["esz"]
    cold = summ["cold"]
    line = {
        "metric": METRIC, "value": cold["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": cold["ms"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if esz == 2 else "f32", "data": "synthetic (seeded, see workloads.py)",
        "config": {"workload": cfg["name"], "batch": b, "seqlen": T, "nheads": H, "headdim": P,
                   "dstate": inp.B.shape[3], "ngroups": inp.B.shape[2], "chunk": inp.chunk,
                   "real_tokens": inp.real_tokens},
        "timing": "value and ms_per_step: the K timed steps, each cold (a 1 GiB write and a read of it "
                  "before the step, outside its HIP events, evict L2 and MALL and leave them clean); "
                  "warm: the same K steps back to back",
        "tflops": cold["tflops"],
        "warm": summ["warm"],
        "roofline": roofline,
        "step_ms": {"cold": {k: cold[k] for k in ("p10", "p50", "p90")},
                    "warm": {k: summ["warm"][k] for k in ("p10", "p50", "p90")}},
        "cpu_baseline": cpu,
        "kernels": kernels,
        "workloads": workloads,
        "backward": backward,
        "backward_packed": backward_packed,
        "decode": decode,
        "block": block,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
