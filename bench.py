#!/usr/bin/env python3
"""Throughput of the Based layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-extra]

A step is one layer forward over the 360M-shaped workload (B=8, H=16,
L=2048, d_k=16, d_v=64, bf16 q/k/v, fp32 outputs): the causal Taylor linear
attention and the window-64 softmax attention on the same inputs, in one
based_layer_fwd call (the state-only pass, the segment scan and the fused
main pass).  ``value`` is sequence positions per second (B*L per step; every
position covers all 16 heads).  The two attentions are also timed as
separate calls (based_linattn_fwd, based_swa_fwd) for comparison.

Inputs are resident in HBM before timing starts.  Eight copies of the input
set are cycled so that successive steps do not find their inputs in the
256 MB last-level (Infinity) cache.  Kernels run on torch's current stream.
Every timed region is one loop of back-to-back calls of one operation with
events on that stream at its two ends only (an event pair around every
launch would cost the GPU several microseconds per call): the step's
duration is the layer operation's duration, and operations compared side by
side (the two separate calls, the two backward calls) get a loop each.

Also reported (same JSON line): the roofline of the dominant kernel, the
layer backward on the step's workload (based_linattn_bwd + based_swa_bwd:
gradients of both attentions for a seeded upstream gradient), the BaseConv
gate on the 360M model's hidden states (8 x 2048 tokens x 1024 channels,
3 taps), the other
forward workloads (1.3B-shaped, 32k long-context), recurrent decode
(256 sequences x 16 heads, 1000 steps) and the fp64 CPU oracle timed on a
bounded sample of the step's workload on this host's cores.
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2516.6  # dense bf16 matrix peak
METRIC = "Based layer fwd tokens/s @L=2k-32k + decode tokens/s; % MFMA/HBM roofline"

D_PHI = 273
D_CMP = 153  # rows of the compact decode state (one per unordered feature pair)


def lin_bytes(dv, es=2):
    """Algorithmic HBM bytes per (position, head) of the linear attention:
    q, k, v read once, y (fp32) written once."""
    return (2 * 16 + dv) * es + 4 * dv


def lin_flops(dv):
    """Algorithmic flops per (position, head): state update 2*D*dv, readout
    2*D*dv, z update D, denominator 2*D (D = 273 Taylor features)."""
    return 4 * D_PHI * dv + 3 * D_PHI


def swa_flops(dv, window=64, dqk=16):
    """Window attention per (position, head): scores 2*W*d_qk, weighted sum 2*W*dv."""
    return 2 * window * (dqk + dv)


def swa_bytes(dv, es=2):
    return (2 * 16 + dv) * es + 4 * dv


def layer_bytes(dv, es=2):
    """Both attentions in one pass: q, k, v read once, y_lin and y_swa written."""
    return (2 * 16 + dv) * es + 2 * 4 * dv


def bwd_bytes(dv, es=2):
    """Algorithmic HBM bytes per (position, head) of one attention's backward:
    q, k, v read, y and dy (fp32) read, dq, dk, dv (fp32) written."""
    return (2 * 16 + dv) * es + 2 * 4 * dv + (2 * 16 + dv) * 4


def decode_bytes(dv=64, window=64, es=2, rows=D_PHI):
    """Per head-step: S and z read + written (fp32, `rows` state rows: 273,
    or 153 in the compact layout), the ring's other window-1 slots read,
    q/k/v read, one ring slot written, y_lin and y_swa written."""
    return (2 * rows * dv * 4 + 2 * rows * 4 + (window - 1) * (16 + dv) * es + (2 * 16 + dv) * es
            + (16 + dv) * es + 2 * dv * 4)


# Kernel sources each timed operation is built from (a profile taken on other
# sources no longer describes the kernel).
OP_SOURCES = {
    "layer": ["linattn_mfma.hip", "launchers.h", "based_device.h"],
    "bwd": ["linattn_bwd_mfma.hip", "swa_bwd_mfma.hip", "linattn_mfma.hip", "launchers.h", "based_device.h"],
    "decode": ["decode.hip", "launchers.h", "based_device.h"],
    "decode_compact": ["decode.hip", "launchers.h", "based_device.h"],
    "baseconv": ["baseconv.hip", "launchers.h", "based_device.h"],
    "decay": ["linattn_mfma.hip", "launchers.h", "based_device.h"],
}
# rocprofv3 kernel-name fragments of each operation's launches
OP_KERNELS = {
    "layer": ["linattn_mfma_kernel<4, 1, 0, 0>", "linattn_state_kernel<4, 0, 1>", "seg_scan_kernel"],
    "bwd": ["query_pass_kernel", "key_pass_kernel", "key_state_kernel", "slice_sum_kernel",
            "linattn_state_kernel<4, 0, 1>", "linattn_state_kernel<2, 0, 2>", "swa_bwd_mfma_kernel<4>"],
    "decode": ["decode_step_kernel<unsigned short, 64, 273>"],
    "decode_compact": ["decode_step_kernel<unsigned short, 64, 153>"],
    "baseconv": ["baseconv_kernel"],
    "decay": ["linattn_mfma_kernel<4, 0, 1, 0>", "linattn_state_kernel<4, 1, 1>"],
}
# the backward's last launch of each call (based_linattn_bwd, then based_swa_bwd)
BWD_KERNEL = "swa_bwd_mfma_kernel"
# the step's last launch of each call (marks the end of the timed step in a trace)
STEP_KERNEL = "linattn_mfma_kernel<4, 1, 0, 0>"
COPY_BYTES = 512 << 20


def source_hash(op):
    h = hashlib.sha256()
    for f in OP_SOURCES[op]:
        with open(os.path.join(ROOT, "linear_attention_lm_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def copy_calibration(reps=10):
    """A plain device copy of COPY_BYTES: the bandwidth this GPU reaches on a
    streaming kernel, and the reference that scales the FETCH_SIZE /
    WRITE_SIZE counters to bytes."""
    src = torch.empty(COPY_BYTES // 4, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    return {"bytes_read": COPY_BYTES, "bytes_written": COPY_BYTES, "us": ms * 1e3,
            "gbs": 2 * COPY_BYTES / (ms * 1e-3) / 1e9}


def load_traffic(op):
    """Measured HBM bytes per call of `op` from the committed counter profile,
    or None when the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{op}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("source_hash") != source_hash(op):
        return None
    return rec["bytes_per_call"]


def time_loop(fn, steps):
    """Mean milliseconds per call of `steps` back-to-back calls fn(i) on the
    current stream, bracketed by a device synchronize and an event on each
    side."""
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(steps):
        fn(i)
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


def step_parity(cfg, dev_set, y_lin, y_swa, layer, heads=((0, 0), (-1, -1))):
    """The step's outputs on its first input set against the fp64 oracle, on
    sampled (batch, head) pairs: per-row infinity-norm relative error."""
    import numpy as np

    from oracle import based_oracle as O

    layer(0)
    torch.cuda.synchronize()
    q, k, v = (t.cpu() for t in dev_set)
    worst = {"y_lin": 0.0, "y_swa": 0.0}
    for b, h in heads:
        yl = O.linattn_chunked(q[b, h], k[b, h], v[b, h], 64)[0]
        ys = O.swa(q[b, h], k[b, h], v[b, h], cfg.window)
        for name, got, ref in (("y_lin", y_lin[b, h], yl), ("y_swa", y_swa[b, h], ys)):
            g = got.double().cpu().numpy()
            e = float((np.abs(g - ref).max(-1) / np.abs(ref).max(-1)).max())
            worst[name] = max(worst[name], e)
    tol = 2e-3 if cfg.dtype == "bf16" else 1e-5
    if max(worst.values()) > tol:
        raise SystemExit(f"step parity failed: {worst} (tolerance {tol})")
    return {"heads": [list(x) for x in heads], "rowinf_rel": worst, "tol": tol}


def bench_fwd(lal, cfg, steps, warmup, nbuf=8, fused=True, settle=0, check=False):
    """Time `steps` layer forwards: one based_layer_fwd call per step, or
    (fused=False) based_linattn_fwd and based_swa_fwd, each in a loop of its
    own (the step's time is their sum).  check: first compare the outputs
    with the oracle on sampled heads; settle: untimed calls of the same
    operation before the `warmup` steps, until the GPU clocks settle.
    Returns a dict."""
    q, k, v = synth.fwd_inputs(cfg, 0)
    sets = []
    for i in range(nbuf):
        sets.append(tuple(t.to("cuda") for t in (q, k, v)))
    B, H, L, dv = cfg.B, cfg.H, cfg.L, cfg.dv
    y_lin = torch.empty(B, H, L, dv, device="cuda")
    y_swa = torch.empty(B, H, L, dv, device="cuda")
    ws_bytes = lal.linattn_workspace_bytes(B, H, L, dv)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")

    def layer(i):
        qq, kk, vv = sets[i % nbuf]
        lal.layer_fwd(qq, kk, vv, cfg.window, y_lin=y_lin, y_swa=y_swa, workspace=ws)

    def lin(i):
        qq, kk, vv = sets[i % nbuf]
        lal.linattn_fwd(qq, kk, vv, y=y_lin, workspace=ws)

    def swa(i):
        qq, kk, vv = sets[i % nbuf]
        lal.swa_fwd(qq, kk, vv, cfg.window, y=y_swa)

    parity = None
    if check:
        parity = step_parity(cfg, sets[0], y_lin, y_swa, layer)
    # untimed calls of the timed operation until the GPU clocks settle
    for i in range(settle):
        if fused:
            layer(i)
        else:
            lin(i)
            swa(i)
    for i in range(warmup):
        if fused:
            layer(i)
        else:
            lin(i)
            swa(i)
    th = B * H * L
    es = 2 if cfg.dtype == "bf16" else 4
    if fused:
        ms = time_loop(layer, steps)
        lb = layer_bytes(dv, es) * th
        out = {"layer_us": ms * 1e3, "layer_bytes": lb, "layer_hbm_gbs": lb / (ms * 1e-3) / 1e9,
               "layer_alg_tflops": (lin_flops(dv) + swa_flops(dv)) * th / (ms * 1e-3) / 1e12}
    else:
        tl, ts = time_loop(lin, steps), time_loop(swa, steps)
        ms = tl + ts
        lb, sb = lin_bytes(dv, es) * th, swa_bytes(dv, es) * th
        out = {"linattn_us": tl * 1e3, "swa_us": ts * 1e3, "linattn_bytes": lb, "swa_bytes": sb,
               "linattn_hbm_gbs": lb / (tl * 1e-3) / 1e9, "swa_hbm_gbs": sb / (ts * 1e-3) / 1e9}
    out.update({"workload": cfg.name, "B": B, "H": H, "L": L, "d_k": 16, "d_v": dv, "window": cfg.window,
                "dtype": cfg.dtype, "fused": fused, "ms_per_step": ms, "tokens_per_s": B * L / (ms * 1e-3),
                "settle_calls": settle})
    if parity is not None:
        out["parity"] = parity
    return out


def bench_tiny(lal, cfg, calls=200):
    """The tiny fp32 layer (launch-bound): microseconds per call of
    back-to-back calls, and the latency of one call on an idle stream
    (median of 50 calls, an event pair around each)."""
    q, k, v = (t.to("cuda") for t in synth.fwd_inputs(cfg, 0))
    y_lin = torch.empty(cfg.B, cfg.H, cfg.L, cfg.dv, device="cuda")
    y_swa = torch.empty_like(y_lin)
    call = lambda i: lal.layer_fwd(q, k, v, cfg.window, y_lin=y_lin, y_swa=y_swa)
    for i in range(50):
        call(i)
    ms = time_loop(call, calls)
    lat = []
    for i in range(50):
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        call(i)
        e1.record()
        torch.cuda.synchronize()
        lat.append(e0.elapsed_time(e1) * 1e3)
    lat.sort()
    return {"workload": cfg.name, "B": cfg.B, "H": cfg.H, "L": cfg.L, "d_v": cfg.dv, "dtype": cfg.dtype,
            "us_per_call_back_to_back": ms * 1e3, "us_latency_median": lat[len(lat) // 2],
            "us_latency_p10": lat[5], "us_latency_p90": lat[45], "calls": calls}


def bwd_inputs(lal, cfg, nbuf=8):
    """Input sets of the layer backward: q, k, v, a seeded upstream gradient
    dy and the forward outputs y_lin, y_swa (made here, before any timing)."""
    q, k, v = synth.fwd_inputs(cfg, 0)
    dy = synth.upstream_grad(cfg, 0)
    sets = []
    for _ in range(nbuf):
        qd, kd, vd, dyd = (t.to("cuda") for t in (q, k, v, dy))
        y_lin, y_swa = lal.layer_fwd(qd, kd, vd, cfg.window)
        sets.append((qd, kd, vd, dyd, y_lin, y_swa))
    torch.cuda.synchronize()
    return sets


def bench_bwd(lal, cfg, steps, warmup, sets, settle=0):
    """Time `steps` layer backwards: based_linattn_bwd and based_swa_bwd, each
    in a loop of its own over the prepared input sets (the step's time is
    their sum), after `settle` + `warmup` untimed calls of each.  Returns a
    dict."""
    nbuf = len(sets)
    B, H, L, dv = cfg.B, cfg.H, cfg.L, cfg.dv
    ws = torch.empty(max(1, lal.linattn_bwd_workspace_bytes(B, H, L, dv)), dtype=torch.uint8, device="cuda")
    gq = torch.empty(B, H, L, 16, device="cuda")
    gk = torch.empty_like(gq)
    gv = torch.empty(B, H, L, dv, device="cuda")

    def lin(i):
        qd, kd, vd, dyd, y_lin, y_swa = sets[i % nbuf]
        lal.linattn_bwd(qd, kd, vd, y_lin, dyd, dq=gq, dk=gk, dv=gv, workspace=ws)

    def swa(i):
        qd, kd, vd, dyd, y_lin, y_swa = sets[i % nbuf]
        lal.swa_bwd(qd, kd, vd, y_swa, dyd, cfg.window, dq=gq, dk=gk, dv=gv)

    for i in range(settle + warmup):
        lin(i)
        swa(i)
    tl, ts = time_loop(lin, steps), time_loop(swa, steps)
    ms = tl + ts
    th = B * H * L
    b1 = bwd_bytes(dv) * th
    return {"workload": cfg.name, "B": B, "H": H, "L": L, "d_k": 16, "d_v": dv, "window": cfg.window,
            "dtype": cfg.dtype, "ms_per_step": ms, "tokens_per_s": B * L / (ms * 1e-3),
            "linattn_bwd_us": tl * 1e3, "swa_bwd_us": ts * 1e3,
            "bytes_per_call": b1, "linattn_bwd_hbm_gbs": b1 / (tl * 1e-3) / 1e9,
            "swa_bwd_hbm_gbs": b1 / (ts * 1e-3) / 1e9,
            "layer_bwd_hbm_frac": 2 * b1 / ((tl + ts) * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "traffic_bytes_per_step": load_traffic("bwd")}


def bench_baseconv(lal, cfg, steps, warmup, nbuf=8, settle=0):
    """Time the BaseConv gate over `nbuf` resident input sets, after `settle` +
    `warmup` untimed calls.  Bytes per element: x and u read once (dtype), y
    written (fp32)."""
    x, u, h, b = synth.baseconv_inputs(cfg, 0)
    sets = [(x.to("cuda"), u.to("cuda")) for _ in range(nbuf)]
    hd, bd = h.to("cuda"), b.to("cuda")
    y = torch.empty(cfg.B, cfg.L, cfg.D, device="cuda")
    for i in range(settle + warmup):
        lal.baseconv_fwd(*sets[i % nbuf], hd, bd, y=y)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(steps):
        lal.baseconv_fwd(*sets[i % nbuf], hd, bd, y=y)
    t1.record()
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) / steps * 1e3
    es = 2 if cfg.dtype == "bf16" else 4
    nbytes = cfg.B * cfg.L * cfg.D * (2 * es + 4)
    return {"workload": cfg.name, "B": cfg.B, "L": cfg.L, "D": cfg.D, "K": cfg.K, "dtype": cfg.dtype,
            "us_per_call": us, "tokens_per_s": cfg.B * cfg.L / (us * 1e-6), "bytes_per_call": nbytes,
            "hbm_gbs": nbytes / (us * 1e-6) / 1e9, "hbm_frac": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "traffic_bytes_per_call": load_traffic("baseconv")}


def bench_decay(lal, cfg, steps, warmup, nbuf=8, settle=0):
    """Time the decayed linear attention (per-head decays from
    synth.decay_rates) over `nbuf` resident input sets, after `settle` +
    `warmup` untimed calls."""
    q, k, v = synth.fwd_inputs(cfg, 0)
    sets = [tuple(t.to("cuda") for t in (q, k, v)) for _ in range(nbuf)]
    g = synth.decay_rates(cfg.H).to("cuda")
    B, H, L, dv = cfg.B, cfg.H, cfg.L, cfg.dv
    y = torch.empty(B, H, L, dv, device="cuda")
    ws = torch.empty(max(lal.linattn_workspace_bytes(B, H, L, dv), 1), dtype=torch.uint8, device="cuda")
    for i in range(settle + warmup):
        lal.linattn_decay_fwd(*sets[i % nbuf], g, y=y, workspace=ws)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(steps):
        lal.linattn_decay_fwd(*sets[i % nbuf], g, y=y, workspace=ws)
    t1.record()
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) / steps * 1e3
    nbytes = lin_bytes(dv) * B * H * L
    # the decayed backward on the same inputs, a seeded dy and the forward's y
    dy = synth.upstream_grad(cfg, 0).to("cuda")
    ys = [lal.linattn_decay_fwd(*sets[i], g) for i in range(nbuf)]
    bws = torch.empty(max(1, lal.linattn_bwd_workspace_bytes(B, H, L, dv)), dtype=torch.uint8, device="cuda")
    gq = torch.empty(B, H, L, 16, device="cuda")
    gk = torch.empty_like(gq)
    gv = torch.empty(B, H, L, dv, device="cuda")
    bwd = lambda i: lal.linattn_decay_bwd(*sets[i % nbuf], g, ys[i % nbuf], dy, dq=gq, dk=gk, dv=gv, workspace=bws)
    for i in range(settle + warmup):
        bwd(i)
    bus = time_loop(bwd, steps) * 1e3
    b1 = bwd_bytes(dv) * B * H * L
    return {"workload": cfg.name + " decayed linear attention", "B": B, "H": H, "L": L, "d_v": dv,
            "us_per_call": us, "tokens_per_s": B * L / (us * 1e-6), "bytes_per_call": nbytes,
            "hbm_gbs": nbytes / (us * 1e-6) / 1e9, "hbm_frac": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "alg_tflops": lin_flops(dv) * B * H * L / (us * 1e-6) / 1e12,
            "traffic_bytes_per_call": load_traffic("decay"),
            "bwd_us_per_call": bus, "bwd_bytes_per_call": b1, "bwd_hbm_gbs": b1 / (bus * 1e-6) / 1e9}


def bench_decode(lal, cfg, warmup=5, decay=False, compact=False):
    """Prefill (untimed), then cfg.steps decode steps timed as one block
    (decay: the decayed linear attention, per-head decays from
    synth.decay_rates; same bytes per step; compact: the state with one row
    per unordered feature pair, 153 rows instead of 273)."""
    (qc, kc, vc), (qs, ks, vs) = synth.decode_inputs(cfg, 0)
    g = synth.decay_rates(cfg.H).cuda() if decay else None
    _, _, st = lal.decode_init(qc.cuda(), kc.cuda(), vc.cuda(), cfg.window, gamma=g, compact=compact)
    del qc, kc, vc
    qd, kd, vd = qs.cuda(), ks.cuda(), vs.cuda()
    B, H, dv = cfg.B, cfg.H, cfg.dv
    y_lin = torch.empty(B, H, dv, device="cuda")
    y_swa = torch.empty(B, H, dv, device="cuda")
    for s in range(warmup):  # advances the state; the timed steps continue from it
        lal.decode_step(st, qd[s], kd[s], vd[s], y_lin=y_lin, y_swa=y_swa, gamma=g)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = cfg.steps - warmup
    t0.record()
    for s in range(warmup, cfg.steps):
        lal.decode_step(st, qd[s], kd[s], vd[s], y_lin=y_lin, y_swa=y_swa, gamma=g)
    t1.record()
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) * 1e3 / n
    byts = decode_bytes(dv, cfg.window, rows=D_CMP if compact else D_PHI) * B * H
    name = "decode" + (" (decayed)" if decay else "") + (", compact state" if compact else "")
    return {
        "workload": name, "sequences": B, "heads": H, "context": cfg.ctx, "steps_timed": n,
        "us_per_step": us, "tokens_per_s": B / (us * 1e-6), "hbm_gbs": byts / (us * 1e-6) / 1e9,
        "hbm_frac": byts / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, "bytes_per_step": byts,
    }


def host_info():
    """This host's CPU model and logical CPU count, and the threads the
    oracle's BLAS calls use."""
    from threadpoolctl import threadpool_info

    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"cpu_model": model, "host_cpus": os.cpu_count(), "blas_threads": threads}


def oracle_fwd_rate(cfg, budget_s):
    """Position-heads per second of the fp64 oracle (chunked linear attention
    + banded window softmax) over whole heads of `cfg`, for about budget_s
    seconds (at least one head).  Returns (rate, heads done, seconds)."""
    from oracle import based_oracle as O

    q, k, v = synth.fwd_inputs(cfg, 0)
    heads = [(b, h) for b in range(cfg.B) for h in range(cfg.H)]
    done = 0
    t0 = time.perf_counter()
    while done < len(heads) and (done == 0 or time.perf_counter() - t0 < budget_s):
        b, h = heads[done]
        O.linattn_chunked(q[b, h], k[b, h], v[b, h], 64)
        O.swa(q[b, h], k[b, h], v[b, h], cfg.window)
        done += 1
    dt = time.perf_counter() - t0
    return done * cfg.L / dt, done, dt


def cpu_baseline(cfg, budget_s=12.0):
    """The fp64 oracle (chunked linear attention + banded window softmax) on a
    bounded sample of the step's heads, on this host's cores."""
    rate, done, dt = oracle_fwd_rate(cfg, budget_s)
    info = host_info()
    return {
        "value": rate / cfg.H, "unit": "tokens/s", "cores": info["blas_threads"], "kind": "oracle",
        "host_cpus": info["host_cpus"], "cpu_model": info["cpu_model"],
        "sample": f"{done} of {cfg.B * cfg.H} (batch, head) pairs of the step workload ({cfg.L} positions each), "
                  f"fp64 chunked linear attention + banded window softmax, {dt:.1f} s; tokens/s = "
                  f"position-heads/s / {cfg.H} heads; cores = the oracle's BLAS threads",
    }


def cpu_oracle_other(budget_s=4.0, decode_steps=3):
    """The same oracle on the other workloads, each on a bounded sample:
    whole heads of the 1.3B-shaped and 32k forwards (tokens/s = position-heads
    per second / heads), and decode: `decode_steps` steps of the full 256 x
    16-head batch (the fp64 recurrence and the window over the ring), each
    step costing the same, so tokens/s = 256 sequences per step time.  The
    decode state starts at zero with a full ring: a step's cost does not
    depend on the state's values."""
    import numpy as np

    from oracle import based_oracle as O

    out = {}
    for name in ("based1p3b", "long32k"):
        cfg = synth.FWD_CONFIGS[name]
        rate, done, dt = oracle_fwd_rate(cfg, budget_s)
        out[name] = {"tokens_per_s": rate / cfg.H, "sample": f"{done} head(s) of {cfg.L} positions, {dt:.1f} s"}
    cfg = synth.DECODE_CONFIG
    _, (qs, ks, vs) = synth.decode_inputs(cfg.replace(ctx=0, steps=decode_steps + 1), 0)
    B, H, W = cfg.B, cfg.H, cfg.window
    st = O.DecodeState(np.zeros((B, H, O.D_PHI, cfg.dv)), np.zeros((B, H, O.D_PHI)), np.zeros((B, H, W, 16)),
                       np.zeros((B, H, W, cfg.dv)), np.full(B, cfg.ctx))
    st.step(qs[0], ks[0], vs[0])  # first touch of the state arrays, untimed
    t0 = time.perf_counter()
    for s in range(1, decode_steps + 1):
        st.step(qs[s], ks[s], vs[s])
    dt = (time.perf_counter() - t0) / decode_steps
    out["decode"] = {"tokens_per_s": B / dt, "s_per_step": dt,
                     "sample": f"{decode_steps} steps of {B} sequences x {H} heads (fp64 state, zero at the "
                               f"start; a step's cost does not depend on the state's values)"}
    out.update(host_info())
    return out


def _counter_rows(d):
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    return rows


def short_name(kernel):
    """A rocprofv3 kernel name without its argument list."""
    return kernel.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")


def summarize_pmc(fetch_dir, write_dir, calls, command, out_dir=None):
    """Turn two rocprofv3 --pmc runs of this script (FETCH_SIZE, then
    WRITE_SIZE) into <out_dir>/traffic_<op>.json (default: profiles/): HBM
    bytes per call of each timed operation, scaled by the counters' reading
    for the copy calibration kernel of known size."""
    out_dir = out_dir or os.path.join(ROOT, "profiles")
    def per_dispatch(rows, counter):
        """(dispatch id, kernel name) -> bytes (summed over the counter's instances)."""
        acc = {}
        for r in rows:
            if r["Counter_Name"] != counter:
                continue
            key = (int(r["Dispatch_Id"]), r["Kernel_Name"])
            acc[key] = acc.get(key, 0.0) + float(r["Counter_Value"]) * 1024.0  # KiB -> B
        return acc

    def by_kernel(acc, lo, hi):
        out = {}
        for (i, name), val in sorted(acc.items()):
            if lo <= i <= hi:
                out.setdefault(name, []).append(val)
        return out

    fetch_all = per_dispatch(_counter_rows(fetch_dir), "FETCH_SIZE")
    write_all = per_dispatch(_counter_rows(write_dir), "WRITE_SIZE")
    everything = by_kernel(fetch_all, 0, 1 << 60)
    copy_names = [k for k in everything if "copy" in k.lower() or "elementwise" in k.lower()]
    big = [k for k in copy_names if max(everything[k]) > 0.25 * COPY_BYTES]
    if not big:
        raise SystemExit("no copy calibration kernel found in the FETCH_SIZE run")
    cname = big[0]
    # the calibration copies only (the same kernel also serves small copies)
    cf = [x for x in everything[cname] if x > 0.25 * COPY_BYTES]
    cw = [x for x in by_kernel(write_all, 0, 1 << 60)[cname] if x > 0.25 * COPY_BYTES]
    f_copy = sorted(cf)[len(cf) // 2]
    w_copy = sorted(cw)[len(cw) // 2]
    f_scale, w_scale = COPY_BYTES / f_copy, COPY_BYTES / w_copy
    # the step workload runs first; its last dispatch is the calls-th launch of the fused main pass
    # the step's launches end where the backward (run right after it, with as
    # many calls) begins; the backward's input set-up runs before the step
    bwd_ids = sorted(i for (i, n) in fetch_all if BWD_KERNEL in n)
    first_bwd = bwd_ids[0] if bwd_ids else 1 << 60
    step_end = max(i for (i, n) in fetch_all if STEP_KERNEL in n and i < first_bwd)
    bwd_end = bwd_ids[calls - 1] if len(bwd_ids) >= calls else step_end
    windows = {"layer": (0, step_end), "bwd": (step_end + 1, bwd_end), "decode": (bwd_end + 1, 1 << 60),
               "decode_compact": (bwd_end + 1, 1 << 60),
               "baseconv": (bwd_end + 1, 1 << 60), "decay": (bwd_end + 1, 1 << 60)}
    os.makedirs(out_dir, exist_ok=True)
    workloads = {"layer": "based360m", "bwd": "based360m layer backward (both attentions)",
                 "decode": "decode (256 x 16 heads)", "decode_compact": "decode, compact state (256 x 16 heads)",
                 "baseconv": "baseconv360m (8 x 2048 x 1024, 3 taps)",
                 "decay": "based360m decayed linear attention"}
    for op, frags in OP_KERNELS.items():
        tot_f = tot_w = 0.0
        detail = {}
        fetch = by_kernel(fetch_all, *windows[op])
        write = by_kernel(write_all, *windows[op])
        for name, vals in fetch.items():
            if any(fr in name for fr in frags):
                wv = write.get(name, [0.0])
                med_f = sorted(vals)[len(vals) // 2] * f_scale
                med_w = sorted(wv)[len(wv) // 2] * w_scale
                detail[short_name(name)] = {"fetch_bytes": med_f, "write_bytes": med_w, "dispatches": len(vals)}
                tot_f += med_f
                tot_w += med_w
        if not detail:
            continue
        rec = {"op": op, "workload": workloads[op], "source_hash": source_hash(op), "command": command,
               "copy_kernel": short_name(cname), "copy_fetch_factor": f_scale, "copy_write_factor": w_scale,
               "bytes_per_call": tot_f + tot_w, "fetch_bytes_per_call": tot_f, "write_bytes_per_call": tot_w,
               "kernels": detail}
        with open(os.path.join(out_dir, f"traffic_{op}.json"), "w") as fh:
            json.dump(rec, fh, indent=1)
        print(json.dumps(rec, indent=1))


# Counter passes of the execution summary (each within one rocprofv3 --pmc
# run's hardware limits: at most 8 SQ counters and 2 GRBM counters).
COUNTER_PASSES = [
    ["SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_SALU", "SQ_INSTS_VALU_TRANS_F32",
     "SQ_WAVE_CYCLES", "SQ_BUSY_CU_CYCLES", "GRBM_GUI_ACTIVE"],
    ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_LDS_BANK_CONFLICT",
     "SQ_LDS_IDX_ACTIVE", "SQ_WAIT_INST_LDS", "SQ_WAIT_ANY", "SQ_INSTS_VMEM", "GRBM_GUI_ACTIVE"],
]
CU_NUM, SIMD_NUM, NXCD = 256, 1024, 8


def summarize_counters(dirs, command, kernels, out_name, out_dir=None):
    """<out_dir>/<out_name> (default directory: profiles/) from rocprofv3
    --pmc runs of this script, one directory per pass of COUNTER_PASSES: per
    kernel whose name contains one of `kernels`, the median over its
    dispatches of every counter, and from them

      cycles          = GRBM_GUI_ACTIVE / 8 (the counter is summed over the
                        eight XCDs, each with its own clock counter)
      MFMA busy %     = SQ_VALU_MFMA_BUSY_CYCLES / (cycles * 1024 SIMDs)
      VALU busy %     = SQ_ACTIVE_INST_VALU / (cycles * 256 CUs)
      LDS active %    = SQ_LDS_IDX_ACTIVE / (cycles * 256 CUs)
      bank conflict   = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE
      waves per SIMD  = 4 * SQ_WAVE_CYCLES / (cycles * 1024 SIMDs)
                        (SQ_WAVE_CYCLES counts quad-cycles)

    (the busy formulas are rocprofv3's own MfmaUtil, VALUBusy and LdsUtil,
    with its max over XCDs taken as the sum / 8) and the instructions each
    wavefront issued."""
    vals = {}  # kernel -> counter -> [per-dispatch values]
    for d in dirs:
        per = {}
        for r in _counter_rows(d):
            name = short_name(r["Kernel_Name"])
            if not any(k in r["Kernel_Name"] for k in kernels):
                continue
            key = (int(r["Dispatch_Id"]), name, r["Counter_Name"])
            v = float(r["Counter_Value"])
            # GRBM_GUI_ACTIVE: one clock for the whole GPU (max over instances);
            # SQ counters: summed over shader engines
            per[key] = max(per.get(key, 0.0), v) if r["Counter_Name"] == "GRBM_GUI_ACTIVE" else per.get(key, 0.0) + v
        for (_, name, cn), v in per.items():
            vals.setdefault(name, {}).setdefault((d, cn), []).append(v)
    lines = ["# Execution counters (rocprofv3 --pmc)", "", f"Command: `{command}`", "",
             "Median per dispatch over every dispatch of the kernel in the run. Derived figures, with",
             "cycles = GRBM_GUI_ACTIVE / 8 (summed over the 8 XCDs' clock counters): MFMA busy =",
             "SQ_VALU_MFMA_BUSY_CYCLES / (cycles x 1024 SIMDs); VALU busy = SQ_ACTIVE_INST_VALU /",
             "(cycles x 256 CUs); LDS active = SQ_LDS_IDX_ACTIVE / (cycles x 256 CUs); bank conflict =",
             "SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE; waves/SIMD = 4 x SQ_WAVE_CYCLES / (cycles x 1024",
             "SIMDs); per-wave instruction counts = SQ_INSTS_* / SQ_WAVES.", "",
             "| kernel | dispatches | cycles | MFMA busy % | VALU busy % | LDS active % | bank conflict | "
             "waves/SIMD | VALU/wave | MFMA/wave | LDS/wave | SALU/wave | trans/wave | VMEM/wave |",
             "|---|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    out_json = {}

    def med(xs):
        xs = sorted(xs)
        return xs[len(xs) // 2] if xs else float("nan")

    def ratio(a, b):
        return a / b if b else float("nan")  # (a kernel without LDS reads no LDS cycles)

    for name, cs in sorted(vals.items()):
        m = {}
        for (d, cn), xs in cs.items():
            m[cn if cn != "GRBM_GUI_ACTIVE" else f"GRBM_GUI_ACTIVE@{dirs.index(d)}"] = med(xs)
        n = max(len(xs) for xs in cs.values())
        gui0 = m.get("GRBM_GUI_ACTIVE@0", float("nan")) / NXCD
        gui1 = m.get("GRBM_GUI_ACTIVE@1", float("nan")) / NXCD
        waves = m.get("SQ_WAVES", float("nan"))
        row = {
            "dispatches": n, "gpu_cycles": gui1,
            "mfma_busy_pct": 100 * ratio(m.get("SQ_VALU_MFMA_BUSY_CYCLES", float("nan")), gui1 * SIMD_NUM),
            "valu_busy_pct": 100 * ratio(m.get("SQ_ACTIVE_INST_VALU", float("nan")), gui1 * CU_NUM),
            "lds_active_pct": 100 * ratio(m.get("SQ_LDS_IDX_ACTIVE", float("nan")), gui1 * CU_NUM),
            "bank_conflict": ratio(m.get("SQ_LDS_BANK_CONFLICT", float("nan")), m.get("SQ_LDS_IDX_ACTIVE", float("nan"))),
            "waves_per_simd": 4 * ratio(m.get("SQ_WAVE_CYCLES", float("nan")), gui0 * SIMD_NUM),
            "valu_per_wave": ratio(m.get("SQ_INSTS_VALU", float("nan")), waves),
            "mfma_per_wave": ratio(m.get("SQ_INSTS_MFMA", float("nan")), waves),
            "lds_per_wave": ratio(m.get("SQ_INSTS_LDS", float("nan")), waves),
            "salu_per_wave": ratio(m.get("SQ_INSTS_SALU", float("nan")), waves),
            "trans_per_wave": ratio(m.get("SQ_INSTS_VALU_TRANS_F32", float("nan")), waves),
            "vmem_per_wave": ratio(m.get("SQ_INSTS_VMEM", float("nan")), waves),
            "raw": m,
        }
        out_json[name] = row
        lines.append(f"| `{name}` | {n} | {gui1:.0f} | {row['mfma_busy_pct']:.1f} | {row['valu_busy_pct']:.1f} | "
                     f"{row['lds_active_pct']:.1f} | {row['bank_conflict']:.3f} | {row['waves_per_simd']:.2f} | "
                     f"{row['valu_per_wave']:.0f} | {row['mfma_per_wave']:.0f} | {row['lds_per_wave']:.0f} | "
                     f"{row['salu_per_wave']:.0f} | {row['trans_per_wave']:.0f} | {row['vmem_per_wave']:.0f} |")
    out_dir = out_dir or os.path.join(ROOT, "profiles")
    os.makedirs(out_dir, exist_ok=True)
    with open(os.path.join(out_dir, out_name), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))
    return out_json


def summarize_stats(stats_dir, command, calls, out_dir=None):
    """<out_dir>/kernel_stats.md (default: profiles/) from a rocprofv3
    --kernel-trace --stats run of this script: average duration of every kernel.  The step workload runs
    first and ends with its `calls`-th launch of the fused main pass; its
    dispatches are reported apart from the rest."""
    files = glob.glob(os.path.join(stats_dir, "**", "*kernel_trace.csv"), recursive=True)
    rows = []
    for f in files:
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    bwd_starts = [int(r["Start_Timestamp"]) for r in rows if BWD_KERNEL in r["Kernel_Name"]]
    first_bwd = bwd_starts[0] if bwd_starts else 1 << 62
    step_starts = [int(r["Start_Timestamp"]) for r in rows
                   if STEP_KERNEL in r["Kernel_Name"] and int(r["Start_Timestamp"]) < first_bwd]
    step_end = step_starts[-1] if step_starts else -1
    bwd_end = bwd_starts[calls - 1] if len(bwd_starts) >= calls else step_end
    groups = {}
    for r in rows:
        name = short_name(r["Kernel_Name"])
        grid = r["Grid_Size_X"] if "Grid_Size_X" in r else r["Grid_Size"]
        blk = r["Workgroup_Size_X"] if "Workgroup_Size_X" in r else r["Workgroup_Size"]
        t = int(r["Start_Timestamp"])
        phase = ""
        if t <= step_end and any(fr in name for fr in OP_KERNELS["layer"]):
            phase = "step"
        elif step_end < t <= bwd_end and any(fr in name for fr in OP_KERNELS["bwd"]):
            phase = "bwd"
        groups.setdefault((name, grid, blk, phase), []).append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines = ["# Kernel durations (rocprofv3 --kernel-trace --stats)", "", f"Command: `{command}`", "",
             "Rows marked *step* are the timed layer step (360M-shaped workload, B8 H16 L2048 d_v64 bf16),",
             "rows marked *bwd* the layer backward on the same workload (both attentions' gradients);",
             "the others are set-up, the separate-call comparison, the 1.3B-shaped and 32k workloads, the",
             "BaseConv gate, the decayed linear attention and the decode loop.", "",
             "| kernel | grid (threads) | block | step | calls | avg us | min us | max us |",
             "|---|---|---|---|---|---|---|---|"]
    for (name, grid, blk, phase), d in groups.items():
        lines.append(f"| `{name}` | {grid} | {blk} | {phase} | {len(d)} | {sum(d) / len(d):.1f} | {min(d):.1f} | "
                     f"{max(d):.1f} |")
    out_dir = out_dir or os.path.join(ROOT, "profiles")
    os.makedirs(out_dir, exist_ok=True)
    out = os.path.join(out_dir, "kernel_stats.md")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=200,
                    help="untimed steps first (enough for the GPU clocks to settle)")
    ap.add_argument("--settle", type=int, default=300,
                    help="untimed calls of each timed operation before its warm-up calls, so that the GPU clocks "
                         "settle")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extra", action="store_true", help="skip the other workloads and decode")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/traffic_<op>.json from two rocprofv3 --pmc runs of this script")
    ap.add_argument("--pmc-command", default="", help="the command that produced the --pmc runs (recorded)")
    ap.add_argument("--summarize-stats", metavar="STATS_DIR",
                    help="write profiles/kernel_stats.md from a rocprofv3 --kernel-trace --stats run of this script")
    ap.add_argument("--summarize-counters", nargs="+", metavar="PASS_DIR",
                    help="write profiles/<--counters-out> from rocprofv3 --pmc runs of this script, one directory "
                         "per pass of COUNTER_PASSES, in that order")
    ap.add_argument("--counters-out", default="counters_layer.md")
    ap.add_argument("--counter-kernels", default="based::",
                    help="semicolon-separated kernel-name fragments to summarise")
    ap.add_argument("--print-counter-pass", type=int, metavar="I",
                    help="print the counters of pass I (for rocprofv3 --pmc) and exit")
    args = ap.parse_args()
    if args.print_counter_pass is not None:
        print(" ".join(COUNTER_PASSES[args.print_counter_pass]))
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.pmc_command, args.counter_kernels.split(";"),
                           args.counters_out)
        return
    if args.summarize_stats:
        summarize_stats(args.summarize_stats, args.pmc_command, args.steps + args.warmup)
        return
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.steps + args.warmup, args.pmc_command)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(batch/head sharding of the layer needs no communication; see DESIGN.md)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    import linear_attention_lm_amd as lal

    cfg = synth.FWD_CONFIGS["based360m"]
    copy = copy_calibration()
    print(f"[bench] copy calibration: {copy['gbs']:.0f} GB/s", file=sys.stderr, flush=True)
    bsets = None if args.no_extra else bwd_inputs(lal, cfg)
    main_res = bench_fwd(lal, cfg, args.steps, args.warmup, settle=args.settle, check=True)
    print(f"[bench] {cfg.name}: {main_res['ms_per_step'] * 1e3:.1f} us/step (layer {main_res['layer_us']:.1f} us)",
          file=sys.stderr, flush=True)
    extra, decode, separate, backward, conv, decay, decode_decay = [], None, None, None, None, None, None
    decode_compact = tiny = cpu_other = None
    if not args.no_extra:
        tiny = bench_tiny(lal, synth.FWD_CONFIGS["tiny"])
        print(f"[bench] tiny fp32 layer: {tiny['us_per_call_back_to_back']:.1f} us/call back to back, "
              f"{tiny['us_latency_median']:.1f} us latency", file=sys.stderr, flush=True)
        backward = bench_bwd(lal, cfg, args.steps, args.warmup, bsets, settle=args.settle)
        del bsets
        print(f"[bench] {cfg.name} backward: linattn {backward['linattn_bwd_us']:.1f} us, swa "
              f"{backward['swa_bwd_us']:.1f} us", file=sys.stderr, flush=True)
        separate = bench_fwd(lal, cfg, max(10, args.steps // 2), args.warmup, fused=False, settle=args.settle)
        print(f"[bench] {cfg.name} separate calls: linattn {separate['linattn_us']:.1f} us, swa "
              f"{separate['swa_us']:.1f} us", file=sys.stderr, flush=True)
        for name in ("based1p3b", "long32k"):
            r = bench_fwd(lal, synth.FWD_CONFIGS[name], max(10, args.steps // 2), args.warmup, nbuf=4,
                          settle=args.settle)
            extra.append(r)
            print(f"[bench] {name}: {r['ms_per_step'] * 1e3:.1f} us/step", file=sys.stderr, flush=True)
        conv = bench_baseconv(lal, synth.CONV_CONFIGS["baseconv360m"], args.steps, args.warmup, settle=args.settle)
        print(f"[bench] baseconv: {conv['us_per_call']:.1f} us/call ({conv['hbm_gbs']:.0f} GB/s)", file=sys.stderr,
              flush=True)
        decay = bench_decay(lal, cfg, args.steps, args.warmup, settle=args.settle)
        print(f"[bench] {cfg.name} decayed linear attention: {decay['us_per_call']:.1f} us/call "
              f"({decay['hbm_gbs']:.0f} GB/s), backward {decay['bwd_us_per_call']:.1f} us/call", file=sys.stderr,
              flush=True)
        decode = bench_decode(lal, synth.DECODE_CONFIG)
        decode["traffic_bytes_per_step"] = load_traffic("decode")
        print(f"[bench] decode: {decode['us_per_step']:.1f} us/step", file=sys.stderr, flush=True)
        decode_decay = bench_decode(lal, synth.DECODE_CONFIG, decay=True)
        print(f"[bench] decode (decayed): {decode_decay['us_per_step']:.1f} us/step", file=sys.stderr, flush=True)
        decode_compact = bench_decode(lal, synth.DECODE_CONFIG, compact=True)
        decode_compact["traffic_bytes_per_step"] = load_traffic("decode_compact")
        print(f"[bench] decode (compact state): {decode_compact['us_per_step']:.1f} us/step", file=sys.stderr,
              flush=True)
    cpu = None if args.no_cpu else cpu_baseline(cfg)
    if not args.no_cpu and not args.no_extra:
        cpu_other = cpu_oracle_other()

    # the step is one operation (state-only pass + segment scan + fused main pass)
    achieved = main_res["layer_hbm_gbs"]
    out = {
        "metric": METRIC, "value": main_res["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": main_res["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) q,k,v; no trained weights)",
        "config": {"workload": "based360m layer fwd: linear attention + window-64 softmax attention, one fused pass",
                   "B": cfg.B, "H": cfg.H, "L": cfg.L, "d_k": 16, "d_v": cfg.dv, "window": cfg.window,
                   "inputs": "bf16", "outputs": "fp32"},
        "roofline": {"kernel": "layer", "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": load_traffic("layer"),
                     "alg_bytes": main_res["layer_bytes"],
                     "mfma_alg_frac": main_res["layer_alg_tflops"] / MFMA_BF16_PEAK_TFS},
        "kernels": {"layer_us": main_res["layer_us"], "layer_hbm_gbs": main_res["layer_hbm_gbs"],
                    "layer_alg_tflops": main_res["layer_alg_tflops"]},
        "separate_calls": separate,
        "backward": backward,
        "baseconv": conv,
        "decay": decay,
        "copy_calibration": copy,
        "cpu_baseline": cpu,
        "cpu_oracle_other_workloads": cpu_other,
        "tiny_layer_latency": tiny,
        "step_parity": main_res.get("parity"),
        "other_workloads": extra,
        "decode": decode,
        "decode_decay": decode_decay,
        "decode_compact": decode_compact,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
