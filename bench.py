#!/usr/bin/env python3
"""Benchmark of the chunk-wise forward of the generalized linear-attention recurrence.

One step = one full chunk-wise forward (chunk operators, then the ordered scan
that produces the outputs and the final state) over one batch of seeded
synthetic input already resident in HBM.  The decay operands A, B are built
by the device parameter kernel before the timed region (they are inputs of
the forward call).  Prints ONE JSON line (rank 0):

  value       whole-job forward tokens/s (tokens = batch x sequence positions)
  roofline    the dominant kernel, measured with HIP events on its stream
  cpu_baseline  the fp64 oracle on a bounded sample of the same workload

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import workloads  # noqa: E402

METRIC = "fwd tokens/sec + % bf16 MFMA peak, rank-2 HDLA B8 H16 T4096 d128"
PEAK = {  # MI355X published peaks
    "hbm_GBs": 8000.0,
    "bf16_mfma_TFs": 2500.0,
    "fp32_mfma_TFs": 157.3,
    # fp32 vector without packed-fp32 issue: 256 CU x 4 SIMD x 16 lanes x 2 flop x 2.4 GHz
    "fp32_valu_TFs": 78.6,
}
KERNEL_SOURCES = {
    "general_fp32": ["structured_decay_sequence_amd/csrc/general.hip"],
    "mfma_bf16": ["structured_decay_sequence_amd/csrc/fast.hip"],
}


def canonical_work(spec):
    """Algorithmic flops and bytes of one forward (per-chunk-head MAC formulas of the
    three stages: chunk summary, inter-chunk scan, output; inputs + outputs once)."""
    C, dk, dv = spec.chunk, spec.dk, spec.dv
    na, nk = C * spec.r_ab, C * spec.r_kv
    mac_a = (2 * na * na * dk + na * nk * dk + na ** 3 / 6 + na * nk * dv + na * na * dv + na * dk * dk
             + nk * dk * dv + na * dk * dv)
    mac_b = dk * dk * dv
    mac_c = 2 * C * na * dk + C * nk * dk + C * dk * dv + C * nk * dv + C * na * dv
    BH = spec.B * spec.H
    N = -(-spec.T // C)
    flops = 2.0 * (mac_a + mac_b + mac_c) * BH * N
    e = 2 if spec.dtype == "bf16" else 4
    dec = 4 if spec.scalar_decay else 4 * dk
    per_tok = e * (dk + spec.r_kv * dk + spec.r_kv * dv + 2 * spec.r_ab * dk + dv) + dec
    nbytes = per_tok * BH * spec.T + BH * dk * dv * 4
    return flops, nbytes


def kernel_work(spec, kernels):
    """Per-launch algorithmic work of each kernel of the two-stage decomposition,
    on the canonical per-token-head byte count (the inputs read once, the
    outputs written once) split by which kernel reads or writes each tensor:

    prepare: reads q, K, A, B and the log-decay;
    scan:    reads V, writes out and the final state.

    The chunk operator M_j that the prepare hands to the scan is not an
    algorithmic byte (the method does not need it in memory); its round trip
    shows up in the counter traffic, reported beside.  flops: the multiply-adds
    each kernel's decomposition performs (masked and triangular products at
    dense size, the triangular inverse at n^3/6)."""
    C, dk, dv = spec.chunk, spec.dk, spec.dv
    na, nk = C * spec.r_ab, C * spec.r_kv
    BH = spec.B * spec.H
    N = -(-spec.T // C)
    e = 2 if spec.dtype == "bf16" else 4
    dec = 4 if spec.scalar_decay else 4 * dk
    prep_in = (e * (dk + spec.r_kv * dk + 2 * spec.r_ab * dk) + dec) * BH * spec.T
    scan_bytes = e * (spec.r_kv * dv + dv) * BH * spec.T + 4 * BH * dk * dv
    prep_mac = ((na + C) * (na + nk) * dk + na ** 3 / 6 + na * na * (dk + nk) + (C + dk) * na * (dk + nk))
    scan_mac = (dk + C) * (dk + nk) * dv
    return {
        "prepare": dict(flops=2.0 * prep_mac * BH * N, bytes=float(prep_in)),
        "scan": dict(flops=2.0 * scan_mac * BH * N, bytes=float(scan_bytes)),
    }


def operator_bytes(spec, kernels):
    """Bytes of the chunk operators one forward writes (and the scan reads back)."""
    C, dk = spec.chunk, spec.dk
    em = 4 if kernels == "general_fp32" else (2 if spec.dtype == "bf16" else 4)
    N = -(-spec.T // C)
    return float(em * (dk + C) * (dk + C * spec.r_kv) * spec.B * spec.H * N)


def kernel_peak(kernels, dtype, bound):
    if bound == "hbm":
        return PEAK["hbm_GBs"], "GB/s"
    # The bf16 path multiplies on bf16 MFMAs; the general path keeps fp32
    # operands and multiplies on fp32 MFMAs (whatever the storage dtype).
    if kernels == "general_fp32":
        return PEAK["fp32_mfma_TFs"], "TFLOP/s"
    return PEAK["bf16_mfma_TFs"], "TFLOP/s"


def _code_tokens(text):
    """Source text without comments and with whitespace collapsed, so that an
    edit of comments or layout alone leaves the hash (and the counters keyed
    on it) valid."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_hash(kernels):
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES.get(kernels, []) + ["structured_decay_sequence_amd/csrc/common.hpp"]:
        path = os.path.join(ROOT, rel)
        if os.path.exists(path):
            h.update(_code_tokens(open(path).read()).encode())
    return h.hexdigest()[:16]


def _counter_record(kernels, kernel, workload):
    """The committed PMC record of a kernel, if it was taken on the current kernel
    source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(f"{kernels}:{kernel}:{workload}")
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha") != source_hash(kernels):
        return None
    return rec


def measured_traffic(kernels, kernel, workload):
    """HBM bytes per launch (scaled FETCH_SIZE + WRITE_SIZE) from the committed PMC summary."""
    rec = _counter_record(kernels, kernel, workload)
    return None if rec is None else rec.get("bytes_per_launch")


def measured_mfma(kernels, kernel, workload):
    """Executed MFMA flops and MFMA-busy fraction per launch from the committed PMC summary."""
    rec = _counter_record(kernels, kernel, workload)
    return None if rec is None else rec.get("mfma")


def build_inputs(spec, torch, lattn, dev):
    """Host-generated seeded inputs -> device; decay operands built on the device."""
    raw = workloads.raw_for(spec)
    td = torch.bfloat16 if spec.dtype == "bf16" else torch.float32
    t = lambda x, d=td: torch.from_numpy(np.ascontiguousarray(x)).to(d).to(dev)
    q = t(raw["q"])
    if spec.family == "hdla":
        k, v = t(raw["k"]), t(raw["v"])
        ld = t(raw["log_lambda"], torch.float32)
        A, B, V = lattn.hdla_params(k, v, ld, t(raw["beta"], torch.float32))
        K = k
    elif spec.family == "gdn":
        k, v = t(raw["k"]), t(raw["v"])
        ld = t(raw["g"], torch.float32)
        A, B, V = lattn.gdn_params(k, v, ld, t(raw["beta"], torch.float32))
        K = k
    else:
        K, V = t(raw["K"]), t(raw["V"])
        ld = t(raw["log_decay"], torch.float32)
        A = None if raw["A"] is None else t(raw["A"])
        B = None if raw["B"] is None else t(raw["B"])
    torch.cuda.synchronize(dev)
    return raw, (q, K, V, ld, A, B)


def fused_leg(spec, draw, torch, lattn, dev, steps, warmup):
    """The same workload through the fused family entry point (decay operands
    formed inside the chunk kernel from the raw parameters; nothing excluded
    from the timed region), timed the same way.  ``draw``: device tensors."""
    decay = draw["log_lambda"] if spec.family == "hdla" else draw["g"]
    plan = lattn.FamilyPlan(spec.family, draw["q"], draw["k"], draw["v"], decay, draw["beta"], chunk=spec.chunk)
    for _ in range(warmup):
        plan.forward()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(dev)
    e0.record(stream)
    for _ in range(steps):
        plan.forward()
    e1.record(stream)
    torch.cuda.synchronize(dev)
    ms = e0.elapsed_time(e1) / steps
    flops, _ = canonical_work(spec)
    nbytes = fused_bytes(spec)
    return {
        "entry": f"lattn_{spec.family}_chunk_fwd",
        "ms_per_step": round(ms, 4),
        "value": round(spec.B * spec.T / (ms / 1e3), 1),
        "unit": "tokens/s",
        "mfma_frac_canonical": round(flops / (ms / 1e3) / (PEAK["bf16_mfma_TFs"] * 1e12), 4),
        "algorithmic_gb": round(nbytes / 1e9, 4),
        "hbm_frac_algorithmic": round(nbytes / (ms / 1e3) / (PEAK["hbm_GBs"] * 1e9), 4),
    }


def fused_bytes(spec):
    """Inputs + outputs of the fused family forward: q, k, v, the log-decay and
    beta in, out and the final state out."""
    e = 2 if spec.dtype == "bf16" else 4
    dec = 4 if spec.scalar_decay else 4 * spec.dk
    per_tok = e * (2 * spec.dk + 2 * spec.dv) + dec + 4
    return float(per_tok * spec.B * spec.H * spec.T + spec.B * spec.H * spec.dk * spec.dv * 4)


# Query-conditioned composition (HLA note, "Method steps"): Gated DeltaNet, the
# family the note builds on, at B=1, H=16, T=4096, d_k = d_v = 128, bf16 storage;
# gating chunks of 256 tokens (the note's length), each summarised from four
# 64-token chunk operators; gates sigmoid(N(-4, 1.5)) with the note's threshold 0.1.
HLA_WORKLOAD = dict(B=1, H=16, T=4096, dk=128, dv=128, chunk=256, mu=-4.0, theta=0.1)


def hla_leg(torch, lattn, dev, steps, warmup):
    """lattn_hla_fwd on the HLA workload, timed with HIP events on its stream.
    The decay operands come from the device parameter kernel before timing (as
    for the generic forward).  flops: the pair products (one C x d_k x (d_k + d_v)
    product per (query chunk, earlier chunk) pair with a gate at or above the
    threshold) plus the chunk operators and chunk writes."""
    w = HLA_WORKLOAD
    Bb, H, T, dk, dv, C = w["B"], w["H"], w["T"], w["dk"], w["dv"], w["chunk"]
    raw = workloads.gdn_raw(Bb, H, T, dk, dv, "bf16", seed=0)
    gates = workloads.hla_gates(Bb, H, T, C, mu=w["mu"], seed=0)
    t = lambda x, d: torch.from_numpy(np.ascontiguousarray(x)).to(d).to(dev)
    q, k, v = (t(raw[n], torch.bfloat16) for n in ("q", "k", "v"))
    A, B, V = lattn.gdn_params(k, v, t(raw["g"], torch.float32), t(raw["beta"], torch.float32))
    ld = t(raw["g"], torch.float32)
    gt = t(gates, torch.float32)
    out = torch.empty((Bb, H, T, dv), dtype=torch.bfloat16, device=dev)
    run = lambda: lattn.hla_fwd(q, k, V, ld, A, B, gt, chunk=C, theta=w["theta"], out=out)
    for _ in range(warmup):
        run()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(dev)
    e0.record(stream)
    for _ in range(steps):
        run()
    e1.record(stream)
    torch.cuda.synchronize(dev)
    ms = e0.elapsed_time(e1) / steps
    N = -(-T // C)
    act = gates.reshape(Bb * H, N, C, N) >= w["theta"]          # [head, query chunk, query, chunk]
    pairs = sum(int(act[:, c, :, :c].any(axis=1).sum()) for c in range(N))
    # the pair products, the 64-token chunk operators and the gating-chunk
    # summaries (scan products over d_k + d_v columns)
    c64 = 64
    n64 = -(-T // c64)
    na, nk = c64, c64
    pair_mac = C * dk * (dk + dv)
    prep_mac = (na + c64) * (na + nk) * dk + na ** 3 / 6 + na * na * (dk + nk) + (c64 + dk) * na * (dk + nk)
    gate_mac = (dk + c64) * (dk + nk) * (dk + dv)
    flops = 2.0 * (pairs * pair_mac + Bb * H * n64 * (prep_mac + gate_mac))
    return {
        "entry": "lattn_hla_fwd",
        "workload": f"gdn B{Bb} H{H} T{T} d{dk} C{C} bf16, gates sigmoid(N({w['mu']}, 1.5)), theta {w['theta']}",
        "ms_per_step": round(ms, 4),
        "value": round(Bb * T / (ms / 1e3), 1),
        "unit": "tokens/s",
        "active_pairs": pairs,
        "all_pairs": Bb * H * N * (N - 1) // 2,
        "gflop": round(flops / 1e9, 2),
        "pair_gflop": round(2.0 * pairs * pair_mac / 1e9, 2),
        # on this bf16 workload every product (chunk operators, gating-chunk
        # summaries, the pair products) runs on bf16 MFMAs
        "mfma_frac_bf16": round(flops / (ms / 1e3) / (PEAK["bf16_mfma_TFs"] * 1e12), 4),
    }


# Log-linear lift (Log-Linear note, "Key design"; its throughput runs use 48
# heads of dimension 64 at 8K-32K tokens): Gated DeltaNet B=1, H=48, T=32768,
# d_k = d_v = 64, chunks of 64, bf16 storage, level weights softplus(N(0, 1)).
LOGLINEAR_WORKLOAD = dict(B=1, H=48, T=32768, dk=64, dv=64, chunk=64)


def loglinear_leg(torch, lattn, dev, steps, warmup):
    """lattn_loglinear_fwd on the log-linear workload, timed with HIP events on its
    stream (decay operands from the device parameter kernel before timing).
    flops: the chunk operators, the weighted chunk-local products and, per chunk
    and inter-chunk level, the state transport (d_k rows) and, where the level is
    read, the output rows."""
    w = LOGLINEAR_WORKLOAD
    Bb, H, T, dk, dv, C = w["B"], w["H"], w["T"], w["dk"], w["dv"], w["chunk"]
    raw = workloads.gdn_raw(Bb, H, T, dk, dv, "bf16", seed=0)
    lam = workloads.loglinear_lambdas(Bb, H, T, seed=0)
    t = lambda x, d: torch.from_numpy(np.ascontiguousarray(x)).to(d).to(dev)
    q, k, v = (t(raw[n], torch.bfloat16) for n in ("q", "k", "v"))
    A, B, V = lattn.gdn_params(k, v, t(raw["g"], torch.float32), t(raw["beta"], torch.float32))
    ld = t(raw["g"], torch.float32)
    lt = t(lam, torch.float32)
    out = torch.empty((Bb, H, T, dv), dtype=torch.bfloat16, device=dev)
    run = lambda: lattn.loglinear_fwd(q, k, V, ld, A, B, lt, chunk=C, out=out)
    for _ in range(warmup):
        run()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(dev)
    e0.record(stream)
    for _ in range(steps):
        run()
    e1.record(stream)
    torch.cuda.synchronize(dev)
    ms = e0.elapsed_time(e1) / steps
    N = -(-T // C)
    nlev = int(N - 1).bit_length()
    na, nk = C, C
    prep_mac = (na + C) * (na + nk) * dk + na ** 3 / 6 + na * na * (dk + nk) + (C + dk) * na * (dk + nk)
    intra_mac = (dk + C) * nk * dv
    scan_mac = 0
    for J in range(N):
        for m in range(nlev):
            if (J >> m) & 1:
                scan_mac += (dk + C) * dk * dv
            elif J % (2 << m):
                scan_mac += dk * dk * dv
    flops = 2.0 * Bb * H * (N * (prep_mac + intra_mac) + scan_mac)
    # At this shape the whole call runs on bf16 MFMAs: the prepare, then the level
    # scan on its bf16 operators; the flops are priced against the bf16 peak over
    # the whole call's time.
    return {
        "entry": "lattn_loglinear_fwd",
        "workload": f"gdn B{Bb} H{H} T{T} d{dk} C{C} bf16, {lattn.loglinear_levels(T)} levels, weights softplus(N(0,1))",
        "ms_per_step": round(ms, 4),
        "value": round(Bb * T / (ms / 1e3), 1),
        "unit": "tokens/s",
        "gflop": round(flops / 1e9, 2),
        "mfma_frac_bf16": round(flops / (ms / 1e3) / (PEAK["bf16_mfma_TFs"] * 1e12), 4),
    }


def backward_flops(spec):
    """Dense-size flops of the chunked backward on MFMAs (bf16 storage, C = 64,
    r_kv = 1): the prepare's chunk operators, the two boundary scans, the
    blocks of L, the two right-hand sides and solves, and the five gradient
    products (each A W0 plus the masked score products, counted dense)."""
    C, dk, dv = spec.chunk, spec.dk, spec.dv
    na, nk = C * spec.r_ab, C
    n_chunks = spec.B * spec.H * -(-spec.T // C)
    prep = (na + C) * (na + nk) * dk + na ** 3 / 6 + na * na * (dk + nk) + (C + dk) * na * (dk + nk)
    scans = (dk + C) * dv * (dk + nk) + dk * dv * (dk + C)
    tri = 2 * na * na * dk
    rhs = 2 * (na * dv * dk + na * C * dk + na * dv * C)
    solve = 2 * (na * na / 2) * dv
    g_tok = lambda kw, nw: C * nw * kw + C * C * kw + C * nw * C + C * na * kw + C * nw * na   # dQ, dK, dV
    g_rank = lambda kw, nw: na * nw * kw + na * C * kw + na * nw * C + na * na * kw + na * nw * na   # dA, dB
    grads = 2 * g_tok(dv, dk) + g_tok(dk, dv) + (2 * g_rank(dv, dk) if spec.r_ab else 0)
    return 2.0 * n_chunks * (prep + scans + tri + rhs + solve + grads)


def backward_bytes(spec):
    """Algorithmic bytes of lattn_chunk_bwd: the forward's inputs, the output
    cotangents and the final-state cotangent read once; the gradients (fp32:
    q, k, v, the log-decay, A, B and the initial state) written once.  What
    the kernels hand each other (boundary states and cotangents, the scaled
    operands, the solved rank rows) is not counted."""
    e = 2 if spec.dtype == "bf16" else 4
    dk, dv = spec.dk, spec.dv
    dec = 1 if spec.scalar_decay else dk
    rd = e * (dk + spec.r_kv * dk + spec.r_kv * dv + 2 * spec.r_ab * dk + dv) + 4 * dec
    wr = 4 * (dk + spec.r_kv * dk + spec.r_kv * dv + 2 * spec.r_ab * dk + dec)
    BH = spec.B * spec.H
    return float((rd + wr) * BH * spec.T + 2 * 4 * BH * dk * dv)


def backward_leg(spec, raw, inputs, torch, lattn, dev):
    """lattn_chunk_bwd on the benchmark workload (same inputs as the forward,
    seeded output cotangents and a final-state cotangent), through a TrainPlan
    (gradients, workspace and the saved buffer allocated once, as the forward's
    ChunkPlan does): one warm-up call, then the mean of three timed calls, HIP
    events on the stream.  At this shape it is the chunked backward on bf16
    MFMAs: the chunk operators, the boundary scans (states forward, cotangents
    in reverse), then per chunk the forward and adjoint UT solves and the
    gradient products; flops are their dense-size count (backward_flops),
    priced against the bf16 MFMA peak.  The training pair is timed the same way
    on the same plan."""
    q, K, V, ld, A, B = inputs
    td = q.dtype
    rng = np.random.default_rng(1)
    dout = torch.from_numpy(rng.standard_normal((spec.B, spec.H, spec.T, spec.dv), dtype=np.float32)).to(td).to(dev)
    dfin = torch.from_numpy(rng.standard_normal((spec.B, spec.H, spec.dk, spec.dv), dtype=np.float32)).to(dev)
    plan = lattn.TrainPlan(q, K, V, ld, A, B, dout, chunk=spec.chunk, dfinal=dfin)
    stream = torch.cuda.current_stream(dev)

    def timed(fn, reps=3):
        fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize(dev)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize(dev)
        return a.elapsed_time(b) / reps
    ms = timed(plan.backward)
    flops = backward_flops(spec)
    nbytes = backward_bytes(spec)
    # The training pair: the forward that keeps the chunk operators, the
    # decay-scaled operands and the boundary states, and the backward that
    # reads them instead of forming them again (same inputs, same cotangents).
    fwd_ms = timed(plan.forward_train)
    bwd_ms = timed(plan.backward_saved)
    del plan
    return {
        "entry": "lattn_chunk_bwd",
        "kind": "chunked backward on bf16 MFMAs: boundary scans, forward and adjoint UT solves, gradient products",
        "ms_per_step": round(ms, 3),
        "value": round(spec.B * spec.T / (ms / 1e3), 1),
        "unit": "tokens/s",
        "gflop": round(flops / 1e9, 2),
        "mfma_frac_bf16": round(flops / (ms / 1e3) / (PEAK["bf16_mfma_TFs"] * 1e12), 4),
        "algorithmic_gb": round(nbytes / 1e9, 4),
        "hbm_frac_algorithmic": round(nbytes / (ms / 1e3) / (PEAK["hbm_GBs"] * 1e9), 4),
        "ratio_to_forward": None,
        "training_pair": {
            "entries": "lattn_chunk_fwd_train + lattn_chunk_bwd_saved",
            "fwd_train_ms": round(fwd_ms, 3),
            "bwd_saved_ms": round(bwd_ms, 3),
            "step_ms": round(fwd_ms + bwd_ms, 3),
            "fwd_plus_bwd_ms": None,
        },
    }


def decode_leg(spec, torch, lattn, dev, steps, warmup):
    """lattn_step (one recurrent token per (batch, head)) at the workload's
    shape.  The step is memory-bound: its roofline is the fp32 state read and
    written once per token plus the token's vectors.  The state rotates over
    enough distinct buffers that their sum exceeds the 256 MB MALL, so every
    step reads the state from HBM.  One step per buffer is captured into a
    graph, so the timing (HIP events around graph replays, on the stream the
    steps run on) holds the kernels and not the host's launch rate; the
    eagerly launched rate is reported beside it."""
    Bb, H, dk, dv = spec.B, spec.H, spec.dk, spec.dv
    state_bytes = Bb * H * dk * dv * 4
    nstates = max(2, -(-(384 << 20) // state_bytes))
    draw = workloads.device_raw(workloads.Spec(spec.name, spec.family, Bb, H, 1, dk, dv, spec.chunk, spec.r_ab,
                                               spec.r_kv, spec.dtype, spec.lam_mu), torch, dev, seed=1)
    q, K, V, ld, A, B = (x[:, :, 0].contiguous() if x is not None else None for x in generic_inputs(spec, draw, lattn))
    states = [torch.zeros((Bb, H, dk, dv), dtype=torch.float32, device=dev) for _ in range(nstates)]
    out = torch.empty((Bb, H, dv), dtype=q.dtype, device=dev)
    run_all = lambda: [lattn.step(q, K, V, ld, A, B, st, out=out) for st in states]
    for _ in range(max(1, warmup // nstates + 1)):
        run_all()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(dev)
    e0.record(stream)
    run_all()
    e1.record(stream)
    torch.cuda.synchronize(dev)
    us_eager = e0.elapsed_time(e1) * 1e3 / nstates
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream(dev)
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        run_all()
    stream.wait_stream(side)
    torch.cuda.synchronize(dev)
    with torch.cuda.graph(graph):
        run_all()
    reps = max(2, steps // nstates)
    graph.replay()
    torch.cuda.synchronize(dev)
    e0.record(stream)
    for _ in range(reps):
        graph.replay()
    e1.record(stream)
    torch.cuda.synchronize(dev)
    us = e0.elapsed_time(e1) * 1e3 / (reps * nstates)
    e = 2 if spec.dtype == "bf16" else 4
    dec = 4 if spec.scalar_decay else 4 * dk
    tok_bytes = e * (dk + spec.r_kv * (dk + dv) + 2 * spec.r_ab * dk + dv) + dec
    nbytes = 2 * state_bytes + Bb * H * tok_bytes
    gbs = nbytes / (us / 1e6) / 1e9
    return {
        "entry": "lattn_step",
        "workload": f"{spec.family} B{Bb} H{H} d_k {dk} d_v {dv} r_ab {spec.r_ab} {spec.dtype}, one token per (batch, head), "
                    f"state rotated over {nstates} buffers ({nstates * state_bytes / 2**20:.0f} MiB)",
        "us_per_step": round(us, 3),
        "us_per_step_eager_launches": round(us_eager, 3),
        "value": round(Bb / (us / 1e6), 1),
        "unit": "tokens/s",
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK["hbm_GBs"], "unit": "GB/s",
                     "frac": round(gbs / PEAK["hbm_GBs"], 4), "bytes_per_step": nbytes},
    }


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(spec, raw, budget_s):
    """Time the fp64 oracle (generic form, as used for parity) on a bounded sample of
    (batch, head) rows of the same workload, on all host cores."""
    import oracle
    cores = len(os.sched_getaffinity(0))
    per_head_core_s = spec.T * (spec.dk * spec.dk * spec.dv) * 2 / 7.8e9  # rough cost model
    n = int(max(1, min(spec.B * spec.H, round(budget_s * cores / max(per_head_core_s, 1e-9)))))
    n = max(1, min(n, spec.B * spec.H))
    flat = lambda x: x.reshape((spec.B * spec.H,) + x.shape[2:])[:n]
    if spec.family == "hdla":
        ld, A, B, K, V = oracle.hdla_to_generic(flat(raw["k"]), flat(raw["v"]), flat(raw["log_lambda"]),
                                               flat(raw["beta"]))
    elif spec.family == "gdn":
        ld, A, B, K, V = oracle.gdn_to_generic(flat(raw["k"]), flat(raw["v"]), flat(raw["g"]), flat(raw["beta"]))
    else:
        ld, A, B, K, V = (flat(raw["log_decay"]), flat(raw["A"]), flat(raw["B"]), flat(raw["K"]),
                          flat(raw["V"]))
    q = flat(raw["q"])
    t0 = time.perf_counter()
    oracle.generic(q, K, V, ld, A, B, nthreads=cores)
    wall = time.perf_counter() - t0
    head_tok_s = n * spec.T / wall
    return {
        "value": head_tok_s / spec.H,
        "unit": "tokens/s",
        "cores": int(oracle.max_threads()),
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": f"{n} of {spec.B * spec.H} (batch, head) rows x {spec.T} tokens, fp64 explicit-P_t recurrence, "
                  f"{wall:.1f} s wall; tokens/s = head-tokens/s / H",
    }


def generic_inputs(spec, draw, lattn):
    """Forward inputs from a workload's device tensors: HDLA / Gated DeltaNet decay
    operands from the device parameter kernel (outside any timed region)."""
    if spec.family == "hdla":
        A, B, V = lattn.hdla_params(draw["k"], draw["v"], draw["log_lambda"], draw["beta"])
        return draw["q"], draw["k"], V, draw["log_lambda"], A, B
    if spec.family == "gdn":
        A, B, V = lattn.gdn_params(draw["k"], draw["v"], draw["g"], draw["beta"])
        return draw["q"], draw["k"], V, draw["g"], A, B
    return draw["q"], draw["K"], draw["V"], draw["log_decay"], draw["A"], draw["B"]


def time_forward(plan, torch, dev, steps, warmup):
    """W untimed forwards, then K timed ones between device synchronizations.
    Each stage is bracketed by HIP events on the stream its kernels run on.
    Returns (ms per step by the host clock, {stage: mean event ms})."""
    for _ in range(warmup):
        plan.prepare()
        plan.scan()
    torch.cuda.synchronize(dev)
    stream = torch.cuda.current_stream(dev)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for e in evs:
        e[0].record(stream)
        plan.prepare()
        e[1].record(stream)
        plan.scan()
        e[2].record(stream)
    torch.cuda.synchronize(dev)
    ms_step = (time.perf_counter() - t0) * 1e3 / steps
    return ms_step, {"prepare": float(np.mean([e[0].elapsed_time(e[1]) for e in evs])),
                     "scan": float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))}


def roofline(spec, kernels, kernel_ms):
    """The dominant kernel against the roofline that bounds it: its share of the
    canonical algorithmic bytes (or of the flops its decomposition performs)
    divided by its event-timed duration, against the published peak."""
    kw = kernel_work(spec, kernels)
    dom = max(kernel_ms, key=kernel_ms.get)
    work = kw[dom]
    comp_peak, _ = kernel_peak(kernels, spec.dtype, "compute")
    t_comp = work["flops"] / (comp_peak * 1e12)
    t_mem = work["bytes"] / (PEAK["hbm_GBs"] * 1e9)
    sec = kernel_ms[dom] / 1e3
    if t_mem >= t_comp:
        bound, achieved, unit, peak = "hbm", work["bytes"] / sec / 1e9, "GB/s", PEAK["hbm_GBs"]
    else:
        bound, achieved, unit, peak = "mfma", work["flops"] / sec / 1e12, "TFLOP/s", comp_peak
    traffic = measured_traffic(kernels, dom, spec.name)
    out = {
        "kernel": dom,
        "bound": bound,
        "achieved": round(achieved, 2),
        "peak": peak,
        "unit": unit,
        "frac": round(achieved / peak, 4),
        "algorithmic_bytes_per_launch": work["bytes"],
        "flops_per_launch": work["flops"],
        "launch_ms": round(kernel_ms[dom], 4),
        "traffic": traffic,
    }
    if traffic:
        out["traffic_over_algorithmic"] = round(traffic / work["bytes"], 3)
    mf = measured_mfma(kernels, dom, spec.name)
    if mf:
        # counter view: the MFMA flops the kernel executed (bf16 + fp32) over its
        # event-timed duration, against the bf16 peak, and the MFMA-busy fraction
        out["mfma_counters"] = dict(mf, frac_of_bf16_peak=round(
            (mf.get("bf16_gflop", 0.0) + mf.get("fp32_gflop", 0.0)) * 1e9 / sec / (PEAK["bf16_mfma_TFs"] * 1e12), 4))
    return out


def workload_entry(spec, kernels, ms_step, kernel_ms):
    flops, nbytes = canonical_work(spec)
    comp_peak, _ = kernel_peak(kernels, spec.dtype, "compute")
    return {
        "kernels": kernels,
        "ms_per_step": round(ms_step, 4),
        "tokens_per_s": round(spec.B * spec.T / (ms_step / 1e3), 1),
        "head_tokens_per_s": round(spec.B * spec.H * spec.T / (ms_step / 1e3), 1),
        # against the matrix peak of the type the path multiplies in (bf16, or fp32 on the general path)
        "mfma_frac_canonical": round(flops / (ms_step / 1e3) / (comp_peak * 1e12), 4),
        "hbm_frac_algorithmic": round(nbytes / (ms_step / 1e3) / (PEAK["hbm_GBs"] * 1e9), 4),
        "canonical_gflop": round(flops / 1e9, 2),
        "algorithmic_gb": round(nbytes / 1e9, 4),
        "operator_gb_round_trip": round(2 * operator_bytes(spec, kernels) / 1e9, 4),
        "kernel_ms": {k: round(v, 4) for k, v in kernel_ms.items()},
        "roofline": roofline(spec, kernels, kernel_ms),
    }


def config_leg(spec, torch, lattn, dev, steps, warmup):
    """One workload timed on device-drawn inputs of its shape and distributions,
    through the generic entry point and (HDLA, Gated DeltaNet) the fused one."""
    draw = workloads.device_raw(spec, torch, dev, seed=spec.seed)
    plan = lattn.ChunkPlan(*generic_inputs(spec, draw, lattn), chunk=spec.chunk)
    kernels = plan_kernels(plan, lattn)
    ms_step, kms = time_forward(plan, torch, dev, steps, warmup)
    entry = workload_entry(spec, kernels, ms_step, kms)
    entry["workload"] = spec.describe()
    del plan
    if spec.family in ("hdla", "gdn") and kernels == "mfma_bf16":
        entry["fused_family"] = fused_leg(spec, draw, torch, lattn, dev, steps, warmup)
    return entry


def plan_kernels(plan, lattn):
    import ctypes
    return lattn._lib.load().lattn_chunk_fwd_kernels(ctypes.byref(plan.dims), plan.r_ab, plan.r_kv,
                                                     plan.chunk).decode()


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default=workloads.HEADLINE, choices=workloads.CONFIG_ORDER)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true", help="skip the timing of the other workloads")
    ap.add_argument("--no-hla", action="store_true", help="skip the query-conditioned composition leg")
    ap.add_argument("--no-loglinear", action="store_true", help="skip the log-linear lift leg")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward-pass leg")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode-step leg")
    ap.add_argument("--cpu-budget-s", type=float, default=10.0, help="target oracle wall time")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after timing, run one plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU: this path has no multi-GPU mode (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE {world}); across GPUs the (batch, head) rows would shard with no communication",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import structured_decay_sequence_amd as lattn

    spec = workloads.CONFIGS[args.config]
    dev = torch.device("cuda:0")
    print(f"[bench] {spec.describe()}: generating inputs", file=sys.stderr, flush=True)
    raw, inputs = build_inputs(spec, torch, lattn, dev)
    plan = lattn.ChunkPlan(*inputs, chunk=spec.chunk)
    kernels = plan_kernels(plan, lattn)
    print(f"[bench] kernels {kernels}: warmup {args.warmup}, timing {args.steps} steps", file=sys.stderr, flush=True)
    ms_step, kms = time_forward(plan, torch, dev, args.steps, args.warmup)

    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize(dev)
        del src, dst

    head = workload_entry(spec, kernels, ms_step, kms)
    result = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32" if kernels == "general_fp32" else spec.dtype,
        "data": "synthetic",
        "config": {
            "workload": spec.name,
            "family": spec.family, "batch": spec.B, "heads": spec.H, "seq_len": spec.T,
            "d_k": spec.dk, "d_v": spec.dv, "chunk": spec.chunk, "r_ab": spec.r_ab, "r_kv": spec.r_kv,
            "storage": spec.dtype, "kernels": kernels, "parallelism": "single-gpu",
        },
    }
    for k in ("mfma_frac_canonical", "hbm_frac_algorithmic", "canonical_gflop", "algorithmic_gb",
              "operator_gb_round_trip", "kernel_ms", "roofline"):
        result[k] = head[k]
    result["cpu_baseline"] = None
    del plan
    if spec.family in ("hdla", "gdn") and kernels == "mfma_bf16":
        td = torch.bfloat16 if spec.dtype == "bf16" else torch.float32
        t = lambda x, d=td: torch.from_numpy(np.ascontiguousarray(x)).to(d).to(dev)
        decay = "log_lambda" if spec.family == "hdla" else "g"
        draw = {"q": t(raw["q"]), "k": t(raw["k"]), "v": t(raw["v"]), decay: t(raw[decay], torch.float32),
                "beta": t(raw["beta"], torch.float32)}
        result["fused_family"] = fused_leg(spec, draw, torch, lattn, dev, args.steps, args.warmup)
        del draw
    if not args.no_configs:
        result["configs"] = {}
        for name in workloads.CONFIG_ORDER:
            if name == spec.name:
                result["configs"][name] = dict(head, workload=spec.describe(),
                                               **({"fused_family": result["fused_family"]}
                                                  if "fused_family" in result else {}))
                continue
            print(f"[bench] workload {name}", file=sys.stderr, flush=True)
            result["configs"][name] = config_leg(workloads.CONFIGS[name], torch, lattn, dev,
                                                 max(3, args.steps // 2), min(args.warmup, 3))
            torch.cuda.empty_cache()
    if not args.no_decode:
        print("[bench] decode-step leg", file=sys.stderr, flush=True)
        result["decode"] = decode_leg(spec, torch, lattn, dev, max(50, 10 * args.steps), 10)
    if spec.name == workloads.HEADLINE and not args.no_hla:
        print("[bench] query-conditioned composition leg", file=sys.stderr, flush=True)
        result["hla"] = hla_leg(torch, lattn, dev, max(1, args.steps // 4), min(args.warmup, 2))
    if spec.name == workloads.HEADLINE and not args.no_backward:
        print("[bench] backward leg", file=sys.stderr, flush=True)
        result["backward"] = backward_leg(spec, raw, inputs, torch, lattn, dev)
        result["backward"]["ratio_to_forward"] = round(result["backward"]["ms_per_step"] / result["ms_per_step"], 2)
        # the same step through the plain calls: lattn_chunk_fwd, then lattn_chunk_bwd
        result["backward"]["training_pair"]["fwd_plus_bwd_ms"] = round(
            result["ms_per_step"] + result["backward"]["ms_per_step"], 3)
    if spec.name == workloads.HEADLINE and not args.no_loglinear:
        print("[bench] log-linear lift leg", file=sys.stderr, flush=True)
        result["loglinear"] = loglinear_leg(torch, lattn, dev, max(1, args.steps // 4), min(args.warmup, 2))
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on a host sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(spec, raw, args.cpu_budget_s)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
