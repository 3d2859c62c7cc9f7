#!/usr/bin/env python3
"""Benchmark of libkda on one MI355X.

Headline (`value`): chunked-prefill tokens/s of the KDA gated delta rule on the
batched prefill workload B=8, H=32, T=8192, d_k=d_v=128, chunk 64, bf16 q/k/v/o,
fp32 gates and state (token = one (sequence, position) across all 32 heads).
One step = one kda_chunk_fwd call over the whole batch, inputs resident in HBM.

Also reported on the same line:
  roofline      achieved algorithmic HBM bytes/s of the prefill pass vs 8 TB/s, the
                measured HBM traffic, and (mfma) algorithmic TFLOP/s of the chunk form's
                products vs the 2.5 PFLOP/s bf16 matrix peak with the matrix cores' busy
                fraction from the committed counters
  decode        kda_recurrent_step on 256 sequences x 32 heads (fp32 128x128
                states, 537 MB), tokens/s = 256 / step time, with its own roofline
  workloads     the other prefill configurations, each with its roofline: prefill
                (1 x 4096 tokens, H=16), varlen (4 packed sequences, 65,536 tokens,
                H=32, chunk 128) and tiny (1 x 256 tokens, H=2, d=64, fp32) by default
  attn_decode   the softmax-attention decode step the pages compare KDA's with
  backward      kda_chunk_bwd on the batched shape with bf16 I/O (the matrix-core pass),
                and with fp32 I/O (backward_f32_io: the direct pass)
  cpu_baseline  the fp64 oracle timed on this host's cores on a bounded sample
                of the same prefill workload

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workloads prefill,varlen,tiny] [--no-bwd]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import kda_synth  # noqa: E402

HBM_PEAK_GBS = 8000.0
METRIC = "KDA tokens/sec (prefill chunked, decode step) at H=32,d=128; % roofline"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# Sources each prefill schedule's kernels are compiled from: a stored traffic
# figure is used only while these files are byte-identical to when the
# counters were taken.
CSRC = os.path.join(ROOT, "gated_delta_rule_48_amd", "csrc")
COMMON_SRC = ["kda_device.hpp", "kda_internal.hpp"]  # included by every kernel source
PATHS = {
    "fused": dict(kernel="kda_fused_kernel", sources=["kda_fused.hip"] + COMMON_SRC,
                  counters="kda_fused_kernel_batched_prefill_counters.md"),
    "segmented": dict(kernel="kda_fused_kernel (segment maps, then segments) + kda_segment_chain_kernel",
                      sources=["kda_fused.hip", "kda_segment.hip"] + COMMON_SRC,
                      counters="kda_segmented_pass_prefill_varlen_counters.md"),
    "split": dict(kernel="kda_prep_kernel + kda_state_kernel",
                  sources=["kda_prep.hip", "kda_state.hip", "kda_solve.hpp"] + COMMON_SRC,
                  counters="kda_split_pass_tiny_counters.md"),
}


def prefill_path(B, T, H, dk, dv, chunk, varlen, bf16, n_seqs=0):
    """Which schedule kda_chunk_fwd runs for these sizes: for bf16 and d_k = d_v = 128 (any
    chunk size asked) the fused pass, one workgroup per (sequence, head) when there are at
    least 256 pairs; below that the planned pass, "segmented" when it cuts sequences (segment
    0 of every sequence and the maps of the middle segments, their composition, then the
    other segments): for equal lengths when the budget leaves more than one segment per
    sequence, for packed ones (where the device plans) when the batch has 8 chunks or more;
    otherwise the split prep + state pass. Same rule as the library's dispatch."""
    if not (bf16 and dk == dv == 128 and T > 0):
        return "split"
    n = n_seqs if varlen else B
    if n * H >= 256:
        return "fused"
    u, c = 256 // H, (T + 63) // 64
    if c < 8:
        return "fused"
    if varlen:
        return "segmented"
    units_a = lambda t: max(-(-c // t) - 1, 1) if c > t else 1  # noqa: E731
    t = plan_budget(c, next(t for t in range(1, c + 1) if B * units_a(t) <= u))
    return "segmented" if c > t else "fused"


def plan_budget(c_max, t_min):
    """The library's budget choice: from the smallest budget that fits the compute units, the
    one minimising 8 T + max(ceil(c_max / T) - 2, 0) (two launches of about T chunk-steps and the
    composition's dependent steps)."""
    cost = lambda t: 8 * t + max(-(-c_max // t) - 2, 0)  # noqa: E731
    best, best_cost, t = t_min, cost(t_min), t_min + 1
    while t <= c_max and 8 * t <= best_cost:
        if cost(t) < best_cost:
            best, best_cost = t, cost(t)
        t += 1
    return best


def sources_digest(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def stored_counter(path_key, workload, key):
    """A figure of the committed rocprofv3 counter summary of this schedule, the line
    `key[workload]: value`, or None when there is none or the kernel sources changed
    since the counters were taken (the summary records their SHA-256)."""
    info = PATHS[path_key]
    fn = os.path.join(ROOT, "profiles", info["counters"])
    if not os.path.exists(fn):
        return None
    txt = open(fn).read()
    m_b = re.search(re.escape(f"{key}[{workload}]:") + r"\s*([0-9.eE+]+)", txt)
    m_h = re.search(r"sources_sha256:\s*([0-9a-f]{64})", txt)
    if not (m_b and m_h) or m_h.group(1) != sources_digest(info["sources"]):
        return None
    return float(m_b.group(1))


def stored_traffic(path_key, workload):
    """HBM bytes per call (FETCH_SIZE + WRITE_SIZE over the call's kernels, each calibrated
    on a device copy of known size), or None."""
    return stored_counter(path_key, workload, "traffic_bytes_per_launch")


def copy_probe(torch, mib):
    """A plain device copy of known size (mib MiB read, mib MiB written), launched
    three times before the timed work, so that a counter run of this script can
    calibrate FETCH_SIZE / WRITE_SIZE against exact byte counts."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[bench] copy probe: 3 x {mib} MiB device copy")
    del src, dst


def hbm_probe(torch):
    """Practical streaming bandwidth on this GPU, for reference next to the 8 TB/s peak:
    event-timed device copies and in-place multiplies of 0.5, 1 and 2 GiB (bytes read +
    bytes written over the time), 10 repetitions after 3 warm-up ones. Logged only."""
    for mib in (512, 1024, 2048):
        n = mib * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device="cuda:0")
        b = torch.empty_like(a)
        for name, fn in (("copy", lambda: b.copy_(a)), ("in-place multiply", lambda: a.mul_(1.0001))):
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(10):
                fn()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / 10
            log(f"[bench] hbm probe: {name} of {mib} MiB: {ms:.3f} ms, "
                f"{2 * mib * (1 << 20) / (ms * 1e-3) / 1e9:.0f} GB/s (read + write)")
        del a, b


def spin_up(torch, fn, seconds):
    """Run fn back to back for about `seconds` before a leg's warm-up steps. The GPU idles
    while a leg's inputs are generated on the host, and its clocks take tens of milliseconds
    of load to return to their sustained level: a few warm-up steps alone leave the timed
    steps partly on the ramp (the batched prefill measured 0.85 ms per step after 5 warm-up
    steps, 0.75 ms after 50). Nothing here is timed or reported except its duration."""
    if seconds <= 0:
        return
    t0 = time.perf_counter()
    n = 0
    while True:
        for _ in range(8):
            fn()
        n += 8
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            break
    log(f"[bench] spin-up: {n} calls in {time.perf_counter() - t0:.2f} s")


def prefill_algorithmic_bytes(token_heads, dk, dv, io_bytes, n_states_out, n_states_in, gate="channel"):
    """q, k, v, o in the I/O dtype, log_alpha (fp32: per key channel, one per token and
    head, or none) and beta (fp32) per token-head, plus the fp32 states read and written."""
    # gates: log_alpha fp32 per key channel, one per token and head, none, or (preact) the
    # decay's pre-activation in the io dtype; then beta (or its pre-activation), fp32
    per = (2 * dk + 2 * dv) * io_bytes + {"channel": 4 * dk, "head": 4, "none": 0, "preact": io_bytes * dk,
                                          "preact_qk": io_bytes * dk}[gate] + 4
    return token_heads * per + 4 * dk * dv * (n_states_out + n_states_in)


BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak


def prefill_algorithmic_flops(seqlens, H, dk, dv, C):
    """Flops of the chunk form's products per call (2 per multiply-add), each dense product
    counted once at its full size: per chunk of C rows and head, the Gram matrices of the
    solve and of the output (K K^T and Q K^T, C x C x dk each), W = T Bk (C x C x dk), U~ = T Bv
    (C x C x dv), the intra-chunk output Aqk U (C x C x dv), and the three state products
    W S, Q S and R^T U (C x dk x dv each). The triangular solve, the decay factors and the
    segment maps of the segmented pass are not counted."""
    macs = 3 * C * C * dk + 2 * C * C * dv + 3 * C * dk * dv
    chunks = sum((n + C - 1) // C for n in seqlens)
    return 2 * macs * chunks * H


def mfma_roofline(flops, ms, path_key, workload):
    """Algorithmic TFLOP/s of the call against the bf16 matrix peak, and the matrix cores'
    busy fraction over the call's kernels from the committed counters (SQ_VALU_MFMA_BUSY_CYCLES
    over 4 x SQ_BUSY_CU_CYCLES: four matrix units per CU), or None."""
    t = flops / (ms * 1e-3) / 1e12
    return {"achieved": round(t, 2), "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(t / BF16_MFMA_PEAK_TFLOPS, 4), "alg_flops_per_launch": flops,
            "busy": stored_counter(path_key, workload, "mfma_busy_frac")}




def bench_prefill(args, kda, torch):
    w = kda_synth.WORKLOADS["batched"]
    B, T, H, dk, dv, C = len(w.seqlens), w.seqlens[0], w.H, w.dk, w.dv, w.chunk
    log(f"[bench] generating prefill inputs B={B} T={T} H={H} d={dk}")
    t0 = time.time()
    x = kda_synth.gen_workload(w)
    log(f"[bench] generated in {time.time() - t0:.1f}s")
    dev = torch.device("cuda:0")
    q = torch.from_numpy(x["q"]).to(dev).to(torch.bfloat16).reshape(B, T, H, dk)
    k = torch.from_numpy(x["k"]).to(dev).to(torch.bfloat16).reshape(B, T, H, dk)
    v = torch.from_numpy(x["v"]).to(dev).to(torch.bfloat16).reshape(B, T, H, dv)
    la = torch.from_numpy(x["log_alpha"]).to(dev).reshape(B, T, H, dk)
    beta = torch.from_numpy(x["beta"]).to(dev).reshape(B, T, H)
    o = torch.empty((B, T, H, dv), dtype=torch.bfloat16, device=dev)
    hT = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    ws = torch.empty(kda.workspace_bytes(B, T, H, dk, dv, C, 0, kda.KDA_BF16), dtype=torch.uint8,
                     device=dev)

    def step():
        kda.chunk_fwd(q, k, v, la, beta, chunk=C, o=o, hT=hT, workspace=ws)

    spin_up(torch, step, args.spin_up)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for i in range(args.steps):
        starts[i].record()
        step()
        ends[i].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ev_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    ms = wall * 1000.0 / args.steps
    tokens = B * T
    token_heads = tokens * H
    alg = prefill_algorithmic_bytes(token_heads, dk, dv, 2, B * H, 0)
    ev_avg = float(np.mean(ev_ms))
    achieved = alg / (ev_avg * 1e-3) / 1e9
    log(f"[bench] prefill: wall {ms:.3f} ms/step, events avg {ev_avg:.3f} min {min(ev_ms):.3f} ms, "
        f"{tokens / (ms * 1e-3):.3e} tokens/s, {achieved:.0f} GB/s algorithmic")
    path = prefill_path(B, T, H, dk, dv, C, False, True)
    res = dict(ms=ms, ev_ms=ev_avg, tokens_per_s=tokens / (ms * 1e-3), alg_bytes=alg,
               achieved_gbs=achieved, workload=w, x=x, path=path,
               mfma=mfma_roofline(prefill_algorithmic_flops(w.seqlens, H, dk, dv, 64), ev_avg, path, "batched"))
    del q, k, v, la, beta, o, hT, ws
    return res


def bench_workload(args, kda, torch, name):
    """kda_chunk_fwd on another synthetic workload of kda_synth (the schedule the library
    picks for it), event-timed like the headline: ms per call, tokens/s and algorithmic
    GB/s against the HBM peak. Equal-length sequences are passed as [B, T, H, d], others
    packed with cu_seqlens."""
    w = kda_synth.WORKLOADS[name]
    log(f"[bench] generating workload {name}: seqlens {w.seqlens}, H={w.H}, d={w.dk}, chunk {w.chunk}, {w.io}")
    x = kda_synth.gen_workload(w)
    dev = torch.device("cuda:0")
    dt = torch.bfloat16 if w.io == "bf16" else torch.float32
    varlen = len(set(w.seqlens)) > 1
    B, T = (1, sum(w.seqlens)) if varlen else (len(w.seqlens), w.seqlens[0])
    lead = (T,) if varlen else (B, T)
    q = torch.from_numpy(x["q"]).to(dev).to(dt).reshape(lead + (w.H, w.dk))
    k = torch.from_numpy(x["k"]).to(dev).to(dt).reshape(lead + (w.H, w.dk))
    v = torch.from_numpy(x["v"]).to(dev).to(dt).reshape(lead + (w.H, w.dv))
    la = torch.from_numpy(x["log_alpha"]).to(dev).reshape(lead + (w.H, w.dk))
    if w.gate == "head":    # one decay per token and head: the first key channel's draw
        la = la[..., 0].contiguous()
    elif w.gate == "none":  # no decay
        la = None
    pre = None
    if w.gate == "preact_qk":  # q and k before silu and normalisation
        r = kda_synth.gen_qk_preact(sum(w.seqlens), w.H, w.dk, w.io, w.seed)
        q = torch.from_numpy(r["q"]).to(dev).to(dt).reshape(lead + (w.H, w.dk))
        k = torch.from_numpy(r["k"]).to(dev).to(dt).reshape(lead + (w.H, w.dk))
    if w.gate in ("preact", "preact_qk"):  # gates formed in the kernels from pre-activations
        p = kda_synth.gen_preact(sum(w.seqlens), w.H, w.dk, w.io, w.seed)
        pre = dict(a=torch.from_numpy(p["a"]).to(dev).to(dt).reshape(lead + (w.H, w.dk)),
                   A_log=torch.from_numpy(p["A_log"]).to(dev), dt_bias=torch.from_numpy(p["dt_bias"]).to(dev),
                   b=torch.from_numpy(p["b"]).to(dev).reshape(lead + (w.H,)))
        la = beta = None
    beta = torch.from_numpy(x["beta"]).to(dev).reshape(lead + (w.H,))
    h0 = None if x["h0"] is None else torch.from_numpy(x["h0"]).to(dev)
    cu = torch.from_numpy(x["cu_seqlens"]).to(dev) if varlen else None
    n_seqs = len(w.seqlens)
    o = torch.empty(lead + (w.H, w.dv), dtype=dt, device=dev)
    hT = torch.empty((n_seqs, w.H, w.dk, w.dv), dtype=torch.float32, device=dev)
    io = kda.KDA_BF16 if w.io == "bf16" else kda.KDA_F32
    ws = torch.empty(kda.workspace_bytes(B, T, w.H, w.dk, w.dv, w.chunk, n_seqs if varlen else 0, io),
                     dtype=torch.uint8, device=dev)

    def step():
        if pre is not None:
            kda.chunk_fwd_preact(q, k, v, pre["a"], pre["A_log"], pre["dt_bias"], pre["b"], scale=w.scale, h0=h0,
                                 cu_seqlens=cu, chunk=w.chunk, o=o, hT=hT, workspace=ws,
                                 qk_norm=w.gate == "preact_qk")
        else:
            kda.chunk_fwd(q, k, v, la, beta, scale=w.scale, h0=h0, cu_seqlens=cu, chunk=w.chunk, o=o, hT=hT,
                          workspace=ws)

    spin_up(torch, step, args.spin_up)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    tokens = sum(w.seqlens)
    alg = prefill_algorithmic_bytes(tokens * w.H, w.dk, w.dv, 2 if w.io == "bf16" else 4, n_seqs * w.H,
                                    0 if h0 is None else n_seqs * w.H, w.gate)
    achieved = alg / (ms * 1e-3) / 1e9
    path = prefill_path(B, T, w.H, w.dk, w.dv, w.chunk, varlen, w.io == "bf16", len(w.seqlens))
    mf = mfma_roofline(prefill_algorithmic_flops(w.seqlens, w.H, w.dk, w.dv, w.chunk if path == "split" else 64),
                       ms, path, name)
    log(f"[bench] workload {name} ({path} pass): {ms:.3f} ms/call, {tokens / (ms * 1e-3):.3e} tokens/s, "
        f"{achieved:.0f} GB/s algorithmic, {mf['achieved']:.1f} TFLOP/s")
    return {"value": tokens / (ms * 1e-3), "unit": "tokens/s", "ms_per_call": round(ms, 4), "pass": path,
            "kernel": PATHS[path]["kernel"],
            "workload": f"seqlens {list(w.seqlens)}, H={w.H}, d_k=d_v={w.dk}, chunk {w.chunk}, {w.io} q/k/v/o, "
                        + {"channel": "decay per key channel", "head": "decay per token and head", "none": "no decay",
                           "preact": "gates formed in the kernel from pre-activations",
                           "preact_qk": "gates, and q and k (silu, L2 norm), formed in the kernel"}[w.gate],
            "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(achieved / HBM_PEAK_GBS, 4), "alg_bytes_per_launch": alg,
                         "traffic": stored_traffic(path, name), "mfma": mf}}


def bench_decode(args, kda, torch):
    d = kda_synth.DECODE
    N, H, dk, dv = d["N"], d["H"], d["dk"], d["dv"]
    bank = args.decode_bank
    log(f"[bench] generating decode state ({N}x{H}x{dk}x{dv} fp32) and {bank} distinct steps")
    dev = torch.device("cuda:0")
    state = torch.from_numpy(kda_synth.gen_decode_state(N, H, dk, dv, d["seed"])).to(dev)
    steps_in = []
    for s in range(bank):
        y = kda_synth.gen_decode_step(N, H, dk, dv, "bf16", "main", d["seed"], s)
        steps_in.append(dict(
            q=torch.from_numpy(y["q"]).to(dev).to(torch.bfloat16),
            k=torch.from_numpy(y["k"]).to(dev).to(torch.bfloat16),
            v=torch.from_numpy(y["v"]).to(dev).to(torch.bfloat16),
            la=torch.from_numpy(y["log_alpha"]).to(dev), beta=torch.from_numpy(y["beta"]).to(dev)))
    o = torch.empty((N, H, dv), dtype=torch.bfloat16, device=dev)

    def step(i):
        s = steps_in[i % bank]
        kda.recurrent_step(s["q"], s["k"], s["v"], s["la"], s["beta"], state, o=o)

    it = iter(range(1 << 30))
    spin_up(torch, lambda: step(next(it)), args.spin_up)
    for i in range(8):
        step(i)
    torch.cuda.synchronize()
    n = args.decode_steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    e0.record()
    for i in range(n):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms = e0.elapsed_time(e1) / n
    nh = N * H
    alg = nh * (2 * 4 * dk * dv + (2 * dk + 2 * dv) * 2 + 4 * dk + 4)
    achieved = alg / (ms * 1e-3) / 1e9
    log(f"[bench] decode: {ms * 1000:.1f} us/step (wall {wall * 1000 / n * 1000:.1f}), "
        f"{N / (ms * 1e-3):.3e} tokens/s, {achieved:.0f} GB/s")
    return dict(ms=ms, tokens_per_s=N / (ms * 1e-3), alg_bytes=alg, achieved_gbs=achieved, steps=n)


def bench_attn(args, kda, torch, name, dec):
    """The comparator: a softmax-attention layer's decode step over a KV cache
    (kda_attn_decode), one new token per sequence, caches drawn on the GPU."""
    B, H, H_kv, T_max, d, io, seed = kda_synth.ATTN_WORKLOADS[name]
    dev = torch.device("cuda:0")
    log(f"[bench] generating attention workload {name}: B={B} H={H} H_kv={H_kv} T_max={T_max} d={d} {io}")
    x = kda_synth.gen_attn_decode_device(B, H, H_kv, T_max, d, torch.bfloat16, seed, dev)
    o = torch.empty((B, H, d), dtype=torch.bfloat16, device=dev)
    n_ws = kda.attn_decode_workspace_bytes(B, H, H_kv, d, T_max, kda.KDA_BF16)
    ws = torch.empty(max(n_ws, 1), dtype=torch.uint8, device=dev)

    def step():
        kda.attn_decode(x["q"], x["k_cache"], x["v_cache"], o=o, workspace=ws)

    spin_up(torch, step, args.spin_up)
    for _ in range(3):
        step()
    torch.cuda.synchronize()
    n = args.attn_steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for e0, e1 in ev:
        e0.record()
        step()
        e1.record()
    torch.cuda.synchronize()
    ms = sum(e0.elapsed_time(e1) for e0, e1 in ev) / n
    alg = B * H_kv * T_max * d * 2 * 2 + 2 * B * H * d * 2  # both caches read once; q read, o written
    achieved = alg / (ms * 1e-3) / 1e9
    log(f"[bench] attention decode {name}: {ms * 1000:.1f} us/step, {B / (ms * 1e-3):.3e} tokens/s, "
        f"{achieved:.0f} GB/s")
    out = {"value": B / (ms * 1e-3), "unit": "tokens/s", "us_per_step": round(ms * 1000, 2), "steps": n,
           "workload": f"{B} sequences x {H} query heads ({H_kv} cached), d={d}, {T_max} cached rows each, "
                       "bf16 caches",
           "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(achieved / HBM_PEAK_GBS, 4), "alg_bytes_per_launch": alg}}
    if dec is not None and name == "attn_batched":  # the same 256 x 32 (sequence, head) pairs
        out["time_vs_kda_decode"] = round(ms / dec["ms"], 2)
    del x, o, ws
    torch.cuda.empty_cache()
    return out


FP32_MATRIX_PEAK_TFLOPS = 157.3  # MI355X dense fp32 matrix (and vector) peak


def bwd_algorithmic_flops(B, T, H, dk, dv, C=64):
    """Flops of the backward pass's products per call (2 per multiply-add), each counted once:
    the chunk-local forward (P N^T, Qe N^T, T Bk, T Bv), the state recursion (W S, R^T U), the
    state-gradient recursion (Aqk^T dO, R dS', QO^T dO, W^T dU) and the chunk-local gradients
    (dO S^T, dO U^T, U dS'^T, dU S^T, T^T dU, dU Bv^T, dW Bk^T, T^T dW, T^T dT, (T^T dT) T^T,
    dA N, dA^T P, dAqk^T Qe, dAqk N). Elementwise work and the triangular solve are not counted."""
    macs = (2 * C * C * dk + C * dk * C + C * dv * C            # chunk-local forward
            + C * dv * dk + dk * dv * C                         # states
            + C * dv * C + C * dv * dk + dk * dv * C + dk * dv * C  # state gradients
            + 3 * C * dk * dv + C * C * dv + C * dv * C + C * C * dv + C * C * dk + C * dk * C
            + 2 * C * C * C + 4 * C * dk * C)                   # chunk-local gradients
    return 2 * macs * B * ((T + C - 1) // C) * H


def bwd_algorithmic_bytes(B, T, H, dk, dv, io_bytes):
    """Bytes the backward pass must move at least: q, k, v, the output gradient and dq, dk,
    dv in the io dtype, log_alpha and dlog_alpha (fp32, per key channel), beta and dbeta per
    token-head, and the fp32 loss gradient of each final state (dhT) read."""
    per = (2 * dk + 2 * dv) * io_bytes + (2 * dk + dv) * io_bytes + 2 * 4 * dk + 2 * 4
    return B * T * H * per + B * H * dk * dv * 4


def bench_bwd(args, kda, torch, io="f32"):
    """The backward pass (kda_chunk_bwd) on the batched workload's shape: B=8, T=8192, H=32,
    d=128, chunk 64, q, k, v and the output gradient in `io` (fp32 arithmetic either way),
    inputs and loss gradients drawn on the GPU (torch's seeded generator)."""
    B, T, H, d = 8, 8192, 32, 128
    dev = torch.device("cuda:0")
    log(f"[bench] generating backward inputs: B={B} T={T} H={H} d={d} {io}")
    g = torch.Generator(device=dev)
    g.manual_seed(1007)
    rn = lambda *s: torch.randn(s, generator=g, device=dev)  # noqa: E731
    q = torch.nn.functional.normalize(rn(B, T, H, d), dim=-1)
    k = torch.nn.functional.normalize(rn(B, T, H, d), dim=-1)
    v, dout = rn(B, T, H, d), rn(B, T, H, d)
    if io == "bf16":
        q, k, v, dout = (x.to(torch.bfloat16) for x in (q, k, v, dout))
    la = -0.1 * torch.nn.functional.softplus(rn(B, T, H, d))
    beta = torch.sigmoid(rn(B, T, H))
    dhT = rn(B, H, d, d)
    ws = torch.empty(kda.chunk_bwd_workspace_bytes(B, T, H, d, d), dtype=torch.uint8, device=dev)

    def step():
        kda.chunk_bwd(q, k, v, la, beta, dout, dhT=dhT, workspace=ws)

    spin_up(torch, step, args.spin_up)
    step()
    torch.cuda.synchronize()
    n = args.bwd_steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    flops = bwd_algorithmic_flops(B, T, H, d, d)
    tflops = flops / (ms * 1e-3) / 1e12
    nbytes = bwd_algorithmic_bytes(B, T, H, d, d, 2 if io == "bf16" else 4)
    gbs = nbytes / (ms * 1e-3) / 1e9
    if io == "bf16":
        # the matrix-core pass (bf16 products): 1.07 TFLOP is 0.43 ms at the bf16 peak, the
        # 5.9 GB of inputs and gradients 0.74 ms at 8 TB/s, so HBM bounds it
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4), "alg_bytes_per_call": nbytes,
                "mfma": {"achieved": round(tflops, 2), "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4), "alg_flops_per_call": flops}}
        kind = "matrix-core pass, bf16 products"
    else:
        # the direct pass (fp32 products): 6.8 ms at the fp32 matrix peak against 1.2 ms of HBM time
        roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": FP32_MATRIX_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tflops / FP32_MATRIX_PEAK_TFLOPS, 4), "alg_flops_per_call": flops,
                "alg_bytes_per_call": nbytes}
        kind = "direct pass, fp32 products"
    log(f"[bench] backward ({io} I/O, {kind}): {ms:.2f} ms/call, {B * T / (ms * 1e-3):.3e} tokens/s, "
        f"{tflops:.1f} TFLOP/s and {gbs:.0f} GB/s algorithmic")
    del q, k, v, dout, la, beta, dhT, ws
    torch.cuda.empty_cache()
    return {"value": B * T / (ms * 1e-3), "unit": "tokens/s", "ms_per_call": round(ms, 3), "steps": n,
            "workload": f"backward of the batched prefill: B={B} x T={T}, H={H}, d_k=d_v={d}, chunk 64, {io} I/O "
                        f"({kind})",
            "roofline": roof}


def bench_bwd_strong(args, kda, torch):
    """The backward's token pass: kda_chunk_bwd on one sequence of 8,192 tokens, one head, d=128,
    once with ordinary gates and once with chunk 1 at log alpha = -8 on every channel (a chunk
    sum of -512, past the chunked passes' range, so the pair is recomputed token by token), in
    both I/O dtypes; the difference of the two times is the token pass's cost for the pair."""
    B, T, H, d = 1, 8192, 1, 128
    dev = torch.device("cuda:0")
    out = {}
    for io in ("bf16", "f32"):
        g = torch.Generator(device=dev)
        g.manual_seed(1011)
        rn = lambda *s: torch.randn(s, generator=g, device=dev)  # noqa: E731
        q = torch.nn.functional.normalize(rn(B, T, H, d), dim=-1)
        k = torch.nn.functional.normalize(rn(B, T, H, d), dim=-1)
        v, dout = rn(B, T, H, d), rn(B, T, H, d)
        if io == "bf16":
            q, k, v, dout = (x.to(torch.bfloat16) for x in (q, k, v, dout))
        la = -torch.nn.functional.softplus(rn(B, T, H, d) - 2.0)
        beta = torch.sigmoid(rn(B, T, H))
        ws = torch.empty(kda.chunk_bwd_workspace_bytes(B, T, H, d, d, io=kda.KDA_BF16 if io == "bf16" else kda.KDA_F32),
                         dtype=torch.uint8, device=dev)
        times = {}
        for case in ("ordinary", "one strong chunk"):
            if case != "ordinary":
                la[:, 64:128] = -8.0

            def step():
                kda.chunk_bwd(q, k, v, la, beta, dout, workspace=ws)

            step()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(args.bwd_steps):
                step()
            e1.record()
            torch.cuda.synchronize()
            times[case] = e0.elapsed_time(e1) / args.bwd_steps
        extra = times["one strong chunk"] - times["ordinary"]
        log(f"[bench] backward token pass ({io} I/O): {times['ordinary']:.3f} ms/call with ordinary gates, "
            f"{times['one strong chunk']:.3f} ms with one strong chunk: {extra:.2f} ms for the pair's {T} tokens "
            f"({extra * 1000 / T:.2f} us per token)")
        out[io] = {"ms_ordinary": round(times["ordinary"], 3), "ms_one_strong_chunk": round(times["one strong chunk"], 3),
                   "us_per_token": round(extra * 1000 / T, 3)}
        del q, k, v, dout, la, beta, ws
        torch.cuda.empty_cache()
    return out


def cpu_baseline(pre, args):
    """The fp64 oracle on the prefill workload's first `--cpu-seqs` sequences (all
    of them by default: all heads, full length), on this host's cores."""
    import oracle
    x, w = pre["x"], pre["workload"]
    n_seq = args.cpu_seqs
    T = w.seqlens[0]
    sl = slice(0, n_seq * T)
    cores = len(os.sched_getaffinity(0))
    cu = np.arange(n_seq + 1, dtype=np.int64) * T
    sub = {n: np.ascontiguousarray(x[n][sl]) for n in ("q", "k", "v", "log_alpha", "beta")}
    log(f"[bench] cpu baseline: oracle on {n_seq} sequences x {w.H} heads x {T} tokens, "
        f"{cores} threads")
    t0 = time.perf_counter()
    oracle.kda_reference(sub["q"], sub["k"], sub["v"], sub["log_alpha"], sub["beta"], w.scale,
                         cu_seqlens=cu, threads=cores)
    dt = time.perf_counter() - t0
    tokens = n_seq * T
    log(f"[bench] cpu baseline: {dt:.2f}s, {tokens / dt:.1f} tokens/s")
    return {"value": tokens / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{n_seq} of the {len(w.seqlens)} sequences (all {w.H} heads, {T} tokens each) of "
                      f"the batched prefill workload; fp64 token-by-token recurrence, {dt:.2f} s"}


def trace_summary(csv_path, last):
    """Markdown table of a rocprofv3 kernel trace (`--kernel-trace --output-format csv`,
    the *_kernel_trace.csv file): per (kernel, grid, workgroup size), in order of first
    dispatch, the number of dispatches, the average duration over all of them and over the
    last `last` (a leg's timed launches are its last --steps dispatches)."""
    import csv
    groups = {}
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            wg = int(r["Workgroup_Size_X"]) * int(r["Workgroup_Size_Y"]) * int(r["Workgroup_Size_Z"])
            grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"]) // max(wg, 1)
            key = (r["Kernel_Name"], grid, wg)
            groups.setdefault(key, []).append((int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    print(f"| kernel | workgroups | threads | dispatches | average (us) | average of the last {last} (us) |")
    print("|---|---|---|---|---|---|")
    for (name, grid, wg), v in sorted(groups.items(), key=lambda kv: min(t for t, _ in kv[1])):
        v.sort()
        d = [(e - b) / 1000.0 for b, e in v]
        tail = d[-last:]
        short = name if len(name) <= 90 else name[:87] + "..."
        print(f"| `{short}` | {grid} | {wg} | {len(d)} | {sum(d) / len(d):.1f} | {sum(tail) / len(tail):.1f} |")


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--trace-summary":
        ap = argparse.ArgumentParser()
        ap.add_argument("--trace-summary", metavar="CSV", required=True)
        ap.add_argument("--last", type=int, default=20)
        a = ap.parse_args()
        trace_summary(a.trace_summary, a.last)
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--spin-up", type=float, default=0.3, metavar="SECONDS",
                    help="untimed back-to-back calls before each leg's warm-up steps (GPU clocks)")
    ap.add_argument("--decode-steps", type=int, default=1024)
    ap.add_argument("--decode-bank", type=int, default=32)
    ap.add_argument("--cpu-seqs", type=int, default=8)
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="run a device copy of MIB MiB first (counter calibration)")
    ap.add_argument("--hbm-probe", action="store_true",
                    help="log the streaming bandwidth of device copies and in-place multiplies first")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--attn", default="attn_batched", metavar="NAMES",
                    help="attention-decode comparator workloads to time (" + ", ".join(kda_synth.ATTN_WORKLOADS) +
                         "; empty for none)")
    ap.add_argument("--attn-steps", type=int, default=50)
    ap.add_argument("--no-bwd", action="store_true",
                    help="skip the backward pass on the batched shape (fp32 and bf16 I/O)")
    ap.add_argument("--bwd", action="store_true", help=argparse.SUPPRESS)  # the default; kept for old commands
    ap.add_argument("--bwd-steps", type=int, default=3)
    ap.add_argument("--bwd-strong", action="store_true",
                    help="also time the backward's token pass (one sequence of 8192 tokens, one head, with and "
                         "without a chunk of strong decay)")
    ap.add_argument("--workloads", default="prefill,varlen,tiny", metavar="NAMES",
                    help="comma-separated further prefill workloads to time and report (" +
                         ", ".join(n for n in kda_synth.WORKLOADS if n != "batched") + "; empty for none)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); the "
              "path has no multi-GPU mode.", file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_delta_rule_48_amd as kda
    kda.load()
    torch.cuda.set_device(0)

    if args.copy_probe > 0:
        copy_probe(torch, args.copy_probe)
    if args.hbm_probe:
        hbm_probe(torch)
    pre = bench_prefill(args, kda, torch)
    dec = None if args.no_decode else bench_decode(args, kda, torch)
    others = {n: bench_workload(args, kda, torch, n) for n in args.workloads.split(",") if n}
    attn = {n: bench_attn(args, kda, torch, n, dec) for n in args.attn.split(",") if n}
    bwd = None if args.no_bwd else {io: bench_bwd(args, kda, torch, io) for io in ("bf16", "f32")}
    bwd_strong = bench_bwd_strong(args, kda, torch) if args.bwd_strong else None
    cpu = None if args.no_cpu_baseline else cpu_baseline(pre, args)

    w = pre["workload"]
    line = {
        "metric": METRIC,
        "value": pre["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": pre["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "KDA batched chunked prefill: B=8 sequences x T=8192 tokens, H=32 heads, "
                               "d_k=d_v=128, chunk 64, bf16 q/k/v/o, fp32 log_alpha/beta/state",
                   "global_batch": len(w.seqlens), "seq_len": w.seqlens[0], "heads": w.H,
                   "d_k": w.dk, "d_v": w.dv, "chunk": w.chunk, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(pre["achieved_gbs"], 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(pre["achieved_gbs"] / HBM_PEAK_GBS, 4),
                     "traffic": stored_traffic(pre["path"], "batched"), "mfma": pre["mfma"],
                     "kernel": PATHS[pre["path"]]["kernel"],
                     "alg_bytes_per_launch": pre["alg_bytes"], "avg_launch_ms": round(pre["ev_ms"], 4)},
        "cpu_baseline": cpu,
    }
    if dec is not None:
        line["decode"] = {"value": dec["tokens_per_s"], "unit": "tokens/s", "us_per_step": round(dec["ms"] * 1000, 2),
                          "steps": dec["steps"], "workload": "256 sequences x 32 heads, fp32 128x128 states, bf16 token",
                          "roofline": {"bound": "hbm", "achieved": round(dec["achieved_gbs"], 1),
                                       "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                       "frac": round(dec["achieved_gbs"] / HBM_PEAK_GBS, 4),
                                       "alg_bytes_per_launch": dec["alg_bytes"]}}
    if attn:
        line["attn_decode"] = attn
    if bwd is not None:
        line["backward"] = bwd["bf16"]
        line["backward_f32_io"] = bwd["f32"]
    if bwd_strong is not None:
        line["backward_token_pass"] = bwd_strong
    if others:
        line["workloads"] = others
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
