#!/usr/bin/env python3
"""Benchmark of the dual-path quantized-base + LoRA linear on one MI355X.

Headline (value): one 7B-style block of seven q8_0 linears at batch 1, each
with a rank-16 LoRA at scale 1.0 (q,k,v,o 4096x4096; gate/up 4096->11008;
down 11008->4096), run through qbl_block (prep/shrink + fused dequant-GEMV +
expand, with the linear glue between the linears).  A step is one block for
one token; the inputs are resident in HBM and the step rotates over
independent copies of the weights and adapters so the 256 MB Infinity Cache
cannot serve them.  value = algorithmic bytes per step / time per step.

Also reported on the same JSON line:
  roofline      the fused GEMV kernel: algorithmic bytes per launch / average
                launch duration (HIP events on the launch stream), vs 8 TB/s
  cpu_baseline  the float64 C oracle on the host cores, same workload
  stack         32 such blocks, two adapters (r16@1.0 then r64@0.5), 256 tokens
  q4_mlp        70B-style q4_sm MLP linears at batch 1 and 8
  q4k_mlp       the same MLP with a q4_K (256-weight super-block) base
  sparse_block  the 7B block with its LoRA and a 10%-dense sparse (CSR) delta
  dar           drift of dequantize-add-requantize merges (the merge the overlay
                avoids) and the requantise kernel's time
  prefill       the JIT-materialisation prefill GEMM (when available)
  stack.lifecycle  load (staging + verification + digest), attach, rollback and
                base-hash costs on the stack
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
METRIC = "batch-1 q8_0+LoRA GEMV effective GB/s and % HBM peak; tokens/s over 32-block stack"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def linear_bytes(wl, i, with_a=True):
    """Algorithmic bytes of one linear at batch 1: quantised base, LoRA factors
    (A only if the shrink is counted), x read once, y written once."""
    L = wl.linears[i]
    r = sum(a.rank for a in wl.adapters)
    b = wl.base_bytes(i) + 4 * r * L.n_out + 4 * (L.n_out + L.k_in)
    if with_a:
        b += 4 * r * L.k_in
    return b


def group_bytes(wl, lins):
    """Algorithmic bytes of one batch-1 launch over linears `lins` sharing one
    input: their quantised bases and LoRA factors, the input read once, one
    output vector written."""
    r = sum(a.rank for a in wl.adapters)
    L0 = wl.linears[lins[0]]
    b = 4 * (L0.k_in + L0.n_out)
    for i in lins:
        L = wl.linears[i]
        b += wl.base_bytes(i) + 4 * r * (L.n_out + L.k_in)
    return b


def build_copies(q, wl, copies, adapter_idx, timing=None):
    """One base holding `copies` copies of the workload's linears, one adapter
    per workload adapter covering every copy; returns (base, adapters, comp, blocks).
    With a `timing` dict, records the wall time and bytes of the base load and
    of the adapter loads (each: staging, upload, read-back verification, digest)."""
    blocks = [q.qbl_quantize(L.qtype, wl.weight(i)) for i, L in enumerate(wl.linears)]
    descs = []
    for c in range(copies):
        for i, L in enumerate(wl.linears):
            descs.append((L.qtype, L.n_out, L.k_in, blocks[i]))
    t0 = time.time()
    base = q.qbl_base_load(descs)
    if timing is not None:
        timing["base_load_s"] = time.time() - t0
        timing["base_bytes"] = sum(int(d[3].nbytes) for d in descs)
    n = len(wl.linears)
    ads = []
    for a in adapter_idx:
        fac = [(wl.lora_a(i, a), wl.lora_b(i, a)) for i in range(n)]
        entries = [(c * n + i, A, B) for c in range(copies) for i, (A, B) in enumerate(fac)]
        t0 = time.time()
        ads.append(q.qbl_adapter_load(base, entries))
        if timing is not None:
            timing["adapter_load_s"] = timing.get("adapter_load_s", 0.0) + time.time() - t0
            timing["adapter_bytes"] = timing.get("adapter_bytes", 0) + sum(A.nbytes + B.nbytes for _, A, B in entries)
    comp = q.qbl_comp_create(base)
    q.qbl_comp_attach(comp, ads, [wl.adapters[a].scale for a in adapter_idx])
    return base, ads, comp, blocks


def free_all(q, base, ads, comp):
    q.qbl_comp_free(comp)
    for a in ads:
        q.qbl_adapter_free(a)
    q.qbl_base_free(base)


def time_loop(torch, fn, steps, warmup):
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def sources_sha256(paths):
    """SHA-256 over the concatenated bytes of the given repository files."""
    import hashlib
    h = hashlib.sha256()
    for rel in paths:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def profile_field(summary, key):
    """A machine-readable figure of a profiles/ summary (indented `key: value`
    lines), or None when the summary is missing or any source file the kernel
    compiles from (its `kernel_sources` line) changed since it was taken."""
    path = os.path.join(ROOT, "profiles", summary)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and line.startswith("    "):
            k, v = line.strip().split(":", 1)
            fields[k.strip()] = v.strip()
    try:
        if sources_sha256(fields["kernel_sources"].split()) != fields["kernel_sources_sha256"]:
            return None
        return float(fields[key])
    except (KeyError, OSError, ValueError):
        return None


def counter_traffic(summary):
    """HBM bytes per launch measured with rocprofv3 byte counters (FETCH_SIZE +
    WRITE_SIZE, scaled by a copy of known size), as recorded in a profiles/
    summary; None when the kernel's sources changed since then."""
    v = profile_field(summary, "traffic_bytes_per_launch")
    return None if v is None else int(v)


def bench_block(torch, q, workloads, args):
    wl = workloads.block()
    copies = args.copies
    log(f"[block] building {copies} copies of one 7B block (q8_0, r16)")
    t0 = time.time()
    base, ads, comp, blocks = build_copies(q, wl, copies, [0])
    log(f"[block] built in {time.time() - t0:.1f}s")
    x = torch.from_numpy(wl.x0()[0]).cuda()
    ys = [torch.empty(4096, dtype=torch.float32, device="cuda") for _ in range(copies)]
    ws = q.workspace(comp, q.OP_BLOCK)

    def step(i):
        q.qbl_block(comp, i % copies, x, ys[i % copies], ws)

    # median over repeats of `steps` timed steps each (HIP events on the stream;
    # batch-1 runs with adapters refuse graph capture, so the steps are stream
    # launches)
    reps = [time_loop(torch, step, args.steps, args.warmup if r == 0 else 2) for r in range(args.repeats)]
    ms = sorted(reps)[len(reps) // 2]
    step_bytes = sum(linear_bytes(wl, i) for i in range(7))
    gbs = step_bytes / (ms * 1e-3) / 1e9
    log(f"[block] {ms * 1e3:.1f} us/step (median of {len(reps)}: {[round(r * 1e3, 1) for r in reps]}), {gbs:.0f} GB/s")

    # kernel durations: the same loop with timing events around every launch
    q.qbl_profile_enable(True)
    ms_prof = time_loop(torch, step, args.steps, 0)
    n_gemv, ms_gemv = q.qbl_profile_read(q.KIND_GEMV)
    n_prep, ms_prep = q.qbl_profile_read(q.KIND_PREP)
    q.qbl_profile_enable(False)
    # algorithmic bytes of the 4 batch-1 launches of a step: each reads its
    # linears' quantised base, A and B factors and its input vector once, and
    # writes one output vector (q+k+v and gate+up are written as their sums)
    gemv_bytes_step = sum(group_bytes(wl, g) for g in ([0, 1, 2], [3], [4, 5], [6]))
    launches_per_step = n_gemv / args.steps
    avg_us = ms_gemv / max(n_gemv, 1) * 1e3
    achieved = gemv_bytes_step / launches_per_step / (avg_us * 1e-6) / 1e9
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": counter_traffic("gemv_block7b_q8_r16_counters.md"),
            "kernel": "gemv_b1_kernel (batch-1 launch: glue + LoRA shrink + q8_0 dequant-GEMV + expand)",
            "timing": "HIP events attached to each GEMV dispatch (hipExtLaunchKernelGGL) on the launch stream",
            "launches_per_step": launches_per_step, "avg_launch_us": round(avg_us, 2),
            "bytes_per_launch": int(gemv_bytes_step / launches_per_step),
            "prep_avg_launch_us": round(ms_prep / max(n_prep, 1) * 1e3, 2) if n_prep else None,
            "step_us_with_timing_events": round(ms_prof * 1e3, 1),
            "step_us_repeats": [round(r * 1e3, 2) for r in reps]}
    # the same kernel's average duration from the committed rocprofv3 kernel
    # trace (kernel-only clock, no timing events), while its sources are unchanged
    k_only = profile_field("gemv_block7b_q8_r16_kernel_trace.md", "avg_launch_us")
    roof["rocprof_avg_launch_us"] = k_only
    if k_only:
        roof["rocprof_frac"] = round(gemv_bytes_step / launches_per_step / (k_only * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
    free_all(q, base, ads, comp)
    return wl, blocks, ms, step_bytes, gbs, roof


def cpu_block(oracle, wl, blocks, seconds, threads):
    """GB/s of the oracle's dual path over the block's seven linears, repeated
    (whole linears, at least one) for about `seconds` of wall time."""
    import numpy as np
    xs = [wl.x(i).astype(np.float64) for i in range(7)]
    ads = [[oracle.Lora(wl.lora_a(i, 0), wl.lora_b(i, 0), 1.0)] for i in range(7)]
    done, total_bytes = 0, 0
    t0 = time.time()
    while time.time() - t0 < seconds or done == 0:
        i = done % 7
        L = wl.linears[i]
        oracle.linear_dual(L.qtype, blocks[i], L.n_out, L.k_in, xs[i], ads[i], nthreads=threads)
        total_bytes += linear_bytes(wl, i)
        done += 1
    el = time.time() - t0
    return total_bytes / el / 1e9, done, el


def cpu_baseline(oracle, workloads, wl, seconds):
    """The oracle (float64, C) timed on the host cores, beside the GPU figures:
    the headline leg (the block's linears, GB/s, all cores) and bounded samples of
    the other workloads, each scaled to its line's unit.  Every input is the
    oracle's own (its quantiser on the seeded weights)."""
    import numpy as np
    threads = oracle.default_threads()
    blocks = [oracle.quantize(L.qtype, wl.weight(i)) for i, L in enumerate(wl.linears)]
    gbs, done, el = cpu_block(oracle, wl, blocks, seconds, threads)
    out = {"value": round(gbs, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
           "sample": f"{done} linears of the block (whole linears in order, float64, row-parallel), {el:.1f}s",
           "legs": {}}
    legs = out["legs"]
    short = max(1.0, seconds / 4)

    # the same leg on one core (one thread; the process is pinned to one CPU
    # where the platform allows it)
    pinned = False
    try:
        keep = os.sched_getaffinity(0)
        os.sched_setaffinity(0, {min(keep)})
        pinned = True
    except (AttributeError, OSError):
        keep = None
    try:
        g1, d1, e1 = cpu_block(oracle, wl, blocks, short, 1)
    finally:
        if pinned:
            os.sched_setaffinity(0, keep)
    legs["block_single_core"] = {"value": round(g1, 3), "unit": "GB/s", "cores": 1, "pinned": pinned,
                                 "sample": f"{d1} linears of the block, {e1:.1f}s"}

    # the 32-block stack: the block's base (the stack's block shape) with the
    # stack's two adapters (r16 @ 1.0, r64 @ 0.5), one token at a time, the
    # oracle's block glue included; tokens/s = 1 / (32 x the block's time)
    st = workloads.stack()
    layers = []
    for i in range(7):
        L = st.linears[i]
        ads = [oracle.Lora(st.lora_a(i, a), st.lora_b(i, a), spec.scale) for a, spec in enumerate(st.adapters)]
        layers.append(oracle.Layer(L.qtype, blocks[i], L.n_out, L.k_in, ads))
    h = st.x0()[0].astype(np.float64)
    nblk, t0 = 0, time.time()
    while time.time() - t0 < short or nblk == 0:
        h = oracle.block(layers, h, nthreads=threads)
        nblk += 1
    el = time.time() - t0
    per_tok = el / nblk * st.blocks
    legs["stack"] = {"value": round(1.0 / per_tok, 4), "unit": "tokens/s", "cores": threads,
                     "sample": f"{nblk} block-tokens of the stack's block shape and adapters in {el:.1f}s, "
                               f"scaled by {st.blocks} blocks per token"}

    # the 70B q4_sm MLP at batch 1: the first 1024 rows of gate (the shrink over
    # all of A, the base and B rows of the sample); GB/s over those bytes
    mlp = workloads.mlp70b()
    L = mlp.linears[0]
    rows = 1024
    wq = oracle.quantize(L.qtype, mlp.weight_rows(0, 0, rows))
    A, B = mlp.lora_a(0, 0), mlp.lora_b(0, 0)[:rows].copy()
    x = mlp.x(0, 1).astype(np.float64)
    ad = [oracle.Lora(A, B, mlp.adapters[0].scale)]
    nb = (mlp.base_bytes(0) * rows) // L.n_out + 4 * A.size + 4 * B.size + 4 * (L.k_in + rows)
    n4, t0 = 0, time.time()
    while time.time() - t0 < short or n4 == 0:
        oracle.linear_dual(L.qtype, wq, rows, L.k_in, x, ad, nthreads=threads)
        n4 += 1
    el = time.time() - t0
    legs["q4_mlp_batch1"] = {"value": round(nb * n4 / el / 1e9, 3), "unit": "GB/s", "cores": threads,
                             "sample": f"{n4} passes over rows 0..{rows - 1} of the 28672x8192 q4_sm gate "
                                       f"linear (r32 shrink over all of A), {el:.1f}s"}

    # the prefill JIT recipe: 512 tokens against the first 256 rows of the
    # 14336x4096 layer (W_eff rows materialised, then the bf16 GEMM); GFLOP/s
    # counted as the GPU line counts them (2mnk + 2rnk)
    pf = workloads.prefill()
    L = pf.linears[0]
    rows = 256
    wq = oracle.quantize(L.qtype, pf.weight_rows(0, 0, rows))
    ad = [oracle.Lora(pf.lora_a(0, 0), pf.lora_b(0, 0)[:rows].copy(), pf.adapters[0].scale)]
    X = oracle.bf16_from_f32(pf.x_prefill_f32())
    r = pf.adapters[0].rank
    flop = 2 * pf.m_tokens * rows * L.k_in + 2 * r * rows * L.k_in
    n5, t0 = 0, time.time()
    while time.time() - t0 < short or n5 == 0:
        oracle.linear_jit(L.qtype, wq, rows, L.k_in, X, ad, nthreads=threads)
        n5 += 1
    el = time.time() - t0
    legs["prefill"] = {"value": round(flop * n5 / el / 1e9, 3), "unit": "GFLOP/s", "cores": threads,
                       "sample": f"{n5} passes of {pf.m_tokens} tokens x rows 0..{rows - 1} of the 14336x4096 "
                                 f"q8_0 layer (r64), {el:.1f}s"}
    return out


def bench_single(torch, q, workloads, oracle, args):
    """The 256x256 q8_0 linear with its two rank-8 adapters at 2.0, batch 1:
    microseconds per qbl_linear call (median of repeats), beside the oracle's
    microseconds for the same call on one core."""
    import numpy as np
    wl = workloads.single()
    L = wl.linears[0]
    blocks = q.qbl_quantize(L.qtype, wl.weight(0))
    base = q.qbl_base_load([(L.qtype, L.n_out, L.k_in, blocks)])
    ads = [q.qbl_adapter_load(base, [(0, wl.lora_a(0, a), wl.lora_b(0, a))]) for a in range(2)]
    comp = q.qbl_comp_create(base)
    q.qbl_comp_attach(comp, ads, [a.scale for a in wl.adapters])
    x = torch.from_numpy(wl.x(0, 1)).cuda()
    y = torch.empty((1, L.n_out), dtype=torch.float32, device="cuda")
    ws = q.workspace(comp, q.OP_LINEAR, 0, 1)
    reps = [time_loop(torch, lambda i: q.qbl_linear(comp, 0, x, y, 1, ws), 200, 20) for _ in range(args.repeats)]
    us = sorted(reps)[len(reps) // 2] * 1e3
    free_all(q, base, ads, comp)
    ob = oracle.quantize(L.qtype, wl.weight(0))
    oads = [oracle.Lora(wl.lora_a(0, a), wl.lora_b(0, a), s.scale) for a, s in enumerate(wl.adapters)]
    xo = wl.x(0, 1).astype(np.float64)
    n, t0 = 0, time.time()
    while time.time() - t0 < 0.5 or n < 10:
        oracle.linear_dual(L.qtype, ob, L.n_out, L.k_in, xo, oads, nthreads=1)
        n += 1
    cpu_us = (time.time() - t0) / n * 1e6
    log(f"[single] {us:.2f} us per call (oracle, one core: {cpu_us:.1f} us)")
    return {"us_per_call": round(us, 2), "repeats_us": [round(r * 1e3, 2) for r in reps],
            "bytes": wl.base_bytes(0) + wl.lora_bytes(0) + 4 * (L.n_out + L.k_in),
            "cpu_oracle_us_one_core": round(cpu_us, 1)}


def bench_stack(torch, q, workloads, args):
    wl = workloads.stack(tokens=args.stack_tokens)
    log("[stack] building 32 blocks (6.9 GB q8_0) + r16/r64 adapters")
    t0 = time.time()
    timing = {}
    base, ads, comp, _ = build_copies(q, wl, 1, [0, 1], timing)
    log(f"[stack] built in {time.time() - t0:.1f}s")
    d = 4096
    x0 = torch.from_numpy(wl.x0()[0]).cuda()
    y = torch.empty((wl.tokens, d), dtype=torch.float32, device="cuda")
    ws = q.workspace(comp, q.OP_BLOCK)
    q.qbl_decode(comp, 0, 32, x0, y, 2, ws)       # warm-up
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    q.qbl_decode(comp, 0, 32, x0, y, wl.tokens, ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    tok_s = wl.tokens / (ms * 1e-3)
    per_tok = sum(linear_bytes(wl, i) for i in range(len(wl.linears)))
    h0 = q.qbl_base_hash(base)
    y_ab = y.clone()
    q.qbl_comp_attach(comp, [ads[1], ads[0]], [0.5, 1.0])
    q.qbl_decode(comp, 0, 32, x0, y, wl.tokens, ws)
    torch.cuda.synchronize()
    changed = not torch.equal(y, y_ab)
    t0 = time.time()
    same_hash = q.qbl_base_hash(base) == h0
    hash_s = time.time() - t0
    life = bench_lifecycle(q, base, ads, comp, timing, hash_s)
    free_all(q, base, ads, comp)
    log(f"[stack] {tok_s:.0f} tok/s, order swap changes output: {changed}, hash unchanged: {same_hash}")
    return {"tokens_per_s": round(tok_s, 1), "tokens": wl.tokens, "ms_per_token": round(ms / wl.tokens, 4),
            "GB_per_s": round(per_tok / (ms / wl.tokens * 1e-3) / 1e9, 1),
            "frac_hbm": round(per_tok / (ms / wl.tokens * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "bytes_per_token": per_tok, "order_swap_changes_output": changed,
            "base_hash_unchanged": same_hash, "lifecycle": life}


def bench_lifecycle(q, base, ads, comp, timing, hash_s):
    """Host-side cost of the lifecycle on the 32-block stack (224 linears, two
    adapters): loads with staging, read-back verification and digests; list
    changes (validation + new list + atomic exchange); rollback; the base hash
    re-read from the device."""
    n = 400
    lists = ([ads[0], ads[1]], [1.0, 0.5]), ([ads[1], ads[0]], [0.5, 1.0])
    t0 = time.perf_counter()
    for i in range(n):
        q.qbl_comp_attach(comp, *lists[i % 2])
    attach_us = (time.perf_counter() - t0) / n * 1e6
    t0 = time.perf_counter()
    for _ in range(n):
        q.qbl_comp_rollback(comp)
    rollback_us = (time.perf_counter() - t0) / n * 1e6
    t0 = time.perf_counter()
    for _ in range(n):
        q.qbl_comp_digest(comp)
    digest_us = (time.perf_counter() - t0) / n * 1e6
    q.qbl_comp_attach(comp, *lists[0])
    out = {"base_load_GB_per_s": round(timing["base_bytes"] / timing["base_load_s"] / 1e9, 2),
           "base_bytes": timing["base_bytes"],
           "adapter_load_GB_per_s": round(timing["adapter_bytes"] / timing["adapter_load_s"] / 1e9, 2),
           "adapter_bytes": timing["adapter_bytes"],
           "attach_us": round(attach_us, 1), "rollback_us": round(rollback_us, 1),
           "comp_digest_us": round(digest_us, 2),
           "base_hash_GB_per_s": round(timing["base_bytes"] / hash_s / 1e9, 2)}
    log(f"[lifecycle] {out}")
    return out


def bench_sparse(torch, q, workloads, args):
    """The 7B block with its rank-16 LoRA and a 10%-dense sparse (DARE/CSR) delta
    after it on every linear; weights, factors and deltas rotated over copies."""
    wl = workloads.block_sparse()
    copies = args.copies
    log(f"[sparse] building {copies} copies of one 7B block (q8_0, r16 + 10% sparse delta)")
    t0 = time.time()
    blocks = [q.qbl_quantize(L.qtype, wl.weight(i)) for i, L in enumerate(wl.linears)]
    n = len(wl.linears)
    base = q.qbl_base_load([(L.qtype, L.n_out, L.k_in, blocks[i]) for c in range(copies)
                            for i, L in enumerate(wl.linears)])
    fac = [(wl.lora_a(i, 0), wl.lora_b(i, 0)) for i in range(n)]
    lora = q.qbl_adapter_load(base, [(c * n + i, A, B) for c in range(copies) for i, (A, B) in enumerate(fac)])
    csr = [wl.sparse_csr(i, 1) for i in range(n)]
    sparse = q.qbl_adapter_load_sparse(base, [(c * n + i, *csr[i]) for c in range(copies) for i in range(n)])
    comp = q.qbl_comp_create(base)
    q.qbl_comp_attach(comp, [lora, sparse], [1.0, 1.0])
    log(f"[sparse] built in {time.time() - t0:.1f}s")
    x = torch.from_numpy(wl.x0()[0]).cuda()
    ys = [torch.empty(4096, dtype=torch.float32, device="cuda") for _ in range(copies)]
    ws = q.workspace(comp, q.OP_BLOCK)

    def step(i):
        q.qbl_block(comp, i % copies, x, ys[i % copies], ws)

    ms = time_loop(torch, step, args.steps, args.warmup)
    nnz = sum(int(c[1].size) for c in csr)
    step_bytes = sum(linear_bytes(wl, i) + wl.sparse_bytes(i, int(csr[i][1].size)) for i in range(n))
    gbs = step_bytes / (ms * 1e-3) / 1e9
    q.qbl_comp_free(comp)
    q.qbl_adapter_free(lora)
    q.qbl_adapter_free(sparse)
    q.qbl_base_free(base)
    log(f"[sparse] {ms * 1e3:.1f} us/step, {gbs:.0f} GB/s ({nnz} sparse entries per block)")
    return {"us_per_step": round(ms * 1e3, 1), "GB_per_s": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
            "bytes_per_step": step_bytes, "sparse_entries": nnz, "density": wl.adapters[1].density}


def bench_dar(torch, q, workloads, args):
    """Drift of the dequantize-add-requantize merge that the overlay avoids, on
    two linears of a 7B block (o 4096x4096, gate 11008x4096, q8_0) with the
    stack's adapters A (r16 @ 1.0) and B (r64 @ 0.5): one merge Q(W + A + B),
    the chains Q(Q(W + A) + B) and Q(Q(W + B) + A), and 8 switch cycles
    W <- Q(Q(W + A) - A).  Errors are relative to the exact merged weight (or,
    for the cycles, to the base) and to the adapters' own delta; the overlay's
    figure is 0 by construction (the base bytes never change).  Also the
    requantise kernel's time."""
    import numpy as np
    wl = workloads.stack(n_blocks=1, tokens=1, name="dar_bench")
    lins = [3, 4]
    out = {"linears": {}}
    x_rng = np.random.default_rng(7)

    def load(blocks_list):
        return q.qbl_base_load([(wl.linears[i].qtype, wl.linears[i].n_out, wl.linears[i].k_in, blk)
                                for i, blk in zip(lins, blocks_list)])

    def merge(blocks_list, terms):
        """terms: list of (adapter index, scale) applied in order; one requantisation."""
        base = load(blocks_list)
        ads = [q.qbl_adapter_load(base, [(j, wl.lora_a(i, a), wl.lora_b(i, a)) for j, i in enumerate(lins)])
               for a, _ in terms]
        comp = q.qbl_comp_create(base)
        q.qbl_comp_attach(comp, ads, [s for _, s in terms])
        res = []
        for j, i in enumerate(lins):
            L = wl.linears[i]
            o = torch.empty(L.n_out * L.k_in // 32 * 34, dtype=torch.uint8, device="cuda")
            q.qbl_requantize(comp, j, o)
            torch.cuda.synchronize()
            res.append(o.cpu().numpy().reshape(L.n_out, -1))
        free_all(q, base, ads, comp)
        return res

    base_blocks = [q.qbl_quantize(wl.linears[i].qtype, wl.weight(i)) for i in lins]
    sA, sB = wl.adapters[0].scale, wl.adapters[1].scale
    once = merge(base_blocks, [(0, sA), (1, sB)])
    chain_ab = merge(merge(base_blocks, [(0, sA)]), [(1, sB)])
    chain_ba = merge(merge(base_blocks, [(1, sB)]), [(0, sA)])
    cyc = base_blocks
    for _ in range(8):
        cyc = merge(merge(cyc, [(0, sA)]), [(0, -sA)])

    # kernel time of one requantisation of both linears under A and B
    base = load(base_blocks)
    ads = [q.qbl_adapter_load(base, [(j, wl.lora_a(i, a), wl.lora_b(i, a)) for j, i in enumerate(lins)])
           for a in (0, 1)]
    comp = q.qbl_comp_create(base)
    q.qbl_comp_attach(comp, ads, [sA, sB])
    outs = [torch.empty(wl.linears[i].n_out * wl.linears[i].k_in // 32 * 34, dtype=torch.uint8, device="cuda")
            for i in lins]
    q.qbl_profile_enable(True)
    for _ in range(5):
        for j in range(len(lins)):
            q.qbl_requantize(comp, j, outs[j])
    torch.cuda.synchronize()
    n_dar, ms_dar = q.qbl_profile_read(q.KIND_DAR)
    q.qbl_profile_enable(False)
    free_all(q, base, ads, comp)
    r = sum(a.rank for a in wl.adapters)
    dar_bytes = sum(2 * wl.base_bytes(i) + 4 * r * (wl.linears[i].n_out + wl.linears[i].k_in) for i in lins)
    dar_us = ms_dar / max(n_dar, 1) * len(lins) * 1e3
    out["requantize_us_both_linears"] = round(dar_us, 1)
    out["requantize_GB_per_s"] = round(dar_bytes / (dar_us * 1e-6) / 1e9, 1)

    for j, i in enumerate(lins):
        L = wl.linears[i]
        deq = lambda blk: q.qbl_dequantize(L.qtype, blk, L.n_out, L.k_in).astype(np.float64)
        W0 = deq(base_blocks[j])
        delta = sA * (wl.lora_b(i, 0).astype(np.float64) @ wl.lora_a(i, 0)) + \
            sB * (wl.lora_b(i, 1).astype(np.float64) @ wl.lora_a(i, 1))
        exact = W0 + delta
        nd, ne, n0 = np.linalg.norm(delta), np.linalg.norm(exact), np.linalg.norm(W0)
        rel = lambda blk: float(np.linalg.norm(deq(blk) - exact))
        x = x_rng.standard_normal(L.k_in)
        y_exact = exact @ x
        y_once = deq(once[j]) @ x
        d_old = base_blocks[j].reshape(L.n_out, -1, 34)[:, :, :2].copy().view(np.float16).astype(np.float64)
        d_new = once[j].reshape(L.n_out, -1, 34)[:, :, :2].copy().view(np.float16).astype(np.float64)
        ratio = d_new[d_old > 0] / d_old[d_old > 0]
        codes_old = base_blocks[j].reshape(L.n_out, -1, 34)[:, :, 2:]
        codes_new = once[j].reshape(L.n_out, -1, 34)[:, :, 2:]
        out["linears"][f"{L.n_out}x{L.k_in}"] = {
            "delta_rel_to_weight": round(nd / n0, 5),
            "once_err_rel_weight": round(rel(once[j]) / ne, 6),
            "once_err_rel_delta": round(rel(once[j]) / nd, 4),
            "chain_ab_err_rel_delta": round(rel(chain_ab[j]) / nd, 4),
            "chain_ba_err_rel_delta": round(rel(chain_ba[j]) / nd, 4),
            "chain_orders_bytes_differ": bool(not np.array_equal(chain_ab[j], chain_ba[j])),
            "cycles8_base_drift_rel_weight": round(float(np.linalg.norm(deq(cyc[j]) - W0)) / n0, 6),
            "cycles8_bytes_changed_frac": round(float((cyc[j] != base_blocks[j]).mean()), 4),
            "once_scale_changed_frac": round(float((ratio != 1.0).mean()), 4),
            "once_scale_ratio_max": round(float(ratio.max()), 4),
            "once_codes_changed_frac": round(float((codes_new != codes_old).mean()), 4),
            "once_output_rel_l2": round(float(np.linalg.norm(y_once - y_exact) / np.linalg.norm(y_exact)), 6),
            "overlay_err": 0.0,
        }
        log(f"[dar] {L.n_out}x{L.k_in}: {out['linears'][f'{L.n_out}x{L.k_in}']}")
    log(f"[dar] requantise {dar_us:.1f} us for both linears ({out['requantize_GB_per_s']} GB/s)")
    return out


def bench_q4(torch, q, wl, args, label):
    out = {}
    log(f"[{label}] building 70B MLP linears ({label}, r32)")
    copies = 2  # 2 x 455 MB rotated: well past the 256 MB Infinity Cache
    base, ads, comp, _ = build_copies(q, wl, copies, [0])
    for batch in (1, 8):
        xs = [torch.from_numpy(wl.x(i, batch)).cuda() for i in range(3)]
        ys = [torch.empty((batch, L.n_out), dtype=torch.float32, device="cuda") for L in wl.linears]
        wss = [q.workspace(comp, q.OP_LINEAR, c * 3 + i, batch) for c in range(copies) for i in range(3)]

        def step(s):
            c = s % copies
            for i in range(3):
                q.qbl_linear(comp, c * 3 + i, xs[i], ys[i], batch, wss[c * 3 + i])

        ms = time_loop(torch, step, max(5, args.steps // 2), 2)
        byts = sum(wl.base_bytes(i) + wl.lora_bytes(i) + 4 * batch * (L.n_out + L.k_in)
                   for i, L in enumerate(wl.linears))
        gbs = byts / (ms * 1e-3) / 1e9
        out[f"batch{batch}"] = {"us_per_mlp": round(ms * 1e3, 1), "GB_per_s": round(gbs, 1),
                                "frac_hbm": round(gbs / HBM_PEAK_GBS, 4), "bytes": byts}
        log(f"[{label}] batch {batch}: {ms * 1e3:.1f} us, {gbs:.0f} GB/s")
    free_all(q, base, ads, comp)
    return out


def bench_probe(torch, q, nbytes=4 << 30, reps=20):
    """Achievable HBM read bandwidth: qbl_hbm_probe streaming a 4 GiB buffer
    (16x the 256 MB Infinity Cache) with the batch-1 kernels' 16-byte
    non-temporal loads; median of `reps` timed passes on the current stream."""
    buf = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(4096, dtype=torch.int32, device="cuda")
    for _ in range(3):
        wg = q.qbl_hbm_probe(buf, sink)
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        q.qbl_hbm_probe(buf, sink)
        e1.record()
        e1.synchronize()
        times.append(e0.elapsed_time(e1))
    ms = sorted(times)[reps // 2]
    gbs = nbytes / (ms * 1e-3) / 1e9
    log(f"[probe] read {nbytes >> 20} MiB in {ms * 1e3:.1f} us: {gbs:.0f} GB/s ({wg} workgroups)")
    del buf, sink
    return {"read_GB_per_s": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4), "bytes": nbytes,
            "workgroups": wg, "us_median": round(ms * 1e3, 1), "passes": reps,
            "access": "read-only, 16-byte non-temporal loads from every lane, grid-stride"}


def bench_prefill(torch, q, workloads, args):
    wl = workloads.prefill()
    copies = 10  # 10 x 62 MB base + factors rotated: past the 256 MB Infinity Cache
    log(f"[prefill] building {copies} copies of the 14336x4096 q8_0 layer (r64)")
    base, ads, comp, _ = build_copies(q, wl, copies, [0])
    x = torch.from_numpy(wl.x_prefill_f32()).to(torch.bfloat16).view(torch.int16).cuda()
    y = torch.empty((wl.m_tokens, wl.linears[0].n_out), dtype=torch.float32, device="cuda")
    wss = [q.workspace(comp, q.OP_JIT, c, wl.m_tokens) for c in range(copies)]

    def step(i):
        q.qbl_linear_jit(comp, i % copies, x, y, wl.m_tokens, wss[i % copies])

    ms = time_loop(torch, step, max(10, args.steps // 4), 3)
    L = wl.linears[0]
    r = wl.adapters[0].rank
    flop = 2 * wl.m_tokens * L.n_out * L.k_in + 2 * r * L.n_out * L.k_in
    q.qbl_profile_enable(True)
    time_loop(torch, step, max(10, args.steps // 4), 0)
    n_jit, ms_jit = q.qbl_profile_read(q.KIND_JIT)
    q.qbl_profile_enable(False)
    avg_us = ms_jit / max(n_jit, 1) * 1e3
    tflops = flop / (ms * 1e-3) / 1e12
    kern_tflops = flop / (avg_us * 1e-6) / 1e12
    free_all(q, base, ads, comp)
    log(f"[prefill] {ms * 1e3:.1f} us/layer, {tflops:.0f} TFLOP/s (kernel {kern_tflops:.0f})")
    return {"us_per_layer": round(ms * 1e3, 1), "TFLOP_per_s": round(tflops, 1),
            "kernel_avg_us": round(avg_us, 1), "kernel_TFLOP_per_s": round(kern_tflops, 1),
            "frac_bf16_peak": round(kern_tflops / BF16_PEAK_TFLOPS, 4), "flop_per_layer": flop,
            "tokens_per_s": round(wl.m_tokens / (ms * 1e-3), 1)}


EXTRAS = ("stack", "q4_mlp", "q4k_mlp", "sparse_block", "dar", "prefill")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--copies", type=int, default=4, help="weight copies rotated per step (>= 600 MB)")
    ap.add_argument("--stack-tokens", type=int, default=256)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--repeats", type=int, default=5, help="timed repeats; the median is reported")
    ap.add_argument("--no-extras", action="store_true", help="skip the stack / q4 / prefill lines")
    ap.add_argument("--extras", default=",".join(EXTRAS),
                    help="comma-separated extra lines to run (default: all of " + ",".join(EXTRAS) + ")")
    ap.add_argument("--calib-copy", type=int, default=0, metavar="MIB",
                    help="also run one plain device copy of this many MiB (a known-size kernel "
                         "for scaling hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the path has no multi-GPU part); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import quantized_base_linear_amd as q
    from synth import workloads
    torch.cuda.set_device(0)

    if args.calib_copy:
        n = args.calib_copy * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[calib] copied {args.calib_copy} MiB")
        del src, dst
    wl, blocks, ms, step_bytes, gbs, roof = bench_block(torch, q, workloads, args)
    result = {
        "metric": METRIC, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "q8_0/f32",
        "data": "synthetic (seeded normal weights, adapters and activations)",
        "config": {"workload": "7B-style block, 7 q8_0 linears (4096/11008), rank-16 LoRA at 1.0, batch 1",
                   "batch": 1, "bytes_per_step": step_bytes, "weight_copies_rotated": args.copies,
                   "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)},
        "roofline": roof,
    }
    probe = bench_probe(torch, q)
    roof["achievable_read_GB_per_s"] = probe["read_GB_per_s"]
    roof["frac_of_achievable"] = round(roof["achieved"] / probe["read_GB_per_s"], 4)
    result["hbm_probe"] = probe
    extras = [] if args.no_extras else [e for e in args.extras.split(",") if e]
    for e in extras:
        if e not in EXTRAS:
            print(f"unknown extra line {e!r}; choose from {','.join(EXTRAS)}", file=sys.stderr)
            sys.exit(2)
    runs = {"stack": lambda: bench_stack(torch, q, workloads, args),
            "q4_mlp": lambda: bench_q4(torch, q, workloads.mlp70b(), args, "q4_sm"),
            "q4k_mlp": lambda: bench_q4(torch, q, workloads.mlp70b_q4k(), args, "q4_K"),
            "sparse_block": lambda: bench_sparse(torch, q, workloads, args),
            "dar": lambda: bench_dar(torch, q, workloads, args),
            "prefill": lambda: bench_prefill(torch, q, workloads, args)}
    for e in EXTRAS:
        if e in extras:
            result[e] = runs[e]()
    import oracle
    result["single_linear"] = bench_single(torch, q, workloads, oracle, args)
    log("[cpu] timing the oracle")
    result["cpu_baseline"] = cpu_baseline(oracle, workloads, wl, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
