#!/usr/bin/env python3
"""Benchmark of the paged-KV attention hot path on one MI355X.

A step is one pass of the whole path over one batch of seeded synthetic input:
the host metadata is prepared once (outside the timed region), then each step
stores the new K/V rows (pkv_store) and runs attention (pkv_decode, or
pkv_prefill_varlen for the prefill workload), for every layer of the workload.
Inputs are resident in HBM before timing starts.

The JSON line reports the 28-layer decode step (B=512, H_q=32, H_kv=8, d=128,
block size 256, context lengths log-uniform in [16, 16384], per-layer views of
one [2, 28, blocks, 256, 8, 128] pool): `value` is the step's algorithmic HBM
bytes over its wall time; `roofline` is the per-layer pkv_decode call
(decode_kernel + decode_merge_kernel) against the published HBM peak and
against a measured ceiling (a load-only probe kernel that reads the same pages
in the same pattern); `cpu_baseline` is the float64 oracle on the host cores,
on a bounded sample of the same workload, with its max-abs error against the
GPU outputs.  The single-layer decode workloads, the prefill workloads and the
other steps are reported under "secondary", each decode and prefill workload
with its own roofline, call-time spread and oracle timing.

Timing: the timed region (K steps) brackets every attention call with a pair
of HIP events on the launch stream (torch's current stream, which the library
uses); mean, median, min and max over those calls are reported, the rooflines
use the mean (the average launch duration), and the wall clock
around the whole region gives ms_per_step.

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload NAME]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged decode attn: achieved HBM GB/s & % peak; prefill TFLOP/s; tokens/s"
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PARITY_TOL = 1e-2           # max-abs bar for bf16 attention outputs


# ------------------------------------------------------------ workload arithmetic

def decode_bytes(plan) -> int:
    """Algorithmic bytes one decode call must move: K+V of every context token,
    Q in and O out, context lengths, and the block-table entries read."""
    kv = sum(2 * n * plan.H_kv * plan.d * 2 for n in plan.lens())
    qo = 2 * plan.B * plan.H_q * plan.d * 2
    tbl = 4 * sum(-(-n // plan.block_size) for n in plan.lens())
    return kv + qo + 4 * plan.B + tbl


def kv_bytes(plan) -> int:
    """K+V bytes of every context token: what the load-only probe reads."""
    return sum(2 * n * plan.H_kv * plan.d * 2 for n in plan.lens())


def store_bytes(plan) -> int:
    """K and V rows read and written, plus the slot of every row."""
    n = plan.total_new
    return 2 * n * plan.row_elems * 2 * 2 + 4 * n


def causal_pairs(num_cached: int, num_new: int) -> int:
    """Unmasked (query, key) pairs of one sequence: query i sees keys 0 .. c + i."""
    return num_new * num_cached + num_new * (num_new + 1) // 2


def prefill_flops(plan) -> int:
    """Causal attention flops over unmasked (query, key) pairs: 4 d H_q per pair."""
    pairs = sum(causal_pairs(s.num_cached, s.num_new) for s in plan.seqs)
    return 4 * plan.d * plan.H_q * pairs


def measured_traffic(workload: str):
    """HBM bytes per decode call from the committed PMC record, or None when the
    decode kernel's source has changed since the counters were taken."""
    import hashlib

    rec_path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(rec_path):
        return None
    rec = json.load(open(rec_path)).get(workload)
    if not rec:
        return None
    h = hashlib.sha256()
    for f in ("pkv_decode.hip", "device_common.h", "decode_schedule.h"):
        h.update(open(os.path.join(ROOT, "paged_kv_cache_110_amd", "csrc", f), "rb").read())
    if h.hexdigest() != rec["decode_source_sha256"]:
        return None
    return (rec["fetch_mb_per_call"] + rec["write_mb_per_call"]) * 1e6


# ------------------------------------------------------------------- timing

def spread(ms_list) -> dict:
    """Median, min, max and mean of per-call durations (ms)."""
    return dict(median=round(statistics.median(ms_list), 5), min=round(min(ms_list), 5),
                max=round(max(ms_list), 5), mean=round(statistics.fmean(ms_list), 5),
                n=len(ms_list))


# Secondary workloads warm up for at least this much wall time (besides their
# step count): the device's clocks drop while it idles (during the oracle legs,
# for one) and need some tens of ms of load to come back, so a warm-up of a few
# sub-millisecond calls leaves the first timed calls about 10% slow.
SECONDARY_WARM_S = 0.25


def warm(torch, fn, calls, seconds=0.0):
    """At least `calls` untimed calls fn(i), and more until `seconds` of wall
    time have passed (synchronising every 8 calls past the minimum, so the wall
    time follows the device's); returns how many ran."""
    t0 = time.perf_counter()
    i = 0
    while i < calls or time.perf_counter() - t0 < seconds:
        fn(i)
        i += 1
        if i >= calls and i % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return i


def timed_calls(torch, fn, n):
    """n calls fn(i), each between its own pair of HIP events on the current
    stream; returns the per-call durations (ms)."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    for i, (a, b) in enumerate(ev):
        a.record()
        fn(i)
        b.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


# ----------------------------------------------------------------- ceilings

def measure_ceilings(torch, probe, log, gib: float = 4.0, runs: int = 10) -> dict:
    """What the device sustains with hand-written probe kernels: a streaming
    read of a buffer of known size with plain loads and with non-temporal ones
    (the form the decode's K/V loads take), a plain copy, and the dense MFMA
    issue rate (bf16 and fp16 32x32x16, register operands) at the best of a
    few occupancies."""
    n = int(gib * (1 << 30))
    src = torch.empty(n // 2, dtype=torch.bfloat16, device="cuda").normal_()
    dst = torch.empty_like(src)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    res = {}
    for _ in range(2):
        probe.read(src, sink)
        probe.read(src, sink, nontemporal=True)
        probe.copy(dst, src)
    rd = timed_calls(torch, lambda i: probe.read(src, sink), runs)
    rdn = timed_calls(torch, lambda i: probe.read(src, sink, nontemporal=True), runs)
    cp = timed_calls(torch, lambda i: probe.copy(dst, src), runs)
    res["read"] = dict(kernel="read_kernel<plain loads> (libpkv_probe)", bytes=n, ms=spread(rd),
                       gb_per_s=round(n / statistics.fmean(rd) / 1e6, 1))
    res["read_nt"] = dict(kernel="read_kernel<non-temporal loads> (libpkv_probe)", bytes=n,
                          ms=spread(rdn), gb_per_s=round(n / statistics.fmean(rdn) / 1e6, 1))
    res["copy"] = dict(kernel="copy_kernel (libpkv_probe)", bytes=2 * n, ms=spread(cp),
                       gb_per_s=round(2 * n / statistics.fmean(cp) / 1e6, 1))
    del src, dst
    torch.cuda.empty_cache()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    msink = torch.zeros(cus * 4 * 8, dtype=torch.float32, device="cuda")
    for name, f16 in (("mfma_bf16", False), ("mfma_f16", True)):
        best = None
        for waves, chains in ((1, 4), (2, 4), (2, 8), (4, 4)):
            iters = 2000
            probe.mfma(msink, cus, waves, iters, chains, f16)
            ms = timed_calls(torch, lambda i: probe.mfma(msink, cus, waves, iters, chains, f16), 5)
            flops = cus * 4 * waves * iters * chains * 32768
            tf = flops / (statistics.fmean(ms) * 1e-3) / 1e12
            if best is None or tf > best["tflops"]:
                best = dict(kernel=f"mfma_kernel ({'f16' if f16 else 'bf16'} 32x32x16, libpkv_probe)",
                            tflops=round(tf, 1), waves_per_simd=waves, chains=chains,
                            flops=flops, ms=spread(ms))
        res[name] = best
    log(f"ceilings: read {res['read']['gb_per_s']} GB/s (non-temporal {res['read_nt']['gb_per_s']}), "
        f"copy {res['copy']['gb_per_s']} GB/s, "
        f"bf16 MFMA {res['mfma_bf16']['tflops']} TFLOP/s, f16 MFMA {res['mfma_f16']['tflops']} TFLOP/s")
    return res


def paged_read_ceiling(torch, probe, plan, meta, views, runs: int = 20,
                       group_heads: bool = False) -> dict:
    """The load-only probe over the same pages as the decode (same tables and
    lengths, the same non-temporal loads), rotating over the given (k_cache,
    v_cache) views so consecutive runs do not find their bytes in the
    last-level cache.  group_heads: the H_kv heads of a page read by one
    workgroup together instead of one workgroup per (page, head)."""
    from paged_kv_cache_110_amd.probe import pages_of

    pages = pages_of(meta["block_tables"], meta["context_lens"], plan.block_size).to("cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")

    def run(i):
        kc, vc = views[i % len(views)]
        probe.paged_read(kc, vc, pages, sink, nontemporal=True, group_heads=group_heads)

    for i in range(2):
        run(i)
    ms = timed_calls(torch, run, runs)
    nbytes = kv_bytes(plan)
    form = "heads of a page together" if group_heads else "one workgroup per (page, head)"
    return dict(kernel=f"paged_read_kernel<non-temporal loads, {form}> (libpkv_probe)", bytes=nbytes,
                ms=spread(ms),
                gb_per_s=round(nbytes / statistics.fmean(ms) / 1e6, 1),
                pages=int(pages.shape[0]))


# ------------------------------------------------------------ the oracle leg

def _errors(got, ref, tol=PARITY_TOL):
    err = (got.double() - ref).abs()
    return (err.max().item() if err.numel() else 0.0), int((err > tol).sum())


def oracle_decode_leg(plan, tens, outs, budget_s, log) -> dict:
    """The float64 oracle, as it stands, on host copies of the same inputs:
    store + decode of every sequence, one (pool, layer) unit at a time until
    about budget_s of oracle compute (each unit at least once for a
    single-layer workload; layers in order for the multi-layer one).  The
    device-to-host copy time is counted apart.  Each unit's oracle output is
    compared with the GPU output of the same unit from the timed steps."""
    import oracle as O

    orc = O.default()
    om = O.prepare_decode(plan.seqs, plan.block_size, plan.max_blocks_per_seq)
    scale = 1.0 / math.sqrt(plan.d)
    units = [(r, l) for l in range(plan.layers) for r in range(len(tens))]
    compute_s = d2h_s = 0.0
    done, max_err, over, values = 0, 0.0, 0, 0
    host = {}
    while done < len(units) or compute_s < budget_s:
        r, l = units[done % len(units)]
        if (r, l) not in host:
            t0 = time.perf_counter()
            t = tens[r]
            h = (t.k_cache(l).cpu(), t.v_cache(l).cpu(), t.q[l].cpu(), t.k_new(l).cpu(),
                 t.v_new(l).cpu(), outs[(r, l)].cpu())
            d2h_s += time.perf_counter() - t0
            if plan.layers == 1:
                host[(r, l)] = h  # small: kept for repeats
        else:
            h = host[(r, l)]
        kc, vc, q, kn, vn, got = h
        t0 = time.perf_counter()
        orc.store(kc, vc, kn, vn, om["slot_mapping"])
        ref = orc.decode(q, kc, vc, om["block_tables"], om["context_lens"], scale)
        compute_s += time.perf_counter() - t0
        e, o = _errors(got, ref)
        max_err, over, values = max(max_err, e), over + o, values + ref.numel()
        done += 1
        del h, kc, vc, q, kn, vn, got, ref
        if plan.layers > 1 and (compute_s >= budget_s or done == len(units)):
            break
    per_unit = compute_s / done
    gbs = (decode_bytes(plan) + store_bytes(plan)) / per_unit / 1e9
    what = (f"{done} of the {plan.layers} layers" if plan.layers > 1 else
            f"{done} runs over {len(units)} independent input set(s)")
    log(f"cpu oracle {plan.name}: {what}, {per_unit * 1e3:.1f} ms per layer step, "
        f"{orc.threads()} threads, max abs err {max_err:.3e}")
    return dict(value=round(gbs, 3), unit="GB/s", cores=orc.threads(), kind="oracle",
                sample=f"{plan.name}: store + decode of all {plan.B} sequences, {what}; float64 C "
                       f"oracle (OpenMP), {per_unit * 1e3:.1f} ms per layer",
                ms_per_layer=round(per_unit * 1e3, 2), compute_s=round(compute_s, 2),
                d2h_s=round(d2h_s, 2), layers_checked=done if plan.layers > 1 else 1,
                max_abs_err=max_err, values_compared=values, values_over_tol=over,
                gpu_speedup=None)


def oracle_prefill_leg(plan, tens, outs, budget_s, log, tail: int = 64) -> dict:
    """The oracle's prefill over a stated subset: the last ``tail`` query rows
    of every sequence, as a prefill chunk behind everything before them (the
    rows that attend the most keys), repeated up to about budget_s and
    compared with the GPU's rows for those positions."""
    import oracle as O

    orc = O.default()
    om = O.prepare_prefill(plan.seqs, plan.block_size, plan.max_blocks_per_seq)
    scale = 1.0 / math.sqrt(plan.d)
    cu = om["cu_seqlens_q"]
    rows, cq, ck, pairs = [], [0], [0], 0
    for b, s in enumerate(plan.seqs):
        k = min(tail, s.num_new)
        rows.extend(range(cu[b + 1] - k, cu[b + 1]))
        cq.append(cq[-1] + k)
        ck.append(ck[-1] + s.total)
        pairs += causal_pairs(s.total - k, k)
    fl = 4 * plan.d * plan.H_q * pairs
    t0 = time.perf_counter()
    t = tens[0]
    kc, vc = t.k_cache().cpu(), t.v_cache().cpu()
    q = t.q[0].cpu()[rows].contiguous()
    got = outs[(0, 0)].cpu()[rows]
    d2h_s = time.perf_counter() - t0
    reps, compute_s = 0, 0.0
    while reps == 0 or compute_s < budget_s:
        t0 = time.perf_counter()
        ref = orc.prefill(q, kc, vc, om["block_tables"], cq, ck, scale)
        compute_s += time.perf_counter() - t0
        reps += 1
    per = compute_s / reps
    max_err, over = _errors(got, ref)
    log(f"cpu oracle {plan.name}: last {tail} rows of each sequence, {per:.2f} s per pass, "
        f"{orc.threads()} threads, max abs err {max_err:.3e}")
    return dict(value=round(fl / per / 1e12, 5), unit="TFLOP/s", cores=orc.threads(), kind="oracle",
                sample=f"{plan.name}: prefill of the last {tail} query rows of each of the {plan.B} "
                       f"sequences behind their full context ({len(rows)} rows, {fl / 1e9:.1f} "
                       f"GFLOP), {reps} pass(es); float64 C oracle",
                s_per_pass=round(per, 3), compute_s=round(compute_s, 2), d2h_s=round(d2h_s, 2),
                max_abs_err=max_err, values_compared=ref.numel(), values_over_tol=over)


# ------------------------------------------------------------ attention workloads

def run_workload(name, steps, warmup, pools, torch, pkv, probe, log, cpu_budget=None, warm_s=0.0):
    """Timed steps of one named workload, the probe ceiling over the same
    pages (decode), and the oracle leg (cpu_budget seconds, None = skipped).
    Warm-up: `warmup` steps, continued until `warm_s` seconds have passed."""
    from workloads import make_plan, make_tensors

    plan = make_plan(name)
    dev = "cuda"
    t0 = time.time()
    tens = [make_tensors(plan, dev, poison=False, seed=plan.seed + 17 * r) for r in range(pools)]
    meta = pkv.prepare_metadata(plan.seqs, plan.block_size, plan.max_blocks_per_seq)
    dm = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in meta.items()}
    scale = 1.0 / math.sqrt(plan.d)
    L = plan.layers
    ws = None
    if plan.kind == "decode":
        nbytes = pkv.decode_workspace_size(plan.B, plan.H_q, plan.H_kv, plan.d, plan.block_size,
                                           plan.max_blocks_per_seq)
        ws = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=dev)
    outs = {(r, l): torch.empty_like(tens[r].q[l]) for r in range(pools) for l in range(L)}
    torch.cuda.synchronize()
    log(f"{name}: inputs ready in {time.time() - t0:.1f}s ({plan.B} seqs, {plan.num_blocks} blocks,"
        f" {L} layer(s), {pools} pool(s))")

    def store(i, layer):
        t = tens[i % pools]
        pkv.store(t.k_new(layer), t.v_new(layer), t.k_cache(layer), t.v_cache(layer),
                  dm["slot_mapping"])

    def attention(i, layer):
        t = tens[i % pools]
        kc, vc = t.k_cache(layer), t.v_cache(layer)
        out = outs[(i % pools, layer)]
        if plan.kind == "decode":
            pkv.decode(t.q[layer], kc, vc, dm["block_tables"], dm["context_lens"], scale,
                       out=out, workspace=ws)
        else:
            pkv.prefill_varlen(t.q[layer], kc, vc, dm["block_tables"], dm["cu_seqlens_q"],
                               dm["cu_seqlens_k"], dm["max_seqlen_q"], dm["max_seqlen_k"], scale,
                               out=out)

    def step(i):
        for layer in range(L):
            store(i, layer)
            attention(i, layer)

    warm_steps = warm(torch, step, warmup, warm_s)
    # the timed region: whole steps; a pair of HIP events around every attention call
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps * L)]
    start = time.perf_counter()
    for i in range(steps):
        for layer in range(L):
            store(i, layer)
            a, b = ev[i * L + layer]
            a.record()
            attention(i, layer)
            b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - start
    call_ms = [a.elapsed_time(b) for a, b in ev]
    ms_step = wall * 1e3 / steps
    res = dict(plan=plan, ms_per_step=ms_step, call=spread(call_ms), warmup_steps=warm_steps)
    if plan.kind == "decode":
        views = [(t.k_cache(l), t.v_cache(l)) for l in range(L) for t in tens]
        res["read_ceiling"] = paged_read_ceiling(torch, probe, plan, meta, views)
        res["read_ceiling_grouped"] = paged_read_ceiling(torch, probe, plan, meta, views,
                                                         group_heads=plan.H_kv <= 16)
    if cpu_budget is not None:
        leg = oracle_decode_leg if plan.kind == "decode" else oracle_prefill_leg
        res["cpu"] = leg(plan, tens, outs, cpu_budget, log)
    del tens, ws, outs
    torch.cuda.empty_cache()
    return res


def summarize(res, ceilings) -> dict:
    """The figures of one attention workload: step throughput, the attention
    call against its roofline (published peak and measured ceiling), and the
    oracle leg."""
    plan = res["plan"]
    call = res["call"]
    mean_s = call["mean"] * 1e-3  # the average launch duration
    out = dict(workload=plan.name, layers=plan.layers, ms_per_step=round(res["ms_per_step"], 4),
               attn_call_ms=call, warmup_steps=res["warmup_steps"])
    if plan.kind == "decode":
        per_call = decode_bytes(plan)
        per_step = (per_call + store_bytes(plan)) * plan.layers
        achieved = per_call / mean_s / 1e9
        rc = res["read_ceiling"]
        rg = res["read_ceiling_grouped"]
        out.update(
            gb_per_s=round(per_step / (res["ms_per_step"] * 1e-3) / 1e9, 2),
            tokens_per_s=round(plan.B / (res["ms_per_step"] * 1e-3), 1),
            kv_tokens_per_layer=plan.kv_tokens(),
            roofline=dict(bound="hbm", kernel=f"pkv_decode call (decode_kernel<{plan.d},"
                                              f"{plan.H_q // plan.H_kv},...> + decode_merge_kernel)",
                          achieved=round(achieved, 2), peak=HBM_PEAK_GBS, unit="GB/s",
                          frac=round(achieved / HBM_PEAK_GBS, 4), bytes_per_launch=per_call,
                          read_ceiling=rc["gb_per_s"],
                          frac_of_read_ceiling=round(achieved / rc["gb_per_s"], 4),
                          read_ceiling_probe=rc,
                          read_ceiling_heads_together=rg["gb_per_s"],
                          frac_of_read_ceiling_heads_together=round(achieved / rg["gb_per_s"], 4)))
        traffic = measured_traffic(plan.name)
        out["roofline"].update(
            traffic=None if traffic is None else round(traffic),
            traffic_unit="HBM bytes per call: FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0 (factors from the "
                         "probe copy kernel), profiles/traffic.json; null when unmeasured or when the "
                         "decode source changed since")
    else:
        fl = prefill_flops(plan)
        achieved = fl / mean_s / 1e12
        mc = ceilings["mfma_bf16"]["tflops"] if ceilings else None
        out.update(
            tokens_per_s=round(plan.total_new / (res["ms_per_step"] * 1e-3), 1),
            roofline=dict(bound="mfma", kernel="prefill_kernel<128,2,4,true>",
                          achieved=round(achieved, 2), peak=BF16_PEAK_TFLOPS, unit="TFLOP/s",
                          frac=round(achieved / BF16_PEAK_TFLOPS, 4), flops_per_launch=fl,
                          mfma_ceiling=mc,
                          frac_of_mfma_ceiling=None if mc is None else round(achieved / mc, 4)))
    if "cpu" in res:
        cpu = dict(res["cpu"])
        if plan.kind == "decode":
            cpu["gpu_speedup"] = round(out["roofline"]["achieved"] / cpu["value"], 1)
        else:
            cpu["gpu_speedup"] = round(achieved / cpu["value"], 1)
        out["cpu_oracle"] = cpu
    return out


def run_packed(steps, warmup, torch, pkv, log, ceilings):
    """Varlen causal prefill over packed K/V (no block table, no prefix): q/k/v
    are row views of one fused projection buffer."""
    from workloads.packed import PACKED_PREFILL as cfg, make_packed, split_fused

    lens, cu, fused = make_packed("cuda")
    q, k, v = split_fused(fused)
    out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    scale = 1.0 / math.sqrt(cfg["d"])
    mx = max(lens)
    warm(torch, lambda i: pkv.prefill_varlen_packed(q, k, v, cu, cu, mx, mx, scale, out=out),
         warmup, SECONDARY_WARM_S)
    ms = timed_calls(torch, lambda i: pkv.prefill_varlen_packed(q, k, v, cu, cu, mx, mx, scale,
                                                                out=out), steps)
    mean = statistics.fmean(ms)
    fl = 4 * cfg["d"] * cfg["H_q"] * sum(causal_pairs(0, n) for n in lens)
    tf = fl / (mean * 1e-3) / 1e12
    mc = ceilings["mfma_bf16"]["tflops"] if ceilings else None
    return dict(workload="packed_prefill", B=cfg["B"], tokens=sum(lens), attn_call_ms=spread(ms),
                tokens_per_s=round(sum(lens) / (mean * 1e-3), 1),
                roofline=dict(bound="mfma", kernel="prefill_kernel<128,2,4,false>",
                              achieved=round(tf, 2), peak=BF16_PEAK_TFLOPS, unit="TFLOP/s",
                              frac=round(tf / BF16_PEAK_TFLOPS, 4), flops_per_launch=fl,
                              mfma_ceiling=mc,
                              frac_of_mfma_ceiling=None if mc is None else round(tf / mc, 4)))


def run_graph(steps, warmup, torch, pkv, log):
    """28-layer decode step (store + decode per layer) at small batches, three
    ways: eager calls from Python, the same launches issued by the library
    (pkv_decode_step_run), and the bucketed graph replay (pkv_decode_graph_replay,
    which pads to the bucket).  Wall time per step over `steps` back-to-back
    steps, synchronised at both ends."""
    from workloads import make_tensors
    from workloads.graph import GRAPH_DECODE as cfg, graph_plan

    plan = graph_plan()
    L, mb = cfg["layers"], cfg["max_batch"]
    tens = make_tensors(plan, "cuda", poison=False)
    meta = pkv.prepare_metadata(plan.seqs, plan.block_size, plan.max_blocks_per_seq)
    dm = {k: (v.to("cuda") if isinstance(v, torch.Tensor) else v) for k, v in meta.items()}
    graph = pkv.DecodeGraph([tens.k_cache(l) for l in range(L)], [tens.v_cache(l) for l in range(L)],
                            mb, plan.H_q, plan.max_blocks_per_seq)
    scale = 1.0 / math.sqrt(plan.d)
    ws = torch.zeros(pkv.decode_workspace_size(mb, plan.H_q, plan.H_kv, plan.d, plan.block_size,
                                               plan.max_blocks_per_seq),
                     dtype=torch.uint8, device="cuda")
    res = dict(workload="graph_decode", layers=L, H_q=plan.H_q, H_kv=plan.H_kv, d=plan.d,
               block_size=plan.block_size, context=list(cfg["context"]), batches={})
    for batch in cfg["batches"]:
        graph.slot_mapping[:batch].copy_(dm["slot_mapping"][:batch])
        graph.context_lens[:batch].copy_(dm["context_lens"][:batch])
        graph.block_tables[:batch].copy_(dm["block_tables"][:batch])
        graph.q[:, :batch].copy_(tens.q[:, :batch])
        graph.kv_new[:, :batch].copy_(tens.kv_new[:, :batch])
        sl, cl, bt = (dm["slot_mapping"][:batch], dm["context_lens"][:batch],
                      dm["block_tables"][:batch])
        outs = [torch.empty_like(tens.q[l][:batch]) for l in range(L)]

        def eager_py():
            for l in range(L):
                kc, vc = tens.k_cache(l), tens.v_cache(l)
                pkv.store(tens.k_new(l)[:batch], tens.v_new(l)[:batch], kc, vc, sl)
                pkv.decode(tens.q[l][:batch], kc, vc, bt, cl, scale, out=outs[l], workspace=ws)

        def timed(fn):
            warm(torch, lambda i: fn(), warmup, SECONDARY_WARM_S)
            t0 = time.perf_counter()
            for _ in range(steps):
                fn()
            torch.cuda.synchronize()
            return (time.perf_counter() - t0) * 1e3 / steps

        row = dict(bucket=graph.bucket(batch),
                   eager_python_ms=round(timed(eager_py), 4),
                   eager_native_ms=round(timed(lambda: graph.run_eager(batch)), 4),
                   graph_ms=round(timed(lambda: graph.replay(batch)), 4))
        kv = sum(2 * s.total * plan.H_kv * plan.d * 2 for s in plan.seqs[:batch]) * L
        row["graph_kv_gb_per_s"] = round(kv / (row["graph_ms"] * 1e-3) / 1e9, 2)
        row["speedup_vs_eager_python"] = round(row["eager_python_ms"] / row["graph_ms"], 3)
        res["batches"][str(batch)] = row
        log(f"graph_decode batch {batch}: {json.dumps(row)}")
    graph.close()
    del tens, ws
    torch.cuda.empty_cache()
    return res


def run_meta(steps, warmup, torch, pkv, log):
    """Step metadata two ways on the decode and prefill workloads: the host
    routine (pkv_prepare_metadata through the binding) plus pinned copies to the
    device, against one kernel (pkv_prepare_metadata_device) that derives it
    from request state kept on the device.  Wall time per step, synchronised;
    the device call's figure is the binding's per-call host time, since the
    kernel itself is shorter."""
    from workloads import make_plan

    res = {}
    for name in ("qwen3_decode", "prefix_prefill"):
        plan = make_plan(name)
        bs, maxb, B = plan.block_size, plan.max_blocks_per_seq, plan.B
        hm = pkv.prepare_metadata(plan.seqs, bs, maxb)
        table = hm["block_tables"].to("cuda")
        computed = torch.tensor([s.num_cached for s in plan.seqs], dtype=torch.int32, device="cuda")
        sched = torch.tensor([s.num_new for s in plan.seqs], dtype=torch.int32, device="cuda")
        total = plan.total_new
        bufs = pkv.prepare_metadata_device(None, computed, sched, table, bs, maxb, total)

        def host():
            m = pkv.prepare_metadata(plan.seqs, bs, maxb)
            for k in ("slot_mapping", "context_lens", "cu_seqlens_q", "cu_seqlens_k", "block_tables"):
                m[k].pin_memory().to("cuda", non_blocking=True)

        def device():
            pkv.prepare_metadata_device(None, computed, sched, table, bs, maxb, total, out=bufs)

        def wall(fn):
            warm(torch, lambda i: fn(), warmup, SECONDARY_WARM_S)
            t0 = time.perf_counter()
            for _ in range(steps):
                fn()
            torch.cuda.synchronize()
            return (time.perf_counter() - t0) * 1e3 / steps

        out_bytes = 4 * (2 * (B + 1) + B + total + B * maxb + 2) + 8 * total
        in_bytes = 4 * (2 * B) + 4 * sum(-(-s.total // bs) for s in plan.seqs)
        row = dict(B=B, new_tokens=total, host_ms=round(wall(host), 4),
                   device_call_ms=round(wall(device), 4), bytes=out_bytes + in_bytes)
        res[name] = row
        log(f"device_metadata {name}: {json.dumps(row)}")
    return dict(workload="device_metadata", **res)


def run_sample(steps, warmup, torch, pkv, log):
    """Gumbel-max sampling of one decode step: 256 rows of bf16 logits over a
    151936-token vocabulary (pkv_sample_gumbel, both launches), a pair of HIP
    events on the launch stream around every call."""
    from workloads.sampling import SAMPLE_DECODE as cfg, make_logits

    logits, temps, seeds, offsets = make_logits("cuda")
    out = torch.empty(cfg["B"], dtype=torch.int64, device="cuda")
    ws = torch.empty(pkv.sample_workspace_size(cfg["B"], cfg["V"]), dtype=torch.uint8, device="cuda")
    step_offsets = [offsets + i for i in range(steps)]  # a fresh draw per step
    warm(torch, lambda i: pkv.sample_gumbel(logits, seeds, temps, offsets, out=out, workspace=ws),
         warmup, SECONDARY_WARM_S)
    calls = timed_calls(torch, lambda i: pkv.sample_gumbel(logits, seeds, temps, step_offsets[i],
                                                           out=out, workspace=ws), steps)
    ms = statistics.fmean(calls)
    n = cfg["B"] * cfg["V"]
    nbytes = 2 * n + cfg["B"] * (4 + 8 + 8 + 8)
    res = dict(workload="gumbel_sample", B=cfg["B"], V=cfg["V"], dtype="bf16", bound="alu",
               ms=round(ms, 4), call_ms=spread(calls),
               logits_per_s=round(n / (ms * 1e-3), 1), gb_per_s=round(nbytes / (ms * 1e-3) / 1e9, 2),
               pct_hbm_peak=round(100 * nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2))
    log(f"gumbel_sample: {json.dumps(res)}")
    return res


SECONDARY = ("qwen3_decode", "long_decode", "wide_gqa_decode", "prefix_prefill", "packed_prefill",
             "graph_decode", "device_metadata", "gumbel_sample")
ATTENTION = ("full_step", "qwen3_decode", "long_decode", "wide_gqa_decode", "prefix_prefill")


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="full_step", choices=list(ATTENTION))
    ap.add_argument("--pools", type=int, default=2,
                    help="independent copies of the cache rotated across steps (single-layer workloads)")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--secondary", default="all",
                    help="comma-separated secondary workloads to run (default: all of "
                         + ", ".join(SECONDARY) + ")")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0,
                    help="seconds of oracle compute for the headline workload's cpu_baseline")
    ap.add_argument("--cpu-budget-secondary", type=float, default=2.0,
                    help="seconds of oracle compute for each secondary attention workload")
    ap.add_argument("--probes-only", action="store_true",
                    help="only run the ceiling probes and print their JSON")
    args = ap.parse_args()

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}): the benchmark measures the "
              "path on one GPU and has no multi-GPU mode", file=sys.stderr)
        return 2

    import torch

    import paged_kv_cache_110_amd as pkv
    from paged_kv_cache_110_amd import probe

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    pkv._lib.load()
    probe.load()
    ceilings = measure_ceilings(torch, probe, log)
    if args.probes_only:
        print(json.dumps(dict(ceilings=ceilings)), flush=True)
        return 0

    wanted = set() if args.no_secondary else (
        set(SECONDARY) if args.secondary == "all" else set(args.secondary.split(",")))
    unknown = wanted - set(SECONDARY)
    if unknown:
        print(f"unknown secondary workloads: {sorted(unknown)}", file=sys.stderr)
        return 2

    def pools_of(name):
        return 1 if name in ("full_step", "prefix_prefill") else args.pools

    cpu_b = None if args.no_cpu_baseline else args.cpu_budget
    main_res = run_workload(args.workload, args.steps, args.warmup, pools_of(args.workload), torch,
                            pkv, probe, log, cpu_budget=cpu_b)
    plan = main_res["plan"]
    s = summarize(main_res, ceilings)
    log(json.dumps({k: v for k, v in s.items() if k != "roofline"}))

    secondary = {}
    n2 = max(5, args.steps)
    cpu2 = None if args.no_cpu_baseline else args.cpu_budget_secondary
    for name in ATTENTION:
        if name == args.workload or name not in wanted:
            continue
        r = run_workload(name, n2, 2, pools_of(name), torch, pkv, probe, log, cpu_budget=cpu2,
                         warm_s=SECONDARY_WARM_S)
        secondary[name] = summarize(r, ceilings)
        log(json.dumps(secondary[name]))
    if "packed_prefill" in wanted:
        secondary["packed_prefill"] = run_packed(n2, 2, torch, pkv, log, ceilings)
        log(json.dumps(secondary["packed_prefill"]))
    if "graph_decode" in wanted:
        secondary["graph_decode"] = run_graph(n2, 3, torch, pkv, log)
    if "device_metadata" in wanted:
        secondary["device_metadata"] = run_meta(n2, 3, torch, pkv, log)
    if "gumbel_sample" in wanted:
        secondary["gumbel_sample"] = run_sample(n2, 3, torch, pkv, log)

    roofline = dict(s["roofline"])
    if plan.kind == "decode":
        value, unit = s["gb_per_s"], "GB/s"
        roofline.update(
            avg_launch_ms=s["attn_call_ms"]["mean"], launch_ms=s["attn_call_ms"],
            copy_ceiling=ceilings["copy"]["gb_per_s"], plain_read_ceiling=ceilings["read"]["gb_per_s"],
            nontemporal_read_ceiling=ceilings["read_nt"]["gb_per_s"])
    else:
        value, unit = s["roofline"]["achieved"], "TFLOP/s"
        roofline.update(traffic=None, avg_launch_ms=s["attn_call_ms"]["mean"],
                        launch_ms=s["attn_call_ms"])
    cpu = None
    if "cpu_oracle" in s:
        cpu = s["cpu_oracle"]

    config = dict(workload=plan.name, B=plan.B, H_q=plan.H_q, H_kv=plan.H_kv, d=plan.d,
                  block_size=plan.block_size, layers=plan.layers, num_blocks=plan.num_blocks,
                  kv_tokens=plan.kv_tokens(), new_tokens=plan.total_new,
                  pools_rotated=pools_of(plan.name),
                  step="store + attention" + (" per layer" if plan.layers > 1 else ""))
    detail = {k: v for k, v in s.items() if k not in ("roofline", "cpu_oracle")}
    line = dict(metric=METRIC, value=value, unit=unit, n_gpus=1, steps=args.steps,
                warmup=args.warmup, ms_per_step=s["ms_per_step"], higher_is_better=True,
                scaling="weak", vs_baseline=None, dtype="bf16", data="synthetic",
                config=config, roofline=roofline, cpu_baseline=cpu, detail=detail,
                ceilings=ceilings, secondary=secondary)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
