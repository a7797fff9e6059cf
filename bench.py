#!/usr/bin/env python3
"""Benchmark of the paged-KV attention hot path on one MI355X.

A step is one pass of the whole path over one batch of seeded synthetic input:
the host metadata is prepared once (outside the timed region), then each step
stores the new K/V rows (pkv_store) and runs attention (pkv_decode, or
pkv_prefill_varlen for the prefill workload); the 28-layer workload does both
for every layer.  Inputs are resident in HBM before timing starts.

The JSON line reports the Qwen3-0.6B-shaped decode workload (B=256, H_q=16,
H_kv=8, d=128, block size 256, context lengths U[128, 2048]) with its decode
roofline (achieved algorithmic HBM bytes per decode call / the call's average
duration) and the CPU oracle timed on a bounded sample.  The other workloads
are reported under "secondary".

Timing: the timed region (K steps) holds no events, only the library calls,
bracketed by synchronisations and the wall clock.  Per-call durations come
from the same calls run back to back right after it, with one pair of HIP
events on the launch stream around each run (events recorded between calls
add their own gaps to what they measure).

Usage: python bench.py [--gpus 1] [--steps 100] [--warmup 20] [--workload NAME]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged decode attn: achieved HBM GB/s & % peak; prefill TFLOP/s; tokens/s"
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published


# ------------------------------------------------------------ workload arithmetic

def decode_bytes(plan) -> int:
    """Algorithmic bytes one decode call must move: K+V of every context token,
    Q in and O out, context lengths, and the block-table entries read."""
    kv = sum(2 * n * plan.H_kv * plan.d * 2 for n in plan.lens())
    qo = 2 * plan.B * plan.H_q * plan.d * 2
    tbl = 4 * sum(-(-n // plan.block_size) for n in plan.lens())
    return kv + qo + 4 * plan.B + tbl


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

def events_ms(torch, fn, n):
    """Average duration of n back-to-back calls fn(i), from one pair of HIP events on
    the current stream (the stream the library launches on)."""
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(n):
        fn(i)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n


def run_workload(name, steps, warmup, pools, torch, pkv, log):
    from workloads import make_plan, make_tensors

    plan = make_plan(name)
    dev = "cuda"
    t0 = time.time()
    tens = [make_tensors(plan, dev, poison=False, seed=plan.seed + 17 * r) for r in range(pools)]
    meta = pkv.prepare_metadata(plan.seqs, plan.block_size, plan.max_blocks_per_seq)
    dm = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in meta.items()}
    scale = 1.0 / math.sqrt(plan.d)
    ws = None
    if plan.kind == "decode":
        nbytes = pkv.decode_workspace_size(plan.B, plan.H_q, plan.H_kv, plan.d, plan.block_size,
                                           plan.max_blocks_per_seq)
        ws = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=dev)
        outs = [torch.empty_like(t.q[0]) for t in tens]
    torch.cuda.synchronize()
    log(f"{name}: inputs ready in {time.time() - t0:.1f}s ({plan.B} seqs, {plan.num_blocks} blocks,"
        f" {pools} pool(s))")

    def store(i, layer):
        t = tens[i % pools]
        pkv.store(t.k_new(layer), t.v_new(layer), t.k_cache(layer), t.v_cache(layer),
                  dm["slot_mapping"])

    def attention(i, layer):
        t = tens[i % pools]
        kc, vc = t.k_cache(layer), t.v_cache(layer)
        if plan.kind == "decode":
            pkv.decode(t.q[layer], kc, vc, dm["block_tables"], dm["context_lens"], scale,
                       out=outs[i % pools], workspace=ws)
        else:
            pkv.prefill_varlen(t.q[layer], kc, vc, dm["block_tables"], dm["cu_seqlens_q"],
                               dm["cu_seqlens_k"], dm["max_seqlen_q"], dm["max_seqlen_k"], scale)

    def step(i):
        for layer in range(plan.layers):
            store(i, layer)
            attention(i, layer)

    # the timed region: whole steps, wall clock between synchronisations, no
    # events inside (recording timing events between calls perturbs them)
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    start = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - start
    ms_step = wall * 1e3 / steps

    # per-call durations: the same calls back to back (pools rotating as in the
    # steps), one pair of HIP events on the launch stream around each run
    L = plan.layers
    attn_ms = events_ms(torch, lambda k: attention(k // L, k % L), steps * L)
    # store calls back to back are bound by the host's call overhead, not the
    # GPU: the store's share is the step time per layer minus the attention call
    store_ms = max(ms_step / L - attn_ms, 0.0)
    res = dict(plan=plan, ms_per_step=ms_step, attn_ms=attn_ms, store_ms=store_ms)
    del tens, ws
    torch.cuda.empty_cache()
    return res


def cpu_baseline(name, budget_s, log):
    """The oracle (as it stands) on the same workload: one full step (store +
    attention) repeated until about budget_s of CPU work, inputs on the host."""
    import torch

    import oracle as O
    from workloads import make_plan, make_tensors

    plan = make_plan(name)
    tens = make_tensors(plan, "cpu", poison=False)
    orc = O.default()
    om = O.prepare_decode(plan.seqs, plan.block_size, plan.max_blocks_per_seq)
    scale = 1.0 / math.sqrt(plan.d)
    reps, total = 0, 0.0
    kc, vc = tens.k_cache().clone(), tens.v_cache().clone()
    while total < budget_s and reps < 1000:
        # storing the same rows again leaves the cache unchanged, so every
        # repetition is the same full step
        t0 = time.perf_counter()
        orc.store(kc, vc, tens.k_new(), tens.v_new(), om["slot_mapping"])
        orc.decode(tens.q[0], kc, vc, om["block_tables"], om["context_lens"], scale)
        total += time.perf_counter() - t0
        reps += 1
    step_s = total / reps
    gbs = (decode_bytes(plan) + store_bytes(plan)) / step_s / 1e9
    log(f"cpu oracle: {reps} full steps of {name}, {step_s * 1e3:.1f} ms each, {orc.threads()} threads")
    return dict(value=round(gbs, 3), unit="GB/s", cores=orc.threads(), kind="oracle",
                sample=f"{reps} full {name} steps (store + decode of all {plan.B} sequences), "
                       f"float64 C oracle, {step_s * 1e3:.1f} ms per step",
                ms_per_step=round(step_s * 1e3, 2))


def run_packed(steps, warmup, torch, pkv, log):
    """Varlen causal prefill over packed K/V (no block table, no prefix): q/k/v
    are row views of one fused projection buffer."""
    from workloads.packed import PACKED_PREFILL as cfg, make_packed, split_fused

    lens, cu, fused = make_packed("cuda")
    q, k, v = split_fused(fused)
    out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    scale = 1.0 / math.sqrt(cfg["d"])
    mx = max(lens)
    for _ in range(warmup):
        pkv.prefill_varlen_packed(q, k, v, cu, cu, mx, mx, scale, out=out)
    torch.cuda.synchronize()
    ms = events_ms(torch, lambda i: pkv.prefill_varlen_packed(q, k, v, cu, cu, mx, mx, scale, out=out),
                   steps)
    fl = 4 * cfg["d"] * cfg["H_q"] * sum(causal_pairs(0, n) for n in lens)
    tf = fl / (ms * 1e-3) / 1e12
    return dict(workload="packed_prefill", B=cfg["B"], tokens=sum(lens), attn_ms=round(ms, 4),
                prefill_tflops=round(tf, 2), prefill_pct_mfma_peak=round(100 * tf / BF16_PEAK_TFLOPS, 2),
                tokens_per_s=round(sum(lens) / (ms * 1e-3), 1), flops=fl)


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
            for _ in range(warmup):
                fn()
            torch.cuda.synchronize()
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
            for _ in range(warmup):
                fn()
            torch.cuda.synchronize()
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
    151936-token vocabulary (pkv_sample_gumbel, both launches), HIP events on
    the launch stream."""
    from workloads.sampling import SAMPLE_DECODE as cfg, make_logits

    logits, temps, seeds, offsets = make_logits("cuda")
    out = torch.empty(cfg["B"], dtype=torch.int64, device="cuda")
    ws = torch.empty(pkv.sample_workspace_size(cfg["B"], cfg["V"]), dtype=torch.uint8, device="cuda")
    step_offsets = [offsets + i for i in range(steps)]  # a fresh draw per step
    for _ in range(warmup):
        pkv.sample_gumbel(logits, seeds, temps, offsets, out=out, workspace=ws)
    torch.cuda.synchronize()
    ms = events_ms(torch, lambda i: pkv.sample_gumbel(logits, seeds, temps, step_offsets[i], out=out,
                                                      workspace=ws), steps)
    n = cfg["B"] * cfg["V"]
    nbytes = 2 * n + cfg["B"] * (4 + 8 + 8 + 8)
    res = dict(workload="gumbel_sample", B=cfg["B"], V=cfg["V"], dtype="bf16", bound="alu",
               ms=round(ms, 4),
               logits_per_s=round(n / (ms * 1e-3), 1), gb_per_s=round(nbytes / (ms * 1e-3) / 1e9, 2),
               pct_hbm_peak=round(100 * nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2))
    log(f"gumbel_sample: {json.dumps(res)}")
    return res


def copy_probe(torch, log, gib: float = 4.0, iters: int = 10) -> dict:
    """Plain device copy (torch copy_) and plain read (torch sum) of a buffer of known
    size: the achievable-bandwidth reference for the roofline, and the known-size
    kernel that scales the FETCH_SIZE / WRITE_SIZE counters."""
    n = int(gib * (1 << 30)) // 2
    src = torch.empty(n, dtype=torch.bfloat16, device="cuda").normal_()
    dst = torch.empty_like(src)
    res = {}
    for name, fn, nbytes in (("copy", lambda: dst.copy_(src), 4 * n),
                             ("read", lambda: src.sum(), 2 * n)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(iters):
            fn()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / iters
        res[name] = dict(bytes=nbytes, ms=round(ms, 4), gb_per_s=round(nbytes / ms / 1e6, 1))
        log(f"{name} probe: {nbytes / 2**30:.2f} GiB in {ms:.3f} ms = {nbytes / ms / 1e6:.0f} GB/s")
    return res


SECONDARY = ("packed_prefill", "graph_decode", "device_metadata", "gumbel_sample",
             "long_decode", "prefix_prefill", "full_step", "wide_gqa_decode")


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="qwen3_decode",
                    choices=["qwen3_decode", "long_decode", "prefix_prefill", "full_step",
                             "wide_gqa_decode"])
    ap.add_argument("--pools", type=int, default=2,
                    help="independent copies of the cache rotated across steps (single-layer workloads)")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--secondary", default="all",
                    help="comma-separated secondary workloads to run (default: all of "
                         + ", ".join(SECONDARY) + ")")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run the plain copy / read probes and print their JSON")
    args = ap.parse_args()

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); this path has no "
              "multi-GPU mode", file=sys.stderr)
        return 2

    import torch

    import paged_kv_cache_110_amd as pkv

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    pkv._lib.load()
    if args.copy_probe:
        print(json.dumps(dict(probe=copy_probe(torch, log))), flush=True)
        return 0

    def summarize(res):
        plan = res["plan"]
        out = dict(workload=plan.name, ms_per_step=round(res["ms_per_step"], 4),
                   attn_ms=round(res["attn_ms"], 4), store_ms=round(res["store_ms"], 4))
        if plan.kind == "decode":
            db = decode_bytes(plan) * plan.layers
            sb = store_bytes(plan) * plan.layers
            out["gb_per_s"] = round((db + sb) / (res["ms_per_step"] * 1e-3) / 1e9, 2)
            out["decode_gb_per_s"] = round(decode_bytes(plan) / (res["attn_ms"] * 1e-3) / 1e9, 2)
            out["decode_pct_hbm_peak"] = round(100 * out["decode_gb_per_s"] / HBM_PEAK_GBS, 2)
            out["tokens_per_s"] = round(plan.B / (res["ms_per_step"] * 1e-3), 1)
            out["kv_tokens_per_layer"] = plan.kv_tokens()
        else:
            fl = prefill_flops(plan)
            out["prefill_tflops"] = round(fl / (res["attn_ms"] * 1e-3) / 1e12, 2)
            out["prefill_pct_mfma_peak"] = round(100 * out["prefill_tflops"] / BF16_PEAK_TFLOPS, 2)
            out["tokens_per_s"] = round(plan.total_new / (res["ms_per_step"] * 1e-3), 1)
            out["flops"] = fl
        return out

    main_res = run_workload(args.workload, args.steps, args.warmup,
                            args.pools if args.workload != "full_step" else 1, torch, pkv, log)
    plan = main_res["plan"]
    s = summarize(main_res)
    log(json.dumps(s))

    secondary = {}
    wanted = set() if args.no_secondary else (
        set(SECONDARY) if args.secondary == "all" else set(args.secondary.split(",")))
    unknown = wanted - set(SECONDARY)
    if unknown:
        print(f"unknown secondary workloads: {sorted(unknown)}", file=sys.stderr)
        return 2
    if wanted:
        n2 = max(5, args.steps // 2)
        if "packed_prefill" in wanted:
            secondary["packed_prefill"] = run_packed(n2, 2, torch, pkv, log)
            log(json.dumps(secondary["packed_prefill"]))
        if "graph_decode" in wanted:
            secondary["graph_decode"] = run_graph(n2, 3, torch, pkv, log)
        if "device_metadata" in wanted:
            secondary["device_metadata"] = run_meta(n2, 3, torch, pkv, log)
        if "gumbel_sample" in wanted:
            secondary["gumbel_sample"] = run_sample(n2, 3, torch, pkv, log)
        for name in ["long_decode", "prefix_prefill", "full_step", "wide_gqa_decode"]:
            if name == args.workload or name not in wanted:
                continue
            r = run_workload(name, max(5, args.steps // 2), 2,
                             1 if name in ("full_step", "prefix_prefill") else args.pools,
                             torch, pkv, log)
            secondary[name] = summarize(r)
            log(json.dumps(secondary[name]))

    if plan.kind == "decode":
        value = s["gb_per_s"]
        unit = "GB/s"
        per_launch = decode_bytes(plan)
        achieved = per_launch / (main_res["attn_ms"] * 1e-3) / 1e9
        traffic = measured_traffic(plan.name)
        roofline = dict(bound="hbm", kernel="pkv_decode call (decode_kernel + decode_merge_kernel)",
                        achieved=round(achieved, 2), peak=HBM_PEAK_GBS, unit="GB/s",
                        frac=round(achieved / HBM_PEAK_GBS, 4),
                        traffic=None if traffic is None else round(traffic),
                        traffic_unit="bytes per call (FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0)",
                        bytes_per_launch=per_launch, avg_launch_ms=round(main_res["attn_ms"], 4))
    else:
        value = s["prefill_tflops"]
        unit = "TFLOP/s"
        fl = prefill_flops(plan)
        achieved = fl / (main_res["attn_ms"] * 1e-3) / 1e12
        roofline = dict(bound="mfma", kernel="prefill_kernel", achieved=round(achieved, 2),
                        peak=BF16_PEAK_TFLOPS, unit="TFLOP/s",
                        frac=round(achieved / BF16_PEAK_TFLOPS, 4), traffic=None,
                        flops_per_launch=fl, avg_launch_ms=round(main_res["attn_ms"], 4))

    if plan.kind == "decode":
        # the same bytes against what plain torch kernels stream on this device
        probe = copy_probe(torch, log, gib=2.0, iters=5)
        torch.cuda.empty_cache()
        roofline["copy_ceiling_gb_per_s"] = probe["copy"]["gb_per_s"]
        roofline["read_ceiling_gb_per_s"] = probe["read"]["gb_per_s"]
        roofline["frac_of_copy"] = round(achieved / probe["copy"]["gb_per_s"], 4)
        roofline["frac_of_read"] = round(achieved / probe["read"]["gb_per_s"], 4)

    cpu = None
    if not args.no_cpu_baseline and plan.kind == "decode" and args.workload != "full_step":
        cpu = cpu_baseline(args.workload, args.cpu_budget, log)

    config = dict(workload=plan.name, B=plan.B, H_q=plan.H_q, H_kv=plan.H_kv, d=plan.d,
                  block_size=plan.block_size, layers=plan.layers, num_blocks=plan.num_blocks,
                  kv_tokens=plan.kv_tokens(), new_tokens=plan.total_new,
                  pools_rotated=args.pools if args.workload != "full_step" else 1,
                  step="store + attention" + (" per layer" if plan.layers > 1 else ""))
    line = dict(metric=METRIC, value=value, unit=unit, n_gpus=1, steps=args.steps,
                warmup=args.warmup, ms_per_step=s["ms_per_step"], higher_is_better=True,
                scaling="weak", vs_baseline=None, dtype="bf16", data="synthetic",
                config=config, roofline=roofline, cpu_baseline=cpu, detail=s,
                secondary=secondary)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
