#!/usr/bin/env python3
"""Decode-step benchmark: batch-1 greedy decode of the Llama-3-8B-shaped model
(32 layers, hidden 4096, 32q/8kv heads x 128, SwiGLU 14336, vocab 128256,
random bf16 weights) after a 39-token random prompt, one persistent
megakernel launch per generated token.

Prints one JSON line: tokens/s, ms/step, fraction of the HBM speed-of-light
(algorithmic bytes per step / 8 TB/s), the dominant kernel's roofline entry,
the kernel-per-op build of the same tiles on the same workload, and the CPU
oracle timed on a bounded sample.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload llama8b]

Other batch-1 workloads: moe30b (48-layer MoE, 128 experts top-8, after an
8192-token synthetic KV context), longctx (the 8B shape after a 131072-token
synthetic context; longctx256k: 262144 tokens), llama70b (80 layers, hidden
8192), tiny.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "batch-1 decode tokens/sec + % of HBM speed-of-light (bytes/step ÷ 8 TB/s)"
PROMPT = 39


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def read_traffic(workload):
    """HBM traffic per launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel source (else None)."""
    p = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(p):
        return None
    with open(p) as fh:
        t = json.load(fh)
    from persistent_runtime_amd.traffic import kernel_source_hash
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch")


def _host_info():
    """Host cores this process may use, CPU model name and RAM in GiB."""
    cores = len(os.sched_getaffinity(0))
    name = ""
    try:
        import subprocess
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                name = line.split(":", 1)[1].strip()
                break
    except Exception:
        pass
    ram = 0.0
    try:
        with open("/proc/meminfo") as fh:
            for line in fh:
                if line.startswith("MemTotal:"):
                    ram = int(line.split()[1]) / 2 ** 20
                    break
    except OSError:
        pass
    return cores, name, ram


def cpu_baseline(model, Wd, steps=3):
    """The oracle (numpy fp32, unchanged) decoding on the host's cores, BLAS
    threads = the cores this process may use: the same model (the device's
    weights copied to the host), one warm-up step that also upcasts the
    weights (not timed), then the median of `steps` decode steps at the
    first positions of the prompt.  When the host's RAM cannot hold the
    model's bf16 and fp32 copies, the model is depth-truncated to 2 and 6
    layers (real per-layer shapes, full LM head) and the per-layer and
    LM-head times are scaled to the full depth."""
    import numpy as np

    import oracle as O
    import synth
    from threadpoolctl import threadpool_limits
    cores, cpu_name, ram = _host_info()
    per_layer = sum(int(v[0].numel()) * 2 for k, v in Wd.items()
                    if k not in ("embed", "lm_head", "final_norm"))
    total = per_layer * model["n_layers"] + 2 * Wd["lm_head"].numel() * 2
    full = ram * 2 ** 30 > 3.5 * total + 16 * 2 ** 30
    prompt = synth.make_prompt(PROMPT, model["vocab"]).tolist()

    def run(cfg):
        Wn = {}
        for k, v in Wd.items():
            if k in ("embed", "lm_head", "final_norm"):
                Wn[k] = synth.to_numpy_bf16(v)
            else:
                Wn[k] = synth.to_numpy_bf16(v[: cfg["n_layers"]])
        Wt = O.OracleWeights(Wn, cfg)
        cache = O.KVCache(cfg)
        O.decode_step(Wt, cfg, cache, prompt[0], 0)  # warm-up: weights upcast once
        ts = []
        for p in range(1, 1 + steps):
            t0 = time.perf_counter()
            O.decode_step(Wt, cfg, cache, prompt[p], p)
            ts.append(time.perf_counter() - t0)
        del Wt, Wn
        return float(np.median(ts))

    with threadpool_limits(limits=cores):
        if full:
            t_step = run(model)
            how = f"full {model['n_layers']}-layer model"
        else:
            d0, d1 = 2, 6
            t0_, t1_ = run(synth.truncated(model, d0)), run(synth.truncated(model, d1))
            t_layer = max((t1_ - t0_) / (d1 - d0), 1e-9)
            t_step = model["n_layers"] * t_layer + max(t0_ - d0 * t_layer, 0.0)
            how = (f"{model['n_layers']}-layer model scaled from {d0}- and {d1}-layer "
                   f"truncations (host RAM {ram:.0f} GiB too small for the full model)")
    return {"value": round(1.0 / t_step, 4), "unit": "tokens/s", "cores": int(cores),
            "kind": "oracle",
            "sample": (f"numpy fp32 oracle, {model['name']} {how}, median of {steps} decode "
                       f"steps at positions 1-{steps} after one warm-up step (weight upcast "
                       f"not timed); {t_step * 1e3:.1f} ms/step"),
            "cpu_model": cpu_name, "host_ram_gib": round(ram, 1)}


def run_decode(plan, tok_ring, pos_all, first, n, logits=None):
    """Launch n greedy steps: step k reads tok_ring[k], writes tok_ring[k+1]."""
    for k in range(first, first + n):
        plan.decode_step(tok_ring[k:k + 1], pos_all[k:k + 1], tok_ring[k + 1:k + 2], logits)


# Batch-1 workloads: (model, how the context is made, its length).  "prompt":
# a 39-token random prompt through mk_prefill; "synthetic": seeded N(0, sd^2)
# bf16 keys/values written straight into the pages (the pages' 8K-context
# MoE run and the 131072-token long-context run).
WORKLOADS = {
    "llama8b": ("llama8b", "prompt", PROMPT),
    "tiny": ("tiny", "prompt", PROMPT),
    "llama70b": ("llama70b", "prompt", PROMPT),
    "moe30b": ("moe30b", "synthetic", 8192),
    "longctx": ("llama8b", "synthetic", 131072),
    "longctx256k": ("llama8b", "synthetic", 262144),
}


def timed_steps(plan, tok_ring, pos_all, first, n, stream, torch):
    """Time n steps with one event between consecutive launches on the
    launch stream; returns (per-launch ms list, total seconds, wall seconds)."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    ev[0].record(stream)
    for k in range(n):
        i = first + k
        plan.decode_step(tok_ring[i:i + 1], pos_all[i:i + 1], tok_ring[i + 1:i + 2])
        ev[k + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    launch_ms = [ev[k].elapsed_time(ev[k + 1]) for k in range(n)]
    return launch_ms, ev[0].elapsed_time(ev[n]) / 1e3, wall


def run_ragged(args, torch):
    """Continuous batching on the 8B shape: B slots, each holding a sequence
    with a synthetic cached context uniform in [128, 16384]; every step each
    sequence retires with probability 1/32 and a new one (fresh context and
    KV) joins its slot.  Only the decode launches are timed (HIP events on
    the launch stream around each step); page-table edits and the joining
    sequences' KV writes happen between them.  Prints one JSON line per
    batch size."""
    import synth
    from persistent_runtime_amd import mk, sol
    from persistent_runtime_amd.kvcache import PagedKV

    dev = torch.device("cuda:0")
    model = synth.MODELS["llama8b"]
    Wd = synth.make_weights(model, device=dev)
    stream = torch.cuda.current_stream()
    batches = [int(b) for b in args.batches.split(",")]
    W_, K_ = args.warmup, args.steps if args.steps is not None else 128
    for B in batches:
        n = W_ + K_
        sched = synth.ragged_schedule(B, n)
        ctx_hi = 16384
        maxp = (ctx_hi + n + 1 + 15) // 16
        in_use = max(sum((p + 1 + 15) // 16 for p in sched["pos"][k]) for k in range(n))
        kv = PagedKV(model, max_batch=B, max_pages_per_seq=maxp, n_pages=in_use + B, device=dev)
        t0 = time.time()
        for b in range(B):
            K, V = synth.make_kv_values(model, sched["ctx0"][b], stream_id=sched["sid0"][b],
                                        device=dev)
            kv.write_tokens(b, K, V)
            del K, V
        torch.cuda.synchronize()
        log(f"[bench] ragged B={B}: {sum(sched['ctx0'])} cached tokens in {kv.n_pages} pages "
            f"({time.time() - t0:.1f}s)")
        opts = {} if args.attn_splits is None else {"attn_splits": args.attn_splits}
        opts["attn_order"] = args.attn_order
        opts["batched_mfma"] = args.batched_mfma
        opts["attn_pool"] = args.attn_pool

        def run(plans, k0, k1, timed):
            """Steps k0..k1 of the schedule, step k on plans[k % len(plans)]
            (the executors alternate step by step, so both see the same mix
            of contexts, joins and retirements); per plan: the timed steps'
            milliseconds and algorithmic bytes."""
            tok = torch.as_tensor(synth.make_prompt(B, model["vocab"], seed=7 + k0),
                                  dtype=torch.int32).to(dev)
            nxt = torch.zeros(B, dtype=torch.int32, device=dev)
            ev = [[] for _ in plans]
            nbytes = [[] for _ in plans]
            for k in range(k0, k1):
                for (b, c, sid) in sched["joins"][k]:  # retire first, then join
                    kv.release(b, upload=False)
                for (b, c, sid) in sched["joins"][k]:
                    K, V = synth.make_kv_values(model, c, stream_id=sid, device=dev)
                    kv.write_tokens(b, K, V)
                    del K, V
                    tok[b] = int(synth.make_prompt(1, model["vocab"], seed=1000 + sid)[0])
                pos = sched["pos"][k]
                added = False
                for b in range(B):
                    added |= kv.assign(b, pos[b] + 1, upload=False)
                if added or sched["joins"][k]:
                    kv.upload()
                pos_d = torch.as_tensor(pos, dtype=torch.int32).to(dev)
                i = k % len(plans)
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                plans[i].decode_step(tok, pos_d, nxt)
                e1.record(stream)
                tok, nxt = nxt, tok
                if timed:
                    ev[i].append((e0, e1))
                    nbytes[i].append(sol.step_bytes(model, [p + 1 for p in pos]))
            for pl in plans:
                pl.check()
            torch.cuda.synchronize()
            return [[a.elapsed_time(b) for a, b in e] for e in ev], nbytes

        plan = mk.Plan(model, Wd, kv.k_pool, kv.v_pool, kv.page_table, max_batch=B,
                       opts=mk.default_options(planned_ctx=ctx_hi, **opts))
        info = plan.info()
        plans = [plan]
        if not args.no_kpo:
            plans.append(mk.Plan(model, Wd, kv.k_pool, kv.v_pool, kv.page_table, max_batch=B,
                                 opts=mk.default_options(planned_ctx=ctx_hi,
                                                         executor=mk.MK_EXEC_KERNEL_PER_OP,
                                                         **opts)))
        run(plans, 0, W_, False)
        ms_all, nb_all = run(plans, W_, n, True)
        ms, nbytes = ms_all[0], nb_all[0]
        kk = len(ms)
        t_ms = sum(ms)
        tok_s = B * kk / (t_ms / 1e3)
        achieved = sum(nbytes) / (t_ms / 1e3) / 1e9
        kpo = None
        if not args.no_kpo:
            ms_k = ms_all[1]
            kpo = {"ms_per_step": round(sum(ms_k) / len(ms_k), 4),
                   "launches_per_step": plans[1].info()["n_phases"],
                   "timing": "alternate steps of the same schedule"}
            kpo["persistent_speedup"] = round(kpo["ms_per_step"] / (t_ms / kk), 3)
        for pl in plans:
            pl.free()
        log(f"[bench] ragged B={B}: {t_ms / kk:.3f} ms/step, {tok_s:.1f} tok/s, "
            f"{achieved:.0f} GB/s" + (f"; kernel-per-op {kpo['ms_per_step']:.3f} ms/step" if kpo else ""))
        out = {
            "metric": "decode tokens/s, continuous batching", "value": round(tok_s, 2),
            "unit": "tokens/s", "n_gpus": 1, "steps": kk, "warmup": W_,
            "ms_per_step": round(t_ms / kk, 4), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": f"llama8b ragged decode, batch {B}, contexts U[128,16384], "
                                   f"16-token shuffled pages, retire/join p=1/32 per step",
                       "batch": B, "attn_splits": args.attn_splits,
                       "attn_order": args.attn_order,
                       "batched_mfma": args.batched_mfma, "attn_pool": args.attn_pool,
                       "tasks_per_step": info["n_tasks"]},
            "sol_fraction": round(achieved / 8000.0, 4),
            "bytes_per_step": int(sum(nbytes) / kk),
            "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": 8000.0,
                         "unit": "GB/s", "frac": round(achieved / 8000.0, 4), "traffic": None,
                         "kernel": "mk_persistent_kernel"},
            "kernel_per_op": kpo,
        }
        print(json.dumps(out), flush=True)
        del kv
        torch.cuda.empty_cache()


def kpo_graph_ms(build, start, tok_ring, pos_all, n, stream, torch):
    """Kernel-per-op step captured in a HIP graph (counters cleared by a
    kernel inside the step, so the graph replays): one replay feeds the
    previous token and the next position, as the eager runs do.  Returns the
    mean ms per replay over n - 2 replays after 2 warm-up replays."""
    from persistent_runtime_amd import mk
    plan = build(mk.MK_EXEC_KERNEL_PER_OP, graph_replay=1)
    dev = tok_ring.device
    ring = torch.zeros(2, dtype=torch.int32, device=dev)
    start(plan, ring)
    tok = ring[0:1].clone()
    pos = pos_all[0:1].clone()
    nxt = torch.zeros(1, dtype=torch.int32, device=dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # eager warm-up on the capture stream
        plan.decode_step(tok, pos, nxt)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plan.decode_step(tok, pos, nxt)
        tok.copy_(nxt)
        pos.add_(1)
    pos.copy_(pos_all[1:2])
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(n - 2):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    plan.check()
    plan.free()
    return e0.elapsed_time(e1) / (n - 2)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="llama8b", choices=sorted(WORKLOADS) + ["ragged"])
    ap.add_argument("--batches", default="4,16,64", help="ragged: batch sizes")
    ap.add_argument("--attn-splits", type=int, default=None,
                    help="KV splits per (sequence, KV head); default: the planner's choice")
    ap.add_argument("--kpo-steps", type=int, default=64, help="kernel-per-op comparison steps")
    ap.add_argument("--attn-pool", type=int, default=0, choices=(-1, 0, 1),
                    help="ragged: attention claimed at run time (0 auto, 1 on, -1 static)")
    ap.add_argument("--batched-mfma", type=int, default=0, choices=(-1, 0, 1),
                    help="ragged: GEMVs as matrix-core tiles (0 auto, 1 for any batch >= 2, -1 off)")
    ap.add_argument("--attn-order", type=int, default=0, choices=(-1, 0, 1),
                    help="ragged: claim order of pooled attention (0: the plan's default, "
                         "longest context first; -1: slot order)")
    ap.add_argument("--weight-lds", choices=("auto", "on", "off"), default="auto",
                    help="LDS weight slots of single-slot GEMV passes (auto: the planner's choice)")
    ap.add_argument("--no-weight-lds", action="store_true", help="the same as --weight-lds off")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kpo", action="store_true")
    ap.add_argument("--calib-copy", action="store_true",
                    help="run a plain 1 GiB device copy (traffic-counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "the decode-step kernel runs on one GPU; --gpus above 1 is "
                                   "not supported (the path would shard by tensor parallelism "
                                   "across GPUs, which is not built)"}))
        sys.exit(2)

    import torch
    import synth
    from persistent_runtime_amd import mk, sol
    from persistent_runtime_amd.kvcache import PagedKV

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calib_copy:
        a = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(4):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes": a.numel() * 4, "launches": 4}))
        return

    if args.workload == "ragged":
        run_ragged(args, torch)
        return
    mname, ctx_kind, ctx0 = WORKLOADS[args.workload]
    model = synth.MODELS[mname]
    default_steps = {"moe30b": 248, "longctx": 56, "longctx256k": 32,
                     "llama70b": 120}.get(args.workload, 504)
    W_, K_ = args.warmup, args.steps if args.steps is not None else default_steps
    total = ctx0 + W_ + K_
    maxp = (total + 15) // 16
    log(f"[bench] workload={args.workload} warmup={W_} steps={K_} ctx {ctx0}..{total - 1}")
    t0 = time.time()
    Wd = synth.make_weights(model, device=dev)
    torch.cuda.synchronize()
    log(f"[bench] weights generated in {time.time() - t0:.1f}s")
    kv = PagedKV(model, max_batch=1, max_pages_per_seq=maxp, device=dev)
    kv.assign(0, maxp * 16)
    if ctx_kind == "synthetic":
        K, V = synth.make_kv_values(model, ctx0, device=dev)
        kv.write_tokens(0, K, V)
        del K, V
        torch.cuda.empty_cache()
    pos_all = torch.arange(ctx0, ctx0 + W_ + K_ + 1, dtype=torch.int32, device=dev)

    def build(executor, graph_replay=0):
        extra = {} if args.attn_splits is None else {"attn_splits": args.attn_splits}
        if args.no_weight_lds or args.weight_lds == "off":
            extra["weight_lds"] = -1
        elif args.weight_lds == "on":
            extra["weight_lds"] = 1
        return mk.Plan(model, Wd, kv.k_pool, kv.v_pool, kv.page_table, max_batch=1,
                       opts=mk.default_options(executor=executor, planned_ctx=total,
                                               graph_replay=graph_replay, **extra))

    def start(plan, ring):
        """Context in place and the first token in ring[0]."""
        if ctx_kind == "prompt":
            prompt = synth.make_prompt(ctx0, model["vocab"]).to(dev)
            plan.prefill(0, prompt, ctx0, 0, ring[0:1])
        else:
            ring[0] = int(synth.make_prompt(1, model["vocab"])[0])

    plan = build(mk.MK_EXEC_PERSISTENT)
    info = plan.info()
    tok_ring = torch.zeros(W_ + K_ + 1, dtype=torch.int32, device=dev)
    start(plan, tok_ring)
    prefill = None
    if ctx_kind == "prompt":
        # the prompt again (it rewrites the same cache entries), timed
        prompt = synth.make_prompt(ctx0, model["vocab"]).to(dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        plan.prefill(0, prompt, ctx0, 0, tok_ring[0:1])
        e1.record()
        torch.cuda.synchronize()
        plan.check()
        pms = e0.elapsed_time(e1)
        prefill = {"tokens": ctx0, "ms": round(pms, 3), "tokens_per_s": round(ctx0 / pms * 1e3, 1),
                   "chunk": 64}
        log(f"[bench] prefill of {ctx0} tokens: {pms:.3f} ms")
    run_decode(plan, tok_ring, pos_all, 0, W_)
    plan.check()
    stream = torch.cuda.current_stream()
    launch_ms, elapsed, wall = timed_steps(plan, tok_ring, pos_all, W_, K_, stream, torch)
    plan.check()
    ms_step = elapsed * 1e3 / K_
    tok_s = K_ / elapsed
    # algorithmic bytes: weights + KV of all attended positions, per step
    ctxs = [ctx0 + W_ + k + 1 for k in range(K_)]
    bytes_steps = [sol.step_bytes(model, [c]) for c in ctxs]
    bytes_mean = sum(bytes_steps) / K_
    avg_launch_s = sum(launch_ms) / K_ / 1e3
    achieved = bytes_mean / avg_launch_s / 1e9
    sol_frac = (bytes_mean / sol.HBM_PEAK_BYTES_PER_S) / (elapsed / K_)
    traffic = read_traffic(args.workload)
    log(f"[bench] persistent: {ms_step:.3f} ms/step, {tok_s:.1f} tok/s, {achieved:.0f} GB/s, "
        f"{100 * sol_frac:.1f}% SoL (wall {wall:.2f}s)")

    kpo = None
    if not args.no_kpo:
        plan_k = build(mk.MK_EXEC_KERNEL_PER_OP)
        ring2 = torch.zeros(W_ + K_ + 1, dtype=torch.int32, device=dev)
        start(plan_k, ring2)
        n = min(args.kpo_steps, W_ + K_)
        run_decode(plan_k, ring2, pos_all, 0, 2)
        kms_list, kel, _ = timed_steps(plan_k, ring2, pos_all, 2, n - 2, stream, torch)
        plan_k.check()
        kms = kel * 1e3 / (n - 2)
        same = bool(torch.equal(ring2[:n], tok_ring[:n]))
        kpo = {"ms_per_step": round(kms, 4), "tokens_per_s": round(1e3 / kms, 2),
               "launches_per_step": plan_k.info()["n_phases"],
               "persistent_speedup": round(kms / ms_step, 3),
               "same_tokens_first_steps": same}
        log(f"[bench] kernel-per-op: {kms:.3f} ms/step ({kpo['launches_per_step']} launches)")
        plan_k.free()
        # the same launches captured once in a HIP graph and replayed
        # the graph's eager warm-up takes position 0, its replays 1..n_g
        gms = kpo_graph_ms(build, start, tok_ring, pos_all, min(n, W_ + K_ - 1), stream, torch)
        kpo["graph_ms_per_step"] = round(gms, 4)
        kpo["persistent_speedup_vs_graph"] = round(gms / ms_step, 3)
        log(f"[bench] kernel-per-op in a HIP graph: {gms:.3f} ms/step")

    sched = None
    if not args.no_kpo:
        # the MPK-style executor (scheduler wavefronts and worker queues) on
        # the same workload
        plan_s = build(mk.MK_EXEC_SCHEDULED)
        ring3 = torch.zeros(W_ + K_ + 1, dtype=torch.int32, device=dev)
        start(plan_s, ring3)
        n = min(args.kpo_steps, W_ + K_)
        run_decode(plan_s, ring3, pos_all, 0, 2)
        _, sel, _ = timed_steps(plan_s, ring3, pos_all, 2, n - 2, stream, torch)
        plan_s.check()
        sms = sel * 1e3 / (n - 2)
        sched = {"ms_per_step": round(sms, 4), "tokens_per_s": round(1e3 / sms, 2),
                 "schedulers": 4, "workers": plan_s.info()["n_cus"] - 1,
                 "persistent_speedup": round(sms / ms_step, 3),
                 "same_tokens_first_steps": bool(torch.equal(ring3[:n], tok_ring[:n]))}
        log(f"[bench] scheduled (MPK-style) executor: {sms:.3f} ms/step")
        plan_s.free()

    plan.free()
    cpu = None
    if not args.no_cpu_baseline:
        t0 = time.time()
        cpu = cpu_baseline(model, Wd)
        log(f"[bench] cpu baseline {cpu['value']} tok/s in {time.time() - t0:.1f}s")

    ctx_desc = (f"{ctx0}-token prompt" if ctx_kind == "prompt"
                else f"{ctx0}-token synthetic KV context")
    out = {
        "metric": METRIC, "value": round(tok_s, 3), "unit": "tokens/s", "n_gpus": 1,
        "steps": K_, "warmup": W_, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{mname} decode, batch 1, {ctx_desc}, "
                               f"ctx {ctx0 + W_}..{total - 1}", "batch": 1,
                   "context": ctx0, "timed_steps": K_,
                   "tasks_per_step": info["n_tasks"], "workgroups": info["n_cus"]},
        "sol_fraction": round(sol_frac, 4),
        "bytes_per_step": int(bytes_mean),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": 8000.0,
                     "unit": "GB/s", "frac": round(achieved / 8000.0, 4),
                     "traffic": traffic, "kernel": "mk_persistent_kernel",
                     "avg_launch_ms": round(avg_launch_s * 1e3, 4)},
        "kernel_per_op": kpo,
        "scheduled_executor": sched,
        "prefill": prefill,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    # release every device resource before the interpreter exits, so no HIP
    # call runs from teardown (after a profiler's own finalisation)
    del kv, Wd
    torch.cuda.synchronize()
    import gc
    gc.collect()


if __name__ == "__main__":
    main()
