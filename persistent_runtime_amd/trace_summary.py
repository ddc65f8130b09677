"""Per-task timing of one persistent decode step: where the step's time goes.

Builds the workload (synthetic weights; a 39-token prompt or a synthetic
cached context), runs warm-up steps, then one step with the plan's timing
trace (debug_trace = 2: every task records, on the device's 100 MHz clock,
when its inputs were complete and when its outputs were about to be
written), and prints a Markdown summary:

- per operation, over all layers: tasks, mean and largest wait (a task's
  inputs-complete time minus the previous task's finish on the same
  worker: dependency wait plus any work the worker did in between), and the
  mean time from inputs complete to finish;
- the critical path of one middle layer: each operation's first
  inputs-complete and last finish, and the gap before it (from the previous
  operation's last finish);
- the idle fraction: summed waits over workers x step time.

    python -m persistent_runtime_amd.trace_summary --workload llama8b
    python -m persistent_runtime_amd.trace_summary --workload moe30b
"""
from __future__ import annotations

import argparse
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))

TICK_US = 0.01  # 100 MHz


def _command():
    return "python -m persistent_runtime_amd.trace_summary " + " ".join(sys.argv[1:])


def main():
    import torch

    import synth
    from persistent_runtime_amd import mk
    from persistent_runtime_amd.kvcache import PagedKV

    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="llama8b",
                    choices=["llama8b", "moe30b", "llama70b", "ragged"])
    ap.add_argument("--batch", type=int, default=64,
                    help="ragged: slots (8B shape, contexts U[128, 16384])")
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--layer", type=int, default=None, help="layer of the critical-path table")
    ap.add_argument("--save", default=None, help="also write the raw trace and task table (.npz)")
    ap.add_argument("--steps", type=int, default=1, help="traced steps (tables use the last)")
    a = ap.parse_args()
    dev = torch.device("cuda:0")
    if a.workload == "ragged":
        return ragged(a, dev)
    model = synth.MODELS[a.workload]
    ctx0 = 8192 if a.workload == "moe30b" else 39
    total = ctx0 + a.warmup + 2
    maxp = (total + 15) // 16
    Wd = synth.make_weights(model, device=dev)
    kv = PagedKV(model, max_batch=1, max_pages_per_seq=maxp, device=dev)
    kv.assign(0, maxp * 16)
    plan = mk.Plan(model, Wd, kv.k_pool, kv.v_pool, kv.page_table, max_batch=1,
                   opts=mk.default_options(debug_trace=2, planned_ctx=total))
    tok = torch.zeros(1, dtype=torch.int32, device=dev)
    if a.workload == "moe30b":
        K, V = synth.make_kv_values(model, ctx0, device=dev)
        kv.write_tokens(0, K, V)
        del K, V
        tok[0] = int(synth.make_prompt(1, model["vocab"])[0])
    else:
        plan.prefill(0, synth.make_prompt(ctx0, model["vocab"]).to(dev), ctx0, 0, tok)
    pos = torch.zeros(1, dtype=torch.int32, device=dev)
    for i in range(a.warmup + 1):
        pos[0] = ctx0 + i
        plan.decode_step(tok, pos, tok)
    plan.check()
    traces = [plan.read_trace().astype(np.int64)]
    for i in range(1, a.steps):
        pos[0] = ctx0 + a.warmup + i
        plan.decode_step(tok, pos, tok)
        plan.check()
        traces.append(plan.read_trace().astype(np.int64))
    tr = traces[-1]
    tasks, _ = mk.inspect_plan(plan.cfg, mk.default_options(
        debug_trace=2, planned_ctx=total, n_cus=plan.info()["n_cus"]))
    plan.free()
    if a.save:
        np.savez_compressed(a.save, traces=np.stack(traces),
                            op=np.array([t.op for t in tasks]),
                            layer=np.array([t.layer for t in tasks]),
                            worker=np.array([t.worker for t in tasks]),
                            nbytes=np.array([t.bytes for t in tasks]))
    summarize(dict(model, name=f"{model['name']}, batch 1"), tasks, tr, ctx0 + a.warmup, a.layer,
              _command())


def ragged(a, dev):
    """The 8B shape with `a.batch` slots of synthetic cached contexts uniform in
    [128, 16384] (the continuous-batching workload), one traced step."""
    import torch

    import synth
    from persistent_runtime_amd import mk
    from persistent_runtime_amd.kvcache import PagedKV
    model = synth.MODELS["llama8b"]
    B = a.batch
    sched = synth.ragged_schedule(B, 1)
    ctx = sched["ctx0"]
    Wd = synth.make_weights(model, device=dev)
    maxp = (16384 + a.warmup + 2 + 15) // 16
    kv = PagedKV(model, max_batch=B, max_pages_per_seq=maxp,
                 n_pages=sum((c + a.warmup + 2 + 15) // 16 for c in ctx) + B, device=dev)
    for b in range(B):
        K, V = synth.make_kv_values(model, ctx[b], stream_id=sched["sid0"][b], device=dev)
        kv.write_tokens(b, K, V)
        kv.assign(b, ctx[b] + a.warmup + 2)
        del K, V
    opts = dict(debug_trace=2, planned_ctx=16384)
    plan = mk.Plan(model, Wd, kv.k_pool, kv.v_pool, kv.page_table, max_batch=B,
                   opts=mk.default_options(**opts))
    tok = torch.as_tensor(synth.make_prompt(B, model["vocab"], seed=7), dtype=torch.int32).to(dev)
    for i in range(a.warmup + 1):
        pos = torch.as_tensor([c + i for c in ctx], dtype=torch.int32).to(dev)
        plan.decode_step(tok, pos, tok)
    plan.check()
    tr = plan.read_trace().astype(np.int64)
    tasks, _ = mk.inspect_plan(plan.cfg, mk.default_options(n_cus=plan.info()["n_cus"], **opts))
    plan.free()
    if a.save:
        np.savez_compressed(a.save, traces=tr[None], op=np.array([t.op for t in tasks]),
                            layer=np.array([t.layer for t in tasks]),
                            worker=np.array([t.worker for t in tasks]),
                            nbytes=np.array([t.bytes for t in tasks]))
    summarize(dict(model, name=f"llama8b ragged, {B} slots"), tasks, tr, max(ctx) + a.warmup,
              a.layer, _command())


def summarize(model, tasks, tr, pos, layer, cmd):
    t_in, t_out, wk = tr[:, 4], tr[:, 5], tr[:, 3]
    base = int(t_in.min())
    t_in = (t_in - base) % (1 << 32)
    t_out = (t_out - base) % (1 << 32)
    step = int(t_out.max())
    T = len(tasks)
    # wait of each task: inputs complete minus the finish of the worker's
    # previous task (the first task of a worker: from the step's start)
    wait = np.zeros(T)
    prev = {}
    for i in sorted(range(T), key=lambda i: (wk[i], i)):
        w = int(wk[i])
        wait[i] = t_in[i] - (prev[w] if w in prev else 0)
        prev[w] = t_out[i]
    ops = [mk_op(t) for t in tasks]
    L = model["n_layers"]
    print(f"# Decode-step timing: {model['name']}, position {pos}\n")
    print(f"Command: `{cmd}`\n")
    print(f"Step (first inputs-complete to last finish): {step * TICK_US:.1f} us; "
          f"{T} tasks on {len(set(wk.tolist()))} workers.\n")
    print("| op | tasks | mean wait us | max wait us | mean run us |")
    print("|---|---|---|---|---|")
    for op in dict.fromkeys(ops):
        idx = [i for i in range(T) if ops[i] == op]
        run = (t_out[idx] - t_in[idx]) * TICK_US
        print(f"| {op} | {len(idx)} | {wait[idx].mean() * TICK_US:.2f} | "
              f"{wait[idx].max() * TICK_US:.2f} | {run.mean():.2f} |")
    busy = sum(int(t_out[i] - t_in[i]) for i in range(T))
    nw = len(set(wk.tolist()))
    print(f"\nIdle fraction (sum of waits / (workers x step)): "
          f"{wait.sum() / (nw * step):.3f}; busy fraction {busy / (nw * step):.3f}.\n")
    l = layer if layer is not None else L // 2
    print(f"## Critical path of layer {l}\n")
    print("| op | first inputs complete us | last finish us | span us | gap before us |")
    print("|---|---|---|---|---|")
    last = None
    for op in dict.fromkeys(ops[i] for i in range(T) if tasks[i].layer == l):
        idx = [i for i in range(T) if tasks[i].layer == l and ops[i] == op]
        s0, s1 = int(t_in[idx].min()), int(t_out[idx].max())
        gap = "" if last is None else f"{(s0 - last) * TICK_US:.2f}"
        print(f"| {op} | {s0 * TICK_US:.1f} | {s1 * TICK_US:.1f} | {(s1 - s0) * TICK_US:.2f} | {gap} |")
        last = s1
    print(f"\n## Spread within each operation of layer {l} (us from the layer's first "
          f"inputs-complete)\n")
    print("| op | inputs complete p0 / p50 / p100 | finish p0 / p50 / p100 | run min / p50 / max |")
    print("|---|---|---|---|")
    first = None
    for op in dict.fromkeys(ops[i] for i in range(T) if tasks[i].layer == l):
        idx = [i for i in range(T) if tasks[i].layer == l and ops[i] == op]
        if first is None:
            first = int(t_in[idx].min())
        a = (t_in[idx] - first) * TICK_US
        f = (t_out[idx] - first) * TICK_US
        r = (t_out[idx] - t_in[idx]) * TICK_US
        q = lambda x: " / ".join(f"{v:.1f}" for v in np.percentile(x, [0, 50, 100]))
        print(f"| {op} | {q(a)} | {q(f)} | {q(r)} |")
    per_layer = []
    for ll in range(L):
        idx = [i for i in range(T) if tasks[i].layer == ll]
        per_layer.append((t_out[idx].max() - t_in[idx].min()) * TICK_US)
    print(f"\nLayer span (first inputs complete to last finish), mean over layers: "
          f"{np.mean(per_layer):.1f} us; step / layers: {step * TICK_US / L:.1f} us.")


def mk_op(t):
    from persistent_runtime_amd import mk
    return mk.OPS[t.op]


if __name__ == "__main__":
    main()
