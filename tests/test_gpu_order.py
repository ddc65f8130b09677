"""Claim order of pooled attention (the MPK summary's roadmap, "भविष्य की
दिशा": priority-based and throughput-oriented task scheduling), through the
C ABI.

With one persistent worker the layer's attention tasks are claimed strictly
one after another, so their start tickets (debug trace) give the claim order
exactly: it must follow (priority, context length) descending for order 2,
context length descending for order 1 (the default), slot order for order
-1, with empty slots last.  The order changes no result: the logits equal those of slot
order bit for bit.
"""
import numpy as np
import pytest
import torch

import synth
from persistent_runtime_amd import mk
from persistent_runtime_amd.kvcache import PagedKV
from synth.configs import TINY

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

DEV = "cuda"
B = 16


def _run(Wd, kv, order, toks, poss, prio, workers=1, trace=1):
    plan = mk.Plan(TINY, Wd, kv.k_pool, kv.v_pool, kv.page_table, max_batch=B,
                   opts=mk.default_options(n_workgroups=workers, debug_trace=trace,
                                           attn_pool=1, attn_splits=2, attn_order=order,
                                           prefill_chunk=-1))
    t = torch.as_tensor(toks, dtype=torch.int32, device=DEV)
    p = torch.as_tensor(poss, dtype=torch.int32, device=DEV)
    rows = torch.arange(B, dtype=torch.int32, device=DEV)
    pr = torch.as_tensor(prio, dtype=torch.int32, device=DEV)
    nxt = torch.zeros(B, dtype=torch.int32, device=DEV)
    lg = torch.zeros(B, TINY["vocab"], dtype=torch.float32, device=DEV)
    plan.batch_step(t, p, rows, nxt, lg, priorities=pr)
    plan.check()
    tr = plan.read_trace() if trace else None
    tasks, _ = mk.inspect_plan(plan.cfg, mk.default_options(
        n_workgroups=workers, n_cus=plan.info()["n_cus"], attn_pool=1, attn_splits=2))
    plan.free()
    return lg.cpu().numpy(), nxt.cpu().numpy(), tr, tasks


def test_claim_order_priority_and_longest_first():
    Wd = synth.make_weights(TINY, device=DEV)
    kv = PagedKV(TINY, max_batch=B, max_pages_per_seq=16, device=DEV)
    g = np.random.default_rng(4)
    ctx = [int(c) for c in g.integers(20, 200, B)]
    ctx[3] = ctx[7]            # a tie in context length: the lower slot first
    for b in range(B):
        K, V = synth.make_kv_values(TINY, ctx[b], stream_id=b, device=DEV)
        kv.write_tokens(b, K, V)
        kv.assign(b, ctx[b] + 1)
    poss = list(ctx)
    poss[11] = -1              # an empty slot
    toks = [int(t) for t in g.integers(0, TINY["vocab"], B)]
    prio = [int(p) for p in g.integers(0, 3, B)]
    ref = None
    for order in (-1, 1, 2):
        lg, ids, tr, tasks = _run(Wd, kv, order, toks, poss, prio)
        if ref is None:
            ref = (lg, ids)
        assert np.array_equal(lg, ref[0]) and np.array_equal(ids, ref[1]), order
        if order == -1:
            want = list(range(B))
        elif order == 1:
            want = sorted(range(B), key=lambda b: (poss[b] < 0, -poss[b], b))
        else:
            want = sorted(range(B), key=lambda b: (poss[b] < 0, -prio[b], -poss[b], b))
        for l in range(TINY["n_layers"]):
            att = [i for i, t in enumerate(tasks) if mk.OPS[t.op] == "ATTN" and t.layer == l]
            seq = [tasks[i].a0 for i in sorted(att, key=lambda i: tr[i, 0])]
            slots = list(dict.fromkeys(seq))  # each slot's tasks are claimed together
            assert slots == want, (order, l, slots, want)
            assert np.all(tr[att, 2] == 1)
