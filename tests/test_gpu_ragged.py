"""Continuous batching on the Llama-3-8B shape at full size: 4, 8, 16 and 64
slots (the matrix-core tiles with split-K, the default from three slots;
from 8 slots the attention tasks are claimed from a shared pool;
and at 4 slots also the vector multi-slot tiles) with seeded synthetic
cached contexts uniform in [128, 16384] over shuffled 16-token pages, in
the launch configuration the ragged benchmark times.

Three decode steps.  Before the second, one sequence retires and a new one
(fresh context and KV) joins its slot; during the third, one slot is empty
(position -1).  The oracle decodes a sample of the slots one by one (the
joining one, the longest context, the shortest and one more) against the
same cached keys and values, fed the same tokens; logits must agree within
the fp32-accumulate bound and greedy ids wherever the oracle's top-2 margin
exceeds 0.05.  Slots left out of the sample must still produce valid ids.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from synth.configs import LLAMA8B
from tests.gpu_common import LOGIT_TOL, MARGIN, oracle_weights
from persistent_runtime_amd import mk
from persistent_runtime_amd.kvcache import PagedKV

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)


@pytest.fixture(scope="module")
def llama8b():
    Wd = synth.make_weights(LLAMA8B, device="cuda")
    return Wd, oracle_weights(Wd, LLAMA8B)


def _host_kv(cfg, ctx, sid):
    K, V = synth.make_kv_values(cfg, ctx, stream_id=sid, device="cuda")
    return K, V, (synth.bf16_to_f32_np(synth.to_numpy_bf16(K)),
                  synth.bf16_to_f32_np(synth.to_numpy_bf16(V)))


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("B,mfma", [(4, 0), (4, -1), (8, 0), (16, 0), (64, 0)],
                         ids=["4", "4-vector", "8", "16", "64"])
def test_llama8b_ragged_batch_join_retire(llama8b, B, mfma):
    cfg = LLAMA8B
    Wd, Wt = llama8b
    sched = synth.ragged_schedule(B, 3)
    ctx = list(sched["ctx0"])
    sid = list(sched["sid0"])
    join_slot, empty_slot = (1, 2) if B < 8 else (5, min(9, B - 1))
    join_ctx, join_sid = 3001, 10_000
    sample = sorted({join_slot, int(np.argmax(ctx)), int(np.argmin(ctx)), 0} - {empty_slot})
    print(f"ragged B={B}: contexts {ctx}; oracle sample {sample}", flush=True)
    maxp = (16384 + 8 + 15) // 16
    n_pages = sum((c + 8 + 15) // 16 for c in ctx) + (join_ctx + 8 + 15) // 16
    kv = PagedKV(cfg, max_batch=B, max_pages_per_seq=maxp, n_pages=n_pages, device="cuda")
    caches = {}
    for b in range(B):
        K, V, (Kh, Vh) = _host_kv(cfg, ctx[b], sid[b])
        kv.write_tokens(b, K, V)
        if b in sample:
            caches[b] = O.KVCache(cfg, K=list(Kh), V=list(Vh))
        del K, V
    plan = mk.Plan(cfg, Wd, kv.k_pool, kv.v_pool, kv.page_table, max_batch=B,
                   opts=mk.default_options(planned_ctx=16384, batched_mfma=mfma))
    tok_d = torch.zeros(B, dtype=torch.int32, device="cuda")
    pos_d = torch.zeros(B, dtype=torch.int32, device="cuda")
    nxt_d = torch.zeros(B, dtype=torch.int32, device="cuda")
    lg_d = torch.zeros(B, cfg["vocab"], dtype=torch.float32, device="cuda")
    toks = synth.make_prompt(B, cfg["vocab"], seed=11).tolist()
    worst = 0.0
    for step in range(3):
        if step == 1:  # one sequence retires, a new one joins its slot
            kv.release(join_slot, upload=False)
            K, V, (Kh, Vh) = _host_kv(cfg, join_ctx, join_sid)
            kv.write_tokens(join_slot, K, V)
            del K, V
            caches[join_slot] = O.KVCache(cfg, K=list(Kh), V=list(Vh))
            ctx[join_slot] = join_ctx
            toks[join_slot] = int(synth.make_prompt(1, cfg["vocab"], seed=12)[0])
        pos = list(ctx)
        if step == 2:
            pos[empty_slot] = -1
        for b in range(B):
            if pos[b] >= 0:
                kv.assign(b, pos[b] + 1, upload=False)
        kv.upload()
        tok_d.copy_(torch.as_tensor(toks, dtype=torch.int32))
        pos_d.copy_(torch.as_tensor(pos, dtype=torch.int32))
        plan.decode_step(tok_d, pos_d, nxt_d, lg_d)
        plan.check()
        g_ids = nxt_d.cpu().numpy()
        g_lg = lg_d.cpu().numpy()
        for b in range(B):
            if pos[b] < 0:
                assert g_ids[b] == -1, (b, g_ids[b])
            else:
                assert 0 <= g_ids[b] < cfg["vocab"], (b, g_ids[b])
        for b in sample:
            ref = O.decode_step(Wt, cfg, caches[b], toks[b], pos[b])
            d = float(np.max(np.abs(g_lg[b] - ref)))
            worst = max(worst, d)
            m = O.top2_margin(ref)
            print(f"ragged B={B}: step {step} slot {b} ctx {pos[b]} max|dlogit| {d:.3e} margin {m:.3f}",
                  flush=True)
            if m > MARGIN:
                assert int(g_ids[b]) == O.greedy_argmax(ref), (step, b)
            toks[b] = O.greedy_argmax(ref)
        for b in range(B):
            if b not in sample and pos[b] >= 0:
                toks[b] = int(g_ids[b])
            if pos[b] >= 0:
                ctx[b] += 1
    assert worst <= LOGIT_TOL, worst
    plan.free()
    del kv, caches
    torch.cuda.empty_cache()
