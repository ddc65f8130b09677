"""The scheduled executor (MPK summary, "Part 2. Runtime": workers with task
queues, scheduler wavefronts with activated-event queues, event-based
execution) against the oracle and against the static-queue executor.

Same bar as the other executors: logits within 3e-2 of the oracle, greedy ids
where the oracle's margin exceeds 0.05, and in the trace every task runs
exactly once and starts after every producer of its inputs finished.  It runs
the same task code as the static executor, so its logits equal that
executor's bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from persistent_runtime_amd import mk
from synth.configs import TINY, LLAMA8B
from tests.gpu_common import LOGIT_TOL, Runner, assert_ids, oracle_weights, teacher_forced_run

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

DEV = "cuda"
SCHED = mk.MK_EXEC_SCHEDULED
TINY_MOE = dict(TINY, name="tiny_moe", ffn_dim=0, n_experts=16, top_k=4, expert_ffn_dim=256)


@pytest.fixture(scope="module")
def tiny():
    Wd = synth.make_weights(TINY, device=DEV)
    return Wd, oracle_weights(Wd, TINY)


@pytest.mark.parametrize("splits", [0, 1, 3])
def test_scheduled_tiny_teacher_forced(tiny, splits):
    print(f"scheduled tiny splits={splits}", flush=True)
    Wd, Wt = tiny
    r = Runner(TINY, Wd, B=1, maxp=8, executor=SCHED, attn_splits=splits, prefill_chunk=-1)
    worst, ids, cache = teacher_forced_run(r, Wt, synth.make_prompt(39, 1024).tolist(), 8)
    assert worst <= LOGIT_TOL, worst
    assert_ids(ids)
    r.plan.free()


def test_scheduled_equals_static_bitwise_batch(tiny):
    """Three sequences with split attention and an empty slot: the scheduled
    and the static-queue executors give the same ids and logits bit for bit
    (both on the vector tiles: the scheduled executor has no matrix-core
    tiles)."""
    Wd, _ = tiny
    out = []
    for ex in (mk.MK_EXEC_PERSISTENT, SCHED):
        r = Runner(TINY, Wd, B=4, maxp=8, attn_splits=3, executor=ex, prefill_chunk=-1,
                   batched_mfma=-1)
        for b in range(3):
            r.prefill(b, synth.make_prompt(20 + 5 * b, 1024).tolist())
        ids, lg = r.step([7, 8, 9, 0], [20, 25, 30, -1])
        out.append((ids.copy(), lg.copy()))
        r.plan.free()
    assert out[1][0][3] == -1
    assert np.array_equal(out[0][0], out[1][0])
    assert np.array_equal(out[0][1], out[1][1])


def test_scheduled_trace_dependencies_and_run_once(tiny):
    Wd, _ = tiny
    r = Runner(TINY, Wd, B=2, maxp=8, executor=SCHED, debug_trace=1, attn_splits=3)
    tasks, _ = mk.inspect_plan(r.plan.cfg, mk.default_options(
        executor=SCHED, n_cus=r.plan.info()["n_cus"], attn_splits=3))
    sig = {}
    for i, t in enumerate(tasks):
        for k in range(t.n_sig):
            sig.setdefault(t.sig_ev[k], []).append(i)
    for step in range(3):
        r.step([5, 9], [step, step + 4])
        tr = r.plan.read_trace()
        assert np.all(tr[:, 2] == 1), "a task did not run exactly once"
        start, fin = tr[:, 0].astype(np.int64), tr[:, 1].astype(np.int64)
        assert np.all(fin > start)
        for c, t in enumerate(tasks):
            for k in range(t.n_wait):
                for p in sig[t.wait_ev[k]]:
                    assert fin[p] < start[c], (step, p, c)
    r.plan.free()


def test_scheduled_tiny_moe(tiny):
    cfg = TINY_MOE
    Wd = synth.make_weights(cfg, device=DEV)
    Wt = oracle_weights(Wd, cfg)
    r = Runner(cfg, Wd, B=1, maxp=8, executor=SCHED, prefill_chunk=-1)
    worst, ids, cache = teacher_forced_run(r, Wt, synth.make_prompt(20, 1024).tolist(), 4)
    assert worst <= LOGIT_TOL, worst
    r.plan.free()


@pytest.mark.timeout(600)
def test_scheduled_llama8b_2layer():
    """The 8B layer shapes (two layers): 256 workgroups, 33k-row projections
    spread over 255 workers, dispatched by four schedulers."""
    cfg = synth.truncated(LLAMA8B, 2)
    Wd = synth.make_weights(cfg, device=DEV)
    Wt = oracle_weights(Wd, cfg)
    r = Runner(cfg, Wd, B=1, maxp=8, executor=SCHED, prefill_chunk=-1)
    worst, ids, cache = teacher_forced_run(r, Wt, synth.make_prompt(12, cfg["vocab"]).tolist(), 3)
    assert worst <= LOGIT_TOL, worst
    assert_ids(ids)
    r.plan.free()
