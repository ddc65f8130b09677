"""Long-context parity: the Llama-3-8B layer shapes truncated to two layers,
batch 1, after a long synthetic cached context (seeded N(0, kv_std^2) bf16
keys and values, the same values given to the oracle's cache).

With one attention split per KV head, every wave of an attention task walks
more than 64 pages, so the page-id chunks after the first are taken; the
automatic split count is checked at the same contexts.  The full 131072-token
context of the long-context workload is one of the cases, and a 262136-token
context (the 256K contexts of the Cohere article, "Folyamatos
batchkezelés") another; one case keeps the
GEMV passes in registers only (no LDS weight slots), where a task whose next
task waits behind attention loads that task's first pass after its own
outputs.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from synth.configs import LLAMA8B, truncated
from tests.gpu_common import LOGIT_TOL, MARGIN, Runner, oracle_weights

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

CFG = truncated(LLAMA8B, 2)
_state = {}


def _weights():
    if "W" not in _state:
        Wd = synth.make_weights(CFG, device="cuda")
        _state["W"] = (Wd, oracle_weights(Wd, CFG))
    return _state["W"]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("ctx,splits,lds", [(20000, 1, 0), (20000, 0, 0), (131064, 1, 0),
                                            (131064, 0, 0), (20000, 0, -1), (262136, 0, 0)])
def test_long_context_attention_chunks(ctx, splits, lds):
    """lds = -1: GEMV passes in registers only (no LDS weight slots)."""
    Wd, Wt = _weights()
    print(f"longctx: ctx {ctx} splits {splits or 'auto'} weight_lds {lds}", flush=True)
    K, V = synth.make_kv_values(CFG, ctx, device="cuda")
    steps = 3
    r = Runner(CFG, Wd, B=1, maxp=(ctx + steps + 15) // 16, planned_ctx=ctx + steps,
               attn_splits=splits, weight_lds=lds)
    r.kv.write_tokens(0, K, V)
    Kh = synth.bf16_to_f32_np(synth.to_numpy_bf16(K))
    Vh = synth.bf16_to_f32_np(synth.to_numpy_bf16(V))
    del K, V
    cache = O.KVCache(CFG, K=list(Kh), V=list(Vh))
    tok = int(synth.make_prompt(1, CFG["vocab"])[0])
    worst = 0.0
    for i in range(steps):
        pos = ctx + i
        g_ids, g_lg = r.step([tok], [pos])
        ref = O.decode_step(Wt, CFG, cache, tok, pos)
        d = float(np.max(np.abs(g_lg[0] - ref)))
        worst = max(worst, d)
        m = O.top2_margin(ref)
        print(f"longctx: step {i} max|dlogit| {d:.3e} margin {m:.3f}", flush=True)
        if m > MARGIN:
            assert int(g_ids[0]) == O.greedy_argmax(ref)
        tok = O.greedy_argmax(ref)
    assert worst <= LOGIT_TOL, worst
    r.plan.free()
    torch.cuda.empty_cache()
