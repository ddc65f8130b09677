"""Full-size parity of the Qwen3-30B-A3B-shaped MoE model (48 layers, 128
experts, top-8), batch 1, at an 8192-token context of synthetic cached keys
and values (seeded N(0, (0.02 sqrt(H))^2) bf16, the same values given to the
oracle's cache), in the launch configuration the benchmark uses.

Three teacher-forced decode steps from a seeded first token; the device's
routing is read back each step and reconciled with the oracle's: expert sets
may differ only at a top-8 boundary closer than 1e-3 (several routings are
then correct), and such a step is compared against the oracle forced to the
device's experts.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from synth.configs import MOE30B
from tests.gpu_common import LOGIT_TOL, MARGIN, Runner, oracle_step_matching_routes

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

CTX = 8192


@pytest.mark.timeout(1000)
def test_moe30b_full_size_synthetic_context():
    cfg = MOE30B
    print("MoE: generating weights and the synthetic context", flush=True)
    Wd = synth.make_weights(cfg, device="cuda")
    K, V = synth.make_kv_values(cfg, CTX, device="cuda")
    r = Runner(cfg, Wd, B=1, maxp=(CTX + 8 + 15) // 16, planned_ctx=CTX + 8)
    r.kv.write_tokens(0, K, V)
    print("MoE: copying weights to the host for the oracle", flush=True)
    Wn = {k: synth.to_numpy_bf16(v) for k, v in Wd.items()}
    Wt = O.OracleWeights(Wn, cfg, cache=False)
    Kh = synth.bf16_to_f32_np(synth.to_numpy_bf16(K))
    Vh = synth.bf16_to_f32_np(synth.to_numpy_bf16(V))
    del K, V
    cache = O.KVCache(cfg, K=list(Kh), V=list(Vh))
    tok = int(synth.make_prompt(1, cfg["vocab"])[0])
    worst, forced_steps = 0.0, 0
    for i in range(3):
        pos = CTX + i
        g_ids, g_lg = r.step([tok], [pos])
        dev_routes, _ = r.plan.read_routing()
        ref, nf = oracle_step_matching_routes(Wt, cfg, cache, tok, pos, dev_routes)
        forced_steps += nf > 0
        d = float(np.max(np.abs(g_lg[0] - ref)))
        worst = max(worst, d)
        m = O.top2_margin(ref)
        print(f"MoE: step {i} max|dlogit| {d:.3e} forced layers {nf} margin {m:.3f}", flush=True)
        if m > MARGIN:
            assert int(g_ids[0]) == O.greedy_argmax(ref)
        tok = O.greedy_argmax(ref)
    assert worst <= LOGIT_TOL, worst
    r.plan.free()
