"""Full-size parity of the Llama-3-8B-shaped model, in the launch
configuration the benchmark times (persistent executor, one workgroup per CU,
attention splits sized for the 551-token context).

The oracle computes the 39-token prompt with its full causal forward (which
also yields its KV cache) and then a few teacher-forced decode steps; the
device runs the same prompt through mk_prefill and mk_decode_step.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from synth.configs import LLAMA8B
from tests.gpu_common import LOGIT_TOL, MARGIN, Runner, oracle_weights

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)


@pytest.mark.timeout(900)
def test_llama8b_full_size_teacher_forced():
    cfg = LLAMA8B
    print("8B: generating weights", flush=True)
    Wd = synth.make_weights(cfg, device="cuda")
    total = 39 + 512
    r = Runner(cfg, Wd, B=1, maxp=(total + 15) // 16, planned_ctx=total)
    prompt = synth.make_prompt(39, cfg["vocab"]).tolist()
    g_tok, g_lg = r.prefill(0, prompt)
    print("8B: device prefill done; oracle full forward", flush=True)
    Wt = oracle_weights(Wd, cfg)
    logits, cache = O.forward_full(Wt, cfg, prompt, return_cache=True)
    ref = logits[-1]
    worst = float(np.max(np.abs(g_lg - ref)))
    ids = [(g_tok, O.greedy_argmax(ref), O.top2_margin(ref))]
    for i in range(3):
        t = O.greedy_argmax(ref)
        g_ids, lg = r.step([t], [39 + i])
        ref = O.decode_step(Wt, cfg, cache, t, 39 + i)
        worst = max(worst, float(np.max(np.abs(lg[0] - ref))))
        ids.append((int(g_ids[0]), O.greedy_argmax(ref), O.top2_margin(ref)))
        print(f"8B: step {i} max|dlogit| so far {worst:.3e}", flush=True)
    assert worst <= LOGIT_TOL, worst
    for g, o, m in ids:
        if m > MARGIN:
            assert g == o, (g, o, m)
    r.plan.free()
