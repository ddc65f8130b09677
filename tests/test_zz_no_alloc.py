"""mk_build_plan_noalloc: a plan whose device state lives in the library's
static scratch array (no device allocation), for callers that cannot
allocate.  Its decode steps must give the same logits and tokens as a plan
from mk_build_plan over the same weights and cache, bit for bit (both run
the same kernels on the same task list), on two static plans built in a row,
the second for a smaller input; the first plan's handle is then refused."""
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


def _steps(plan, B, prompt_lens, n_steps, V):
    """Prefill each slot with its own prompt, then n_steps batched steps.
    Returns the logits and next tokens of every step."""
    out = []
    for b, n in enumerate(prompt_lens):
        toks = synth.make_prompt(n, V, seed=40 + b).to(DEV)
        plan.prefill(b, toks, n, 0)
    plan.check()
    tok = torch.tensor([3 + b for b in range(B)], dtype=torch.int32, device=DEV)
    nxt = torch.zeros(B, dtype=torch.int32, device=DEV)
    lg = torch.zeros(B, V, dtype=torch.float32, device=DEV)
    for i in range(n_steps):
        pos = torch.tensor([n + i for n in prompt_lens], dtype=torch.int32, device=DEV)
        plan.decode_step(tok, pos, nxt, lg)
        plan.check()
        out.append((lg.cpu().numpy().copy(), nxt.cpu().numpy().copy()))
        tok.copy_(nxt)
    return out


def _compare(Wd, B, maxp, prompt_lens, n_steps, splits):
    res = []
    for noalloc in (False, True):
        kv = PagedKV(TINY, max_batch=B, max_pages_per_seq=maxp, device=DEV)
        for b in range(B):
            kv.assign(b, maxp * 16)
        # (the allocation-free plan prefills token by token: it has no
        # internal prompt-chunk plan; the allocating one is set to match)
        plan = mk.Plan(TINY, Wd, kv.k_pool, kv.v_pool, kv.page_table, max_batch=B,
                       opts=mk.default_options(attn_splits=splits, prefill_chunk=-1),
                       noalloc=noalloc)
        res.append(_steps(plan, B, prompt_lens, n_steps, TINY["vocab"]))
        if noalloc:
            static_plan = plan
        else:
            plan.free()
    for (la, ta), (lb, tb) in zip(*res):
        assert np.array_equal(la, lb)
        assert np.array_equal(ta, tb)
    return static_plan


def test_noalloc_plan_matches_allocating_plan():
    Wd = synth.make_weights(TINY, device=DEV)
    first = _compare(Wd, B=3, maxp=8, prompt_lens=[21, 30, 9], n_steps=4, splits=3)
    second = _compare(Wd, B=1, maxp=4, prompt_lens=[17], n_steps=3, splits=1)
    # the second static plan replaced the first one's device state
    tok = torch.zeros(3, dtype=torch.int32, device=DEV)
    pos = torch.zeros(3, dtype=torch.int32, device=DEV)
    with pytest.raises(mk.MkError) as e:
        first.decode_step(tok, pos, tok)
    assert e.value.code == mk.MK_ERR_INVALID_ARG
    second.free()
    first.free()


def test_noalloc_plan_too_large_is_refused():
    """A plan whose device state exceeds the static scratch is refused with
    MK_ERR_UNSUPPORTED (the 8B shape: its RoPE table alone for 262144
    positions is 64 MiB)."""
    cfg = synth.MODELS["llama8b"]
    maxp = 262144 // 16
    k = torch.zeros(16, dtype=torch.bfloat16, device=DEV)
    table = torch.zeros((1, maxp), dtype=torch.int32, device=DEV)
    W = {n: torch.zeros(1, dtype=torch.bfloat16, device=DEV) for n in ("embed", "lm_head",
                                                                        "final_norm")}
    L = cfg["n_layers"]
    row = torch.zeros(8, dtype=torch.bfloat16, device=DEV)
    for n in ("attn_norm", "ffn_norm", "wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down"):
        W[n] = row.expand(L, 8)
    with pytest.raises(mk.MkError) as e:
        mk.Plan(cfg, W, k.view(1, 1, 1, 1, 16), k.view(1, 1, 1, 16, 1), table, max_batch=1,
                noalloc=True)
    assert e.value.code == mk.MK_ERR_UNSUPPORTED
    assert "static scratch" in str(e.value)
