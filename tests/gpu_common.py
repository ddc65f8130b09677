"""Shared helpers of the GPU parity tests (imported by tests marked `gpu`)."""
from __future__ import annotations

import numpy as np
import torch

import oracle as O
import synth
from persistent_runtime_amd import mk
from persistent_runtime_amd.kvcache import PagedKV

LOGIT_TOL = 3e-2      # max |dlogit| for bf16-weight, fp32-accumulate math
MARGIN = 0.05         # greedy ids must match where the oracle's top-2 gap exceeds this


def oracle_weights(Wd: dict, cfg: dict, dtype=np.float32, cache=True):
    Wn = {k: synth.to_numpy_bf16(v) for k, v in Wd.items()}
    return O.OracleWeights(Wn, cfg, dtype, cache=cache)


def bf16_ulp(x):
    a = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 1e-30)))
    return np.exp2(e - 7)


class Runner:
    """One plan plus device-side token/position buffers."""

    def __init__(self, cfg, Wd, B=1, maxp=8, n_pages=None, dev="cuda", **opt):
        self.cfg, self.B, self.dev = cfg, B, dev
        self.kv = PagedKV(cfg, max_batch=B, max_pages_per_seq=maxp, n_pages=n_pages, device=dev)
        for b in range(B):
            self.kv.assign(b, maxp * 16)
        self.plan = mk.Plan(cfg, Wd, self.kv.k_pool, self.kv.v_pool, self.kv.page_table,
                            max_batch=B, opts=mk.default_options(**opt))
        self.tok = torch.zeros(B, dtype=torch.int32, device=dev)
        self.pos = torch.full((B,), -1, dtype=torch.int32, device=dev)
        self.nxt = torch.zeros(B, dtype=torch.int32, device=dev)
        self.logits = torch.zeros(B, cfg["vocab"], dtype=torch.float32, device=dev)

    def prefill(self, slot, prompt):
        t = torch.as_tensor(prompt, dtype=torch.int32).to(self.dev)
        nt = torch.zeros(1, dtype=torch.int32, device=self.dev)
        lg = torch.zeros(self.cfg["vocab"], dtype=torch.float32, device=self.dev)
        self.plan.prefill(slot, t, len(prompt), 0, nt, lg)
        self.plan.check()
        return int(nt.item()), lg.cpu().numpy()

    def step(self, tokens, positions):
        self.tok.copy_(torch.as_tensor(tokens, dtype=torch.int32))
        self.pos.copy_(torch.as_tensor(positions, dtype=torch.int32))
        self.plan.decode_step(self.tok, self.pos, self.nxt, self.logits)
        self.plan.check()
        return self.nxt.cpu().numpy().copy(), self.logits.cpu().numpy().copy()


def teacher_forced_run(runner: Runner, Wt, prompt, n_steps, slot=0):
    """Prefill `prompt` then decode n_steps with the oracle's greedy tokens
    fed to both sides.  Returns (max |dlogit|, list of (gpu id, oracle id,
    oracle margin))."""
    cfg = runner.cfg
    cache = O.KVCache(cfg)
    for p, t in enumerate(prompt):
        ref = O.decode_step(Wt, cfg, cache, int(t), p)
    g_tok, g_lg = runner.prefill(slot, prompt)
    worst = float(np.max(np.abs(g_lg - ref)))
    ids = [(g_tok, O.greedy_argmax(ref), O.top2_margin(ref))]
    pos = len(prompt)
    for i in range(n_steps):
        t_ref = O.greedy_argmax(ref)
        toks = [0] * runner.B
        poss = [-1] * runner.B
        toks[slot], poss[slot] = t_ref, pos
        g_ids, g_lg = runner.step(toks, poss)
        ref = O.decode_step(Wt, cfg, cache, t_ref, pos)
        worst = max(worst, float(np.max(np.abs(g_lg[slot] - ref))))
        ids.append((int(g_ids[slot]), O.greedy_argmax(ref), O.top2_margin(ref)))
        pos += 1
    return worst, ids, cache


def assert_ids(ids):
    for g, o, m in ids:
        if m > MARGIN:
            assert g == o, (g, o, m)


ROUTE_TIE = 1e-3      # top-k boundary margin below which either routing is correct


def oracle_step_matching_routes(Wt, cfg, cache, token, pos, dev_ids, slot=0):
    """One oracle decode step whose MoE routing is reconciled with the
    device's: a layer whose expert set differs from the oracle's is accepted
    only when the sets differ by one expert at the top-k boundary and the
    oracle's boundary margin is below ROUTE_TIE; the step is then re-run with
    the device's experts forced at those layers (later layers see the forced
    activations and are compared again).  Any other difference fails.
    `dev_ids`: device routing [L, B, top_k].  Returns (logits, n forced)."""
    import copy
    snapK, snapV = list(cache.K), list(cache.V)
    forced = {}
    for _ in range(cfg["n_layers"] + 1):
        cache.K, cache.V = list(snapK), list(snapV)
        info = []
        ref = O.decode_step(Wt, cfg, cache, token, pos, forced_experts=forced or None, info=info)
        new = {}
        for rec in info:
            l = rec["layer"]
            o_ids = sorted(int(e) for e in rec["ids"])
            d_ids = sorted(int(e) for e in dev_ids[l, slot])
            if o_ids == d_ids or l in forced:
                continue
            diff = set(o_ids) ^ set(d_ids)
            assert len(diff) == 2 and rec["margin"] < ROUTE_TIE, (
                f"layer {l}: device experts {d_ids} vs oracle {o_ids}, margin {rec['margin']}")
            new[l] = d_ids
            break  # later layers depend on this one: re-run before comparing them
        if not new:
            return ref, len(forced)
        forced.update(new)
    raise AssertionError("routing reconciliation did not converge")
