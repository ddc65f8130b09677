"""Host-only tests of the C-ABI library: symbols, config checks and the planner.

The dependency rule the planner implements is the MPK author's (Hacker News
thread, post #58): task B depends on task A when A writes tensor elements
that B reads.  The brute-force check below derives every task's read and
write regions from the documented meaning of its fields (include/mk.h,
mk_task.h) and verifies that every overlapping (writer, later reader) pair is
ordered by the planner's events, transitively; and that every region is
written by exactly one task per step.
"""
import os
import re

import pytest

from persistent_runtime_amd import mk
from persistent_runtime_amd.sol import waves
from synth.configs import LLAMA8B, LLAMA70B, MOE30B, TINY, truncated

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_library_exports_every_declared_symbol():
    hdr = open(os.path.join(ROOT, "include", "mk.h")).read()
    decl = set(re.findall(r"^\s*(?:int|void|const char \*)\s*(mk_\w+)\s*\(", hdr, re.M))
    assert decl, "no declarations parsed"
    assert decl == set(mk.EXPORTS), decl ^ set(mk.EXPORTS)
    for name in decl:
        assert hasattr(mk.lib, name), name


def _cfg(model, B=1, maxp=64, n_pages=None):
    return mk.make_config(model, max_batch=B, max_pages_per_seq=maxp, n_pages=n_pages)


STATIC = ("QKV", "OPROJ", "GATEUP", "DOWN", "ROUTER", "LMHEAD")


def _kdim(model, op):
    """Row length (input columns) of a static-weight GEMV."""
    if op == "OPROJ":
        return model["n_q_heads"] * model["head_dim"]
    if op == "DOWN":
        return model["ffn_dim"]
    return model["hidden"]


def _ksplit(model, t):
    """(k0, kc, ns, ks) of a matrix-core tile (rows_per_pass = kc | rb << 16
    for split-K tiles, the row length otherwise)."""
    K = _kdim(model, mk.OPS[t.op])
    kc = min(t.rows_per_pass & 0xFFFF, K)
    ns = -(-K // kc)
    return t.a3, kc, ns, t.a3 // kc


def _split_rows(t, ns, ks):
    """Rows (relative to a1) that split-K tile ks of ns writes."""
    rs = -(-t.a2 // ns)
    lo = min(t.a2, ks * rs)
    return lo, min(t.a2, lo + rs)


def _mfma(B, batched_mfma=0):
    """Whether a plan's static-weight GEMVs are matrix-core tiles: from 3 slots
    by default, from 2 on request, never beyond 64 (the models here have
    every row count a multiple of 16)."""
    if B > 64 or batched_mfma < 0:
        return False
    return B >= (2 if batched_mfma > 0 else 3)


def _check_graph(model, tasks, thr, B, mfma=False):
    T = len(tasks)
    sig = {}
    for i, t in enumerate(tasks):
        for k in range(t.n_sig):
            sig.setdefault(t.sig_ev[k], []).append(i)
    last_sig, last_phase = {}, {}
    for e, s in sig.items():
        # completions reported (runs report once; split attention reports one
        # per (slot, KV head) between its splits)
        assert thr[e] == sum(tasks[p].sig_count for p in s), (e, thr[e], len(s))
        last_sig[e] = max(s)
        last_phase[e] = max(tasks[p].phase for p in s)
    for i, t in enumerate(tasks):
        for k in range(t.n_wait):
            e = t.wait_ev[k]
            assert e in sig, f"task {i} waits on unsignalled event {e}"
            assert last_sig[e] < i, "ticket order must be topological"
            assert last_phase[e] < t.phase
    # GEMV tiles cover every weight row exactly once per layer
    L, H = model["n_layers"], model["hidden"]
    nq, nkv, hd = model["n_q_heads"], model["n_kv_heads"], model["head_dim"]
    cover = {}
    kcover = {}
    for t in tasks:
        op = mk.OPS[t.op]
        if mfma and op in STATIC:
            # matrix-core tiles: the column ranges of a row block tile the row
            k0, kc, ns, ks = _ksplit(model, t)
            kcover.setdefault((op, t.layer, t.a0, t.a1, t.a2), []).append(
                (k0, min(k0 + kc, _kdim(model, op))))
            if k0 != 0:
                continue
        if op in ("QKV", "OPROJ", "GATEUP", "DOWN", "ROUTER", "LMHEAD", "EGATEUP", "EDOWN"):
            m = (t.a0 if op == "QKV" else (t.a0, t.a3) if op == "EGATEUP"
                 else t.a0 if op == "EDOWN" else 0)
            cover.setdefault((op, t.layer, m), []).append((t.a1, t.a1 + t.a2))
    want = {"OPROJ": H, "LMHEAD": model["vocab"], "DOWN": H,
            "GATEUP": model["ffn_dim"], "ROUTER": model["n_experts"],
            "EGATEUP": model["expert_ffn_dim"], "EDOWN": H}
    for (op, l, m), rr in cover.items():
        rr.sort()
        n = (nq * hd if m == 0 else nkv * hd) if op == "QKV" else want[op]
        assert rr[0][0] == 0 and rr[-1][1] == n, (op, l, m)
        assert all(a[1] == b[0] for a, b in zip(rr, rr[1:])), (op, l, m)
    for key, kk in kcover.items():
        kk.sort()
        assert kk[0][0] == 0 and kk[-1][1] == _kdim(model, key[0]), key
        assert all(a[1] == b[0] for a, b in zip(kk, kk[1:])), key
    return sig


def _regions(model, t, B, S, mfma=False, shared=False):
    """(reads, writes) of one task, as lists of (buffer, layer, slot, sub, lo, hi)."""
    R, W = _regions_rows(model, t, B, S, shared)
    op = mk.OPS[t.op]
    if mfma and op in STATIC and op != "LMHEAD":
        # a split-K tile writes only its slice of the block's rows (summed
        # over the block's column ranges after they have all arrived; an
        # arrival counter, not an event, orders that)
        k0, kc, ns, ks = _ksplit(model, t)
        lo, hi = _split_rows(t, ns, ks)
        W = [(n, l, b, sub, a + lo, a + hi) for (n, l, b, sub, a, _) in W]
        R = [r for r in R if not (op in ("OPROJ", "DOWN") and r[4] == t.a1 and r[5] == t.a1 + t.a2)]
        if op in ("OPROJ", "DOWN"):
            src = "x" if op == "OPROJ" else "xmid"
            R += [(src, t.layer, b, 0, t.a1 + lo, t.a1 + hi) for b in range(B)]
    return R, W


def _regions_rows(model, t, B, S, shared=False):
    op = mk.OPS[t.op]
    l, H = t.layer, model["hidden"]
    nq, nkv, hd = model["n_q_heads"], model["n_kv_heads"], model["head_dim"]
    G = nq // nkv
    QD = nq * hd
    F, E, K = model["ffn_dim"], model["n_experts"], model["top_k"]
    Fe = model["expert_ffn_dim"]
    R, W = [], []
    allb = range(B)
    if op == "EMBED":
        W.append(("x", 0, t.a0, 0, 0, H))
    elif op == "QKV":
        name = "qkv"[t.a0]
        n = QD if t.a0 == 0 else nkv * hd
        for b in allb:
            R.append(("x", l, b, 0, 0, H))
            W.append((name, l, b, 0, t.a1, t.a1 + t.a2))
    elif op == "KVAPP":
        # shared-sequence plans, modelled as one prompt chunk: slot b holds
        # the sequence's b-th new position and stores its key/value there
        b = t.a0
        R += [("k", l, b, 0, 0, nkv * hd), ("v", l, b, 0, 0, nkv * hd)]
        W += [("cache", l, 0, g, b, b + 1) for g in range(nkv)]
    elif op == "ATTN":
        b, g, s = t.a0, t.a1, t.a2
        R.append(("q", l, b, 0, g * G * hd, (g + 1) * G * hd))
        if shared:  # every chunk position up to its own, from the cache
            R.append(("cache", l, 0, g, 0, b + 1))
        else:
            R += [("k", l, b, 0, g * hd, (g + 1) * hd), ("v", l, b, 0, g * hd, (g + 1) * hd)]
        if S > 1:
            # The split that arrives last merges the group's partials into
            # the attention output; an arrival counter, not an event, orders
            # it after the other splits, so the model credits the output to
            # the split that reports the group's completion (the last index).
            W.append(("part", l, b, g, s, s + 1))
            if s == S - 1:
                W.append(("attn", l, b, 0, g * G * hd, (g + 1) * G * hd))
        else:
            W.append(("attn", l, b, 0, g * G * hd, (g + 1) * G * hd))
    elif op == "OPROJ":
        for b in allb:
            R += [("attn", l, b, 0, 0, QD), ("x", l, b, 0, t.a1, t.a1 + t.a2)]
            W.append(("xmid", l, b, 0, t.a1, t.a1 + t.a2))
    elif op == "GATEUP":
        for b in allb:
            R.append(("xmid", l, b, 0, 0, H))
            W.append(("h", l, b, 0, t.a1, t.a1 + t.a2))
    elif op == "DOWN":
        for b in allb:
            R += [("h", l, b, 0, 0, F), ("xmid", l, b, 0, t.a1, t.a1 + t.a2)]
            W.append(("x", l + 1, b, 0, t.a1, t.a1 + t.a2))
    elif op == "ROUTER":
        for b in allb:
            R.append(("xmid", l, b, 0, 0, H))
            W.append(("rl", l, b, 0, t.a1, t.a1 + t.a2))
    elif op == "EGATEUP":
        # routes the slot itself from the router logits; the slot's first
        # task also publishes the routing (ids and weights)
        b, j = t.a0, t.a3
        R += [("rl", l, b, 0, 0, E), ("xmid", l, b, 0, 0, H)]
        W.append(("he", l, b, j, t.a1, t.a1 + t.a2))
        if t.a1 == 0 and j == 0:
            W.append(("tk", l, b, 0, 0, K))
    elif op == "EDOWN":
        # routes the slot itself from the router logits, then rows a1..a1+a2
        # of every routed expert, weighted sum + residual
        b = t.a0
        R += [("rl", l, b, 0, 0, E), ("xmid", l, b, 0, t.a1, t.a1 + t.a2)]
        R += [("he", l, b, j, 0, Fe) for j in range(K)]
        W.append(("x", l + 1, b, 0, t.a1, t.a1 + t.a2))
    elif op == "LMHEAD":
        for b in allb:
            R.append(("x", model["n_layers"], b, 0, 0, H))
            W += [("logits", 0, b, 0, t.a1, t.a1 + t.a2), ("amax", 0, b, 0, t.a4, t.a4 + 1)]
    elif op == "ARGMAX":
        R.append(("amax", 0, t.a0, 0, 0, 10 ** 9))
        W.append(("next", 0, t.a0, 0, 0, 1))
    return R, W


def _overlap(a, b):
    return a[:4] == b[:4] and a[4] < b[5] and b[4] < a[5]


def _bruteforce_deps(model, B, S=None, **optkw):
    opts = mk.default_options(n_cus=optkw.pop("n_cus", 8), **optkw)
    tasks, thr = mk.inspect_plan(_cfg(model, B=B, maxp=8), opts)
    mfma = _mfma(B, optkw.get("batched_mfma", 0))
    shared = optkw.get("shared_seqs", 0) > 0
    if shared:
        assert sum(1 for t in tasks if mk.OPS[t.op] == "KVAPP") == B * model["n_layers"]
    sig = _check_graph(model, tasks, thr, B, mfma)
    # S actually used: count ATTN tasks per (layer 0, slot 0, head 0)
    S = sum(1 for t in tasks if mk.OPS[t.op] == "ATTN" and t.layer == 0 and t.a0 == 0 and t.a1 == 0)
    T = len(tasks)
    anc = [0] * T  # bitset of ancestors
    for i, t in enumerate(tasks):
        a = 0
        for k in range(t.n_wait):
            for p in sig[t.wait_ev[k]]:
                a |= anc[p] | (1 << p)
        anc[i] = a
    regs = [_regions(model, t, B, S, mfma, shared) for t in tasks]
    written = []
    for i, (_, W) in enumerate(regs):
        for w in W:
            for (j, w2) in written:
                assert not _overlap(w, w2), f"region written twice: tasks {j} and {i}: {w}"
            written.append((i, w))
    n_edges = 0
    for c in range(T):
        for r in regs[c][0]:
            for (p, w) in written:
                if _overlap(r, w):
                    assert p < c, f"task {c} reads {r} written by later task {p}"
                    assert (anc[c] >> p) & 1, f"task {c} does not depend on producer {p} of {r}"
                    n_edges += 1
    # every read region that a step writes has a producer (no reads of stale data)
    return T, n_edges


@pytest.mark.parametrize("B,mfma", [(1, 0), (3, 0), (3, -1), (2, 1)])
def test_dependencies_match_region_overlap_tiny(B, mfma):
    T, n = _bruteforce_deps(TINY, B, batched_mfma=mfma)
    assert T > 0 and n > 0


def test_dependencies_match_region_overlap_tiny_split_attention():
    T, n = _bruteforce_deps(TINY, 2, attn_splits=3)
    assert n > 0


def test_dependencies_match_region_overlap_batched_split_k():
    """Matrix-core batch of 16 on 8 workers: the down projection is cut into
    column ranges (split-K); every tile writes its own slice of rows and the
    dependency structure still covers every read."""
    tasks, _ = mk.inspect_plan(_cfg(TINY, B=16, maxp=8), mk.default_options(n_cus=8))
    splits = [t for t in tasks if mk.OPS[t.op] == "DOWN" and _ksplit(TINY, t)[2] > 1]
    assert splits
    T, n = _bruteforce_deps(TINY, 16)
    assert n > 0


@pytest.mark.parametrize("B,mfma", [(3, 0), (3, -1), (16, 0)])
def test_dependencies_match_region_overlap_shared_sequences(B, mfma):
    """Shared-sequence plans (a prompt chunk's tokens in the slots): every
    attention task depends on the key/value stores of its own and every
    earlier position of the chunk (matrix cores at 3 and 16 slots, the vector
    path at 3, split attention)."""
    T, n = _bruteforce_deps(TINY, B, shared_seqs=1, attn_splits=2, batched_mfma=mfma)
    assert n > 0


def test_dependencies_match_region_overlap_moe():
    moe = dict(MOE30B, n_layers=2, hidden=512, n_q_heads=4, n_kv_heads=2,
               n_experts=16, top_k=4, expert_ffn_dim=256, vocab=512)
    T, n = _bruteforce_deps(moe, 2, attn_splits=2)
    assert n > 0


@pytest.mark.parametrize("model", [TINY, LLAMA8B, MOE30B, LLAMA70B], ids=lambda m: m["name"])
def test_full_size_plans_are_valid(model):
    for B in (1, 4):
        opts = mk.default_options(n_cus=256)
        tasks, thr = mk.inspect_plan(_cfg(model, B=B, maxp=40), opts)
        _check_graph(model, tasks, thr, B, mfma=_mfma(B))
        # weight bytes the tiles read = the model's per-step weight bytes
        wbytes = sum(t.bytes for t in tasks if mk.OPS[t.op] != "EMBED")
        assert wbytes > 0


def test_tile_bytes_8b():
    tasks, _ = mk.inspect_plan(_cfg(LLAMA8B, maxp=40), mk.default_options(n_cus=256))
    from persistent_runtime_amd.sol import weight_bytes_per_step
    tot = sum(t.bytes for t in tasks)
    # tasks read every weight once (norm gains are read by each tile: not counted)
    norms = LLAMA8B["n_layers"] * 2 * LLAMA8B["hidden"] * 2
    lm_norm_reads = sum(1 for t in tasks if mk.OPS[t.op] == "LMHEAD") * LLAMA8B["hidden"] * 2
    assert tot - lm_norm_reads == weight_bytes_per_step(LLAMA8B) - norms - LLAMA8B["hidden"] * 2


def test_invalid_configs_rejected():
    bad = [dict(TINY, head_dim=96), dict(TINY, n_q_heads=3), dict(TINY, hidden=200),
           dict(TINY, ffn_dim=0)]
    codes = []
    for m in bad:
        with pytest.raises(mk.MkError) as e:
            mk.inspect_plan(_cfg(m))
        codes.append(e.value.code)
    assert set(codes) <= {mk.MK_ERR_INVALID_CONFIG, mk.MK_ERR_UNSUPPORTED}
    c = _cfg(TINY)
    c.page_size = 8
    with pytest.raises(mk.MkError):
        mk.inspect_plan(c)


def test_gemv_shares_balanced_and_passes_fit():
    """Static-weight GEMVs of the 8B plan on 256 workgroups: every worker (for
    the output projection: every worker without attention tasks) gets a
    contiguous share of each operation whose bytes differ from the others'
    by at most one row, and every pass fits one tile (7 waves x (16 register
    + 8 LDS) chunks of 1 KiB at batch 1), at most 6 passes per task."""
    tasks, _ = mk.inspect_plan(_cfg(LLAMA8B, maxp=40), mk.default_options(n_cus=256))
    H, F, V = LLAMA8B["hidden"], LLAMA8B["ffn_dim"], LLAMA8B["vocab"]
    row_bytes = {"QKV": H * 2, "OPROJ": H * 2, "GATEUP": 2 * H * 2, "DOWN": F * 2,
                 "LMHEAD": H * 2}
    for op, rb in row_bytes.items():
        layer = LLAMA8B["n_layers"] if op == "LMHEAD" else 3
        sel = [t for t in tasks if mk.OPS[t.op] == op and t.layer == layer]
        per_worker = {}
        for t in sel:
            assert 0 < t.rows_per_pass <= t.a2
            passes = -(-t.a2 // t.rows_per_pass)
            assert passes <= 6, (op, passes)
            assert t.rows_per_pass * rb <= 7 * 24 * 1024, (op, t.rows_per_pass)
            assert (t.rows_per_pass * rb) % 1024 == 0
            per_worker[t.worker] = per_worker.get(t.worker, 0) + t.a2 * rb
        if op == "QKV":
            # shares follow the q/k/v boundaries: one task per worker, the
            # largest share within 10% of the mean; the workers that run
            # attention take none (they wait for q, k, v meanwhile)
            assert len(sel) == len(per_worker) >= 240, (op, len(sel), len(per_worker))
            mean = sum(per_worker.values()) / len(per_worker)
            assert max(per_worker.values()) <= 1.1 * mean, op
            attn = {t.worker for t in tasks if mk.OPS[t.op] == "ATTN" and t.layer == layer}
            assert attn and not attn & set(per_worker), op
            continue
        if op == "OPROJ":
            # attention (one task per KV head at this short context) runs on
            # workers of its own, the projection's rows on all the others
            attn = {t.worker for t in tasks if mk.OPS[t.op] == "ATTN" and t.layer == layer}
            assert 0 < len(attn) <= 64 and not attn & set(per_worker), op
            assert len(per_worker) + len(attn) == 256, (op, len(per_worker))
        else:
            assert len(per_worker) == 256, (op, len(per_worker))
        assert max(per_worker.values()) - min(per_worker.values()) <= rb, op
    # the rows of each operation are covered exactly once
    for op, total in (("GATEUP", F), ("DOWN", H), ("OPROJ", H), ("LMHEAD", V)):
        layer = LLAMA8B["n_layers"] if op == "LMHEAD" else 3
        rows = sorted((t.a1, t.a2) for t in tasks if mk.OPS[t.op] == op and t.layer == layer)
        pos = 0
        for r0, n in rows:
            assert r0 == pos
            pos += n
        assert pos == total, op


def test_truncated_model_plans():
    tasks, _ = mk.inspect_plan(_cfg(truncated(LLAMA8B, 2), maxp=40))
    assert sum(1 for t in tasks if mk.OPS[t.op] == "LMHEAD") > 0


def test_batched_plans_use_16_row_groups():
    """Batches of 16..64 slots: every static-weight GEMV task covers whole
    16-row groups, at most 14 per task (7 per matrix for gate/up); the
    dependency structure stays valid."""
    for model in (LLAMA8B, TINY):
        for B in (16, 64):
            tasks, thr = mk.inspect_plan(_cfg(model, B=B, maxp=8), mk.default_options(n_cus=256))
            _check_graph(model, tasks, thr, B, mfma=True)
            per_op = {}
            for t in tasks:
                op = mk.OPS[t.op]
                if op in ("QKV", "OPROJ", "GATEUP", "DOWN", "LMHEAD"):
                    assert t.a1 % 16 == 0 and t.a2 % 16 == 0, (op, t.a1, t.a2)
                    assert t.a2 // 16 <= (7 if op == "GATEUP" else 14), (op, t.a2)
                    k0, kc, ns, ks = _ksplit(model, t)
                    assert k0 % 32 == 0 and kc % 32 == 0 and 1 <= ns <= 16, (op, k0, kc, ns)
                    per_op.setdefault((op, t.layer), []).append((t, ns))
            for (op, l), tt in per_op.items():
                if max(ns for _, ns in tt) > 1:
                    # split operations: every tile on its own worker (the
                    # tiles of a block wait for each other)
                    assert len({t.worker for t, _ in tt}) == len(tt) <= 256, (op, l)
            if model is LLAMA8B:
                # the large batch splits K wherever the row blocks alone
                # would leave most workers idle
                assert any(ns > 1 for (op, l), tt in per_op.items() if op == "DOWN"
                           for _, ns in tt)


def test_claimed_attention_annotations():
    """Batches of 16 and more claim attention at run time: every ATTN task names its
    layer's first ATTN task (a4) and carries count | claims per step << 16
    (rpp); the first of each worker's consecutive entries of a layer holds
    their number (a3), and the entries of every layer add up to its count."""
    for B in (16, 64):
        tasks, thr = mk.inspect_plan(_cfg(LLAMA8B, B=B, maxp=1024),
                                     mk.default_options(n_cus=256, planned_ctx=16384))
        _check_graph(LLAMA8B, tasks, thr, B, mfma=_mfma(B))
        attn = [(i, t) for i, t in enumerate(tasks) if mk.OPS[t.op] == "ATTN"]
        assert len(attn) > 256, (B, len(attn))  # more tasks than workers: claimed
        by_layer = {}
        for i, t in attn:
            by_layer.setdefault(t.layer, []).append((i, t))
        for l, tt in by_layer.items():
            first, n = tt[0][0], len(tt)
            holders = sum(1 for _, t in tt if t.a3 > 0)
            assert sum(t.a3 for _, t in tt) == n
            for _, t in tt:
                assert t.a4 == first and t.rows_per_pass == n | (n + holders) << 16
            # a worker's entries of the layer are consecutive in its queue
            for _, t in tt:
                if t.a3 > 0:
                    run = [u for _, u in tt if u.worker == t.worker]
                    assert len(run) == t.a3
    for B in (1, 4):  # one task per worker or fewer: static placement
        tasks, _ = mk.inspect_plan(_cfg(LLAMA8B, B=B, maxp=1024),
                                   mk.default_options(n_cus=256, planned_ctx=16384))
        assert all(t.a3 == 0 for t in tasks if mk.OPS[t.op] == "ATTN")


def test_lds_weight_slots_only_where_the_stage_leaves_room():
    """Single-slot plans extend passes into LDS (up to 168 KiB) when every
    staged activation row fits 72 KiB; the 70B shape (28672-wide down
    projection rows) and batches on the vector path keep register-only passes
    (112 KiB)."""
    from synth.configs import LLAMA70B

    def max_pass(model, B, **kw):
        tasks, _ = mk.inspect_plan(_cfg(model, B=B, maxp=40), mk.default_options(n_cus=256, **kw))
        best = 0
        for t in tasks:
            op = mk.OPS[t.op]
            if op in ("QKV", "OPROJ", "GATEUP", "DOWN", "LMHEAD"):
                rb = (2 if op == "GATEUP" else 1) * 2 * _kdim(model, op)
                best = max(best, min(t.rows_per_pass, t.a2) * rb)
        return best
    assert 7 * 16 * 1024 < max_pass(LLAMA8B, 1) <= 7 * 24 * 1024
    assert max_pass(LLAMA8B, 1, weight_lds=-1) <= 7 * 16 * 1024
    assert max_pass(LLAMA70B, 1) <= 7 * 16 * 1024
    assert max_pass(LLAMA8B, 4, batched_mfma=-1) <= 7 * 16 * 1024
    # MoE: off unless asked for
    assert max_pass(MOE30B, 1) <= 7 * 16 * 1024 < max_pass(MOE30B, 1, weight_lds=1)


def test_single_split_for_short_single_sequence_contexts():
    """One sequence whose context is at most 768 keys keeps one split per KV
    head (no merge hop); longer contexts, and batches, keep the split count
    that covers the CUs."""
    def splits(ctx, B=1):
        tasks, _ = mk.inspect_plan(_cfg(LLAMA8B, B=B, maxp=(ctx + 15) // 16),
                                   mk.default_options(n_cus=256, planned_ctx=ctx))
        return sum(1 for t in tasks if mk.OPS[t.op] == "ATTN" and t.layer == 0 and t.a0 == 0
                   and t.a1 == 0)
    assert splits(551) == 1 and splits(768) == 1
    assert splits(769) == 6 and splits(1047) == 8
    assert splits(768, B=4) > 1


def test_split_counts_and_attention_worker_roles():
    """Split rule: at most 128 partials (query heads x splits) per merge, so
    the MoE shape (8 query heads per KV head) plans 16 splits at an
    8192-token context and the 8B shape (4 per KV head) 32 at 131072;
    claimed attention from 8 slots with 2 x workers / (KV heads x slots)
    splits.  Where attention has workers of its own (single sequence), they
    take no QKV rows, and on the MoE shape they hold the router rows."""
    def attn(tasks, layer=3):
        return [t for t in tasks if mk.OPS[t.op] == "ATTN" and t.layer == layer]
    moe, _ = mk.inspect_plan(_cfg(MOE30B, maxp=(8192 + 64) // 16),
                             mk.default_options(n_cus=256, planned_ctx=8192 + 64))
    a = attn(moe)
    assert max(t.a2 for t in a) + 1 == 16
    aw = {t.worker for t in a}
    assert len(aw) == len(a) == MOE30B["n_kv_heads"] * 16
    router = [t for t in moe if mk.OPS[t.op] == "ROUTER" and t.layer == 3]
    assert {t.worker for t in router} <= aw
    assert sum(t.a2 for t in router) == MOE30B["n_experts"]
    qkv = [t for t in moe if mk.OPS[t.op] == "QKV" and t.layer == 3]
    assert not {t.worker for t in qkv} & aw
    lc, _ = mk.inspect_plan(_cfg(LLAMA8B, maxp=(131072 + 64) // 16),
                            mk.default_options(n_cus=256, planned_ctx=131072 + 64))
    assert max(t.a2 for t in attn(lc)) + 1 == 32
    for B, S in ((8, 8), (16, 4), (32, 2), (64, 1)):
        tasks, _ = mk.inspect_plan(_cfg(LLAMA8B, B=B, maxp=1024),
                                   mk.default_options(n_cus=256, planned_ctx=16384))
        a = attn(tasks)
        assert max(t.a2 for t in a) + 1 == S, B
        assert all(t.a4 == a[0].a4 for t in a) and sum(t.a3 for t in a) == len(a), B  # claimed
