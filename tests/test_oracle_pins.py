"""Pins for the CPU oracle: each check ties it to something other than itself.

Kinds of pin used here: brute force on tiny inputs (pure-Python loops with
math.exp), closed forms, invariants, special cases that reduce to a textbook
or library routine (torch's own primitives, complex rotation), and the bound
between the fp32 oracle and its float64 shadow.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O
import synth
from synth.configs import TINY

RNG = np.random.default_rng(1234)


# ---------------------------------------------------------------- GEMV ------
def test_projection_matches_triple_loop():
    """The oracle's projection (W @ x on bf16-valued weights) against a
    brute-force loop, through a 1-layer tiny model's first op."""
    W = RNG.standard_normal((24, 40)).astype(np.float32)
    x = RNG.standard_normal(40).astype(np.float32)
    ref = [sum(float(W[i, j]) * float(x[j]) for j in range(40)) for i in range(24)]
    Wu = synth.to_numpy_bf16(torch.from_numpy(W).to(torch.bfloat16))
    Wt = O.OracleWeights({"w": Wu}, {}, np.float64)
    got = Wt.get("w") @ x.astype(np.float64)
    Wr = synth.bf16_to_f32_np(Wu).astype(np.float64)
    ref_r = [sum(Wr[i, j] * float(x[j]) for j in range(40)) for i in range(24)]
    assert np.max(np.abs(got - np.array(ref_r))) < 1e-12
    # bf16 rounding of the weights moves results by at most ~2^-8 relative
    assert np.max(np.abs(got - np.array(ref))) < 0.05


def test_bf16_upcast_exact():
    a = torch.tensor([1.0, -2.5, 3.140625, 1e-3, 65504.0]).to(torch.bfloat16)
    u = synth.to_numpy_bf16(a)
    assert np.array_equal(synth.bf16_to_f32_np(u), a.float().numpy())


# ------------------------------------------------------------- RMSNorm ------
def test_rmsnorm_closed_form_unit_gain():
    x = RNG.standard_normal((5, 64)).astype(np.float64) * 3.0
    eps = 1e-5
    y = O.rmsnorm(x, np.ones(64), eps, np.float64)
    ms = np.mean(x * x, axis=-1)
    assert np.allclose(np.mean(y * y, axis=-1), ms / (ms + eps), rtol=1e-12)


def test_rmsnorm_scale_invariance_and_gain():
    x = RNG.standard_normal(128)
    g = RNG.standard_normal(128)
    y1 = O.rmsnorm(x, g, 0.0, np.float64)
    y2 = O.rmsnorm(1000.0 * x, g, 0.0, np.float64)
    assert np.allclose(y1, y2, rtol=1e-12)
    assert np.allclose(y1 / g, O.rmsnorm(x, np.ones(128), 0.0, np.float64))


def test_rmsnorm_matches_torch():
    x = RNG.standard_normal((3, 256)).astype(np.float32)
    g = RNG.standard_normal(256).astype(np.float32)
    ref = F.rms_norm(torch.from_numpy(x), (256,), torch.from_numpy(g), eps=1e-5).numpy()
    assert np.allclose(O.rmsnorm(x, g, 1e-5), ref, atol=1e-5)


# ---------------------------------------------------------------- RoPE ------
def test_rope_frequencies_closed_form():
    hd, theta = 64, 10000.0
    cos, sin = O.rope_cos_sin([7], hd, theta, np.float64)
    for i in (0, 1, 17, 31):
        ang = 7 * math.pow(theta, -2.0 * i / hd)
        assert abs(cos[0, i] - math.cos(ang)) < 1e-15
        assert abs(sin[0, i] - math.sin(ang)) < 1e-15


def test_rope_identity_at_zero_and_norm_preserved():
    hd = 128
    v = RNG.standard_normal((3, hd))
    c0, s0 = O.rope_cos_sin([0], hd, 5e5, np.float64)
    assert np.array_equal(O.rope(v, c0[0], s0[0]), v)
    c, s = O.rope_cos_sin([12345], hd, 5e5, np.float64)
    r = O.rope(v, c[0], s[0])
    h = hd // 2
    assert np.allclose(v[:, :h] ** 2 + v[:, h:] ** 2, r[:, :h] ** 2 + r[:, h:] ** 2)


def test_rope_is_complex_rotation_of_half_pairs():
    """Rotate-half RoPE equals multiplying z_i = v_i + 1j v_{i+h} by e^{j p w_i}."""
    hd, theta, p = 64, 10000.0, 33
    v = RNG.standard_normal(hd)
    c, s = O.rope_cos_sin([p], hd, theta, np.float64)
    r = O.rope(v, c[0], s[0])
    h = hd // 2
    w = theta ** (-2.0 * np.arange(h) / hd)
    z = (v[:h] + 1j * v[h:]) * np.exp(1j * p * w)
    assert np.allclose(r[:h], z.real) and np.allclose(r[h:], z.imag)


def test_rope_relative_position():
    hd = 64
    q, k = RNG.standard_normal(hd), RNG.standard_normal(hd)

    def dot(m, n):
        cm, sm = O.rope_cos_sin([m], hd, 10000.0, np.float64)
        cn, sn = O.rope_cos_sin([n], hd, 10000.0, np.float64)
        return O.rope(q, cm[0], sm[0]) @ O.rope(k, cn[0], sn[0])

    assert abs(dot(10, 3) - dot(110, 103)) < 1e-9
    assert abs(dot(10, 3) - dot(57, 50)) < 1e-9


# ------------------------------------------------------------- softmax ------
def test_softmax_brute_force_and_sums():
    s = RNG.standard_normal((4, 9)) * 5
    p = O.softmax(s)
    for r in range(4):
        den = sum(math.exp(float(v)) for v in s[r])
        for j in range(9):
            assert abs(p[r, j] - math.exp(float(s[r, j])) / den) < 1e-14
    assert np.allclose(p.sum(axis=-1), 1.0, atol=1e-6)
    big = np.array([1000.0, 1001.0, 999.0], np.float32)
    assert np.isfinite(O.softmax(big)).all()
    assert abs(O.softmax(big).sum() - 1) < 1e-6


# ----------------------------------------------------------- attention ------
def _mha_bruteforce(q, K, V):
    nq, hd = q.shape
    out = np.zeros_like(q)
    for h in range(nq):
        sc = [sum(q[h, d] * K[t, h, d] for d in range(hd)) / math.sqrt(hd)
              for t in range(K.shape[0])]
        m = max(sc)
        e = [math.exp(x - m) for x in sc]
        z = sum(e)
        for d in range(hd):
            out[h, d] = sum(e[t] * V[t, h, d] for t in range(K.shape[0])) / z
    return out


def test_attention_single_position_returns_v():
    q = RNG.standard_normal((4, 16))
    K = RNG.standard_normal((1, 2, 16))
    V = RNG.standard_normal((1, 2, 16))
    o = O.attention(q, K, V, 2)
    assert np.allclose(o[0], V[0, 0]) and np.allclose(o[1], V[0, 0])
    assert np.allclose(o[2], V[0, 1]) and np.allclose(o[3], V[0, 1])


def test_attention_mha_brute_force():
    q = RNG.standard_normal((3, 8))
    K = RNG.standard_normal((5, 3, 8))
    V = RNG.standard_normal((5, 3, 8))
    assert np.allclose(O.attention(q, K, V, 3), _mha_bruteforce(q, K, V), atol=1e-12)


def test_attention_gqa_equals_repeated_mha_and_torch_sdpa():
    nq, nkv, hd, T = 8, 2, 16, 11
    q = RNG.standard_normal((nq, hd))
    K = RNG.standard_normal((T, nkv, hd))
    V = RNG.standard_normal((T, nkv, hd))
    o = O.attention(q, K, V, nkv)
    Kr = np.repeat(K, nq // nkv, axis=1)
    Vr = np.repeat(V, nq // nkv, axis=1)
    assert np.allclose(o, O.attention(q, Kr, Vr, nq), atol=1e-12)
    ref = F.scaled_dot_product_attention(
        torch.from_numpy(q)[:, None, :], torch.from_numpy(Kr).permute(1, 0, 2),
        torch.from_numpy(Vr).permute(1, 0, 2))[:, 0, :].numpy()
    assert np.allclose(o, ref, atol=1e-12)


def test_attention_split_lse_merge_equals_unsplit():
    """Splitting the keys into chunks, each giving (max, sum, weighted values),
    and merging with log-sum-exp weights reproduces the unsplit result."""
    hd, T = 16, 37
    q = RNG.standard_normal((1, hd))
    K = RNG.standard_normal((T, 1, hd))
    V = RNG.standard_normal((T, 1, hd))
    full = O.attention(q, K, V, 1)[0]
    parts = []
    for lo, hi in ((0, 5), (5, 20), (20, 37)):
        s = (K[lo:hi, 0] @ q[0]) / math.sqrt(hd)
        m = s.max()
        e = np.exp(s - m)
        parts.append((m, e.sum(), e @ V[lo:hi, 0]))
    M = max(p[0] for p in parts)
    num = sum(np.exp(m - M) * o for m, _, o in parts)
    den = sum(np.exp(m - M) * l for m, l, _ in parts)
    assert np.allclose(num / den, full, atol=1e-12)


# ------------------------------------------------------------- SwiGLU -------
def test_silu_against_torch_and_identities():
    z = RNG.standard_normal(1000).astype(np.float64) * 6
    assert np.allclose(O.silu(z), F.silu(torch.from_numpy(z)).numpy(), atol=1e-14)
    assert O.silu(np.float64(0.0)) == 0.0
    assert np.allclose(O.silu(-z), O.silu(z) - z, atol=1e-12)
    g, u = RNG.standard_normal(10), RNG.standard_normal(10)
    assert np.allclose(O.swiglu(g, u), F.silu(torch.from_numpy(g)).numpy() * u)


# ---------------------------------------------------------------- MoE -------
def test_route_topk_special_cases():
    r = RNG.standard_normal(16)
    ids, w, margin = O.route_topk(r, 16)
    assert np.array_equal(ids, np.arange(16))
    assert np.allclose(w, torch.softmax(torch.from_numpy(r), 0).numpy())
    assert margin == np.inf
    ids, w, margin = O.route_topk(r, 1)
    assert ids.tolist() == [int(np.argmax(r))] and w.tolist() == [1.0]
    ids, w, margin = O.route_topk(r, 5)
    assert np.all(np.diff(ids) > 0) and abs(w.sum() - 1) < 1e-12
    srt = np.sort(r)[::-1]
    assert abs(margin - (srt[4] - srt[5])) < 1e-15
    assert set(ids.tolist()) == set(np.argsort(-r)[:5].tolist())


def test_route_topk_ties_take_lower_index():
    r = np.array([0.0, 2.0, 1.0, 2.0, 1.0, 1.0])
    ids, w, margin = O.route_topk(r, 3)
    assert ids.tolist() == [1, 2, 3]          # among the 1.0 ties, index 2 wins
    assert margin == 0.0


def _tiny_moe_cfg(E=4, k=4):
    return dict(TINY, name="tinymoe", n_layers=1, ffn_dim=0, n_experts=E,
                top_k=k, expert_ffn_dim=32, hidden=64, n_q_heads=2,
                n_kv_heads=1, head_dim=32, vocab=50)


def test_moe_all_experts_equals_dense_softmax_mixture():
    cfg = _tiny_moe_cfg(E=4, k=4)
    W = {k: synth.to_numpy_bf16(v) for k, v in synth.make_weights(cfg).items()}
    Wt = O.OracleWeights(W, cfg, np.float64)
    b = RNG.standard_normal(64)
    y = O.model._ffn(Wt, cfg, 0, b, np.float64)
    r = torch.from_numpy(Wt.get("router", 0) @ b)
    p = torch.softmax(r, 0).numpy()
    ref = np.zeros(64)
    for e in range(4):
        Wg = torch.from_numpy(Wt.get("e_gate", 0, e))
        Wu = torch.from_numpy(Wt.get("e_up", 0, e))
        Wd = torch.from_numpy(Wt.get("e_down", 0, e))
        bt = torch.from_numpy(b)
        ref += p[e] * (Wd @ (F.silu(Wg @ bt) * (Wu @ bt))).numpy()
    assert np.allclose(y, ref, atol=1e-12)


def test_moe_top1_is_argmax_expert():
    cfg = _tiny_moe_cfg(E=4, k=1)
    W = {k: synth.to_numpy_bf16(v) for k, v in synth.make_weights(cfg).items()}
    Wt = O.OracleWeights(W, cfg, np.float64)
    b = RNG.standard_normal(64)
    info = []
    y = O.model._ffn(Wt, cfg, 0, b, np.float64, info=info)
    e = int(np.argmax(Wt.get("router", 0) @ b))
    assert info[0]["ids"].tolist() == [e]
    bt = torch.from_numpy(b)
    ref = (torch.from_numpy(Wt.get("e_down", 0, e)) @ (
        F.silu(torch.from_numpy(Wt.get("e_gate", 0, e)) @ bt) *
        (torch.from_numpy(Wt.get("e_up", 0, e)) @ bt))).numpy()
    assert np.allclose(y, ref, atol=1e-12)


# --------------------------------------------------------------- model ------
def _tiny_weights(cfg, dtype=np.float32):
    W = {k: synth.to_numpy_bf16(v) for k, v in synth.make_weights(cfg).items()}
    return W, O.OracleWeights(W, cfg, dtype)


def test_incremental_decode_equals_full_recompute_tiny():
    """The key invariant: logits of incremental decoding with a KV cache equal
    those of a full causal recompute, at every position."""
    cfg = TINY
    W, Wt = _tiny_weights(cfg, np.float64)
    toks = synth.make_prompt(20, cfg["vocab"]).tolist()
    full = O.forward_full(Wt, cfg, toks)
    cache = O.KVCache(cfg, np.float64)
    for p, t in enumerate(toks):
        lg = O.decode_step(Wt, cfg, cache, t, p)
        assert np.max(np.abs(lg - full[p])) < 1e-10, p


def test_full_forward_cache_equals_incremental_cache():
    cfg = TINY
    W, Wt = _tiny_weights(cfg, np.float64)
    toks = synth.make_prompt(17, cfg["vocab"]).tolist()
    _, fc = O.forward_full(Wt, cfg, toks, return_cache=True)
    ic = O.KVCache(cfg, np.float64)
    for p, t in enumerate(toks):
        O.decode_step(Wt, cfg, ic, t, p)
    for l in range(cfg["n_layers"]):
        assert np.allclose(fc.K[l], ic.K[l], atol=1e-12)
        assert np.allclose(fc.V[l], ic.V[l], atol=1e-12)
    # continuing from the full-forward cache gives the same next logits
    a = O.decode_step(Wt, cfg, fc, 5, 17)
    b = O.decode_step(Wt, cfg, ic, 5, 17)
    assert np.max(np.abs(a - b)) < 1e-10


def test_incremental_decode_equals_full_recompute_moe():
    cfg = dict(_tiny_moe_cfg(E=8, k=2), n_layers=2)
    W, Wt = _tiny_weights(cfg, np.float64)
    toks = synth.make_prompt(9, cfg["vocab"]).tolist()
    full = O.forward_full(Wt, cfg, toks)
    cache = O.KVCache(cfg, np.float64)
    for p, t in enumerate(toks):
        lg = O.decode_step(Wt, cfg, cache, t, p)
        assert np.max(np.abs(lg - full[p])) < 1e-10, p


def _torch_forward(W, cfg, toks, kv_bf16=False):
    """An independent composition of torch library primitives (rms_norm,
    complex-number rotation, causal SDPA with GQA, silu), float64; with
    kv_bf16 the rotated keys and the values pass through torch's bfloat16
    conversion (from float32) before attention."""
    t = lambda a: torch.from_numpy(synth.bf16_to_f32_np(a).astype(np.float64))
    T = len(toks)
    H, nq, nkv, hd = cfg["hidden"], cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    X = t(W["embed"])[torch.tensor(toks)]
    h = hd // 2
    w = cfg["rope_theta"] ** (-torch.arange(h, dtype=torch.float64) * 2 / hd)
    rot = torch.polar(torch.ones(T, h, dtype=torch.float64),
                      torch.arange(T, dtype=torch.float64)[:, None] * w[None])

    def rr(Z):  # [T, n, hd]
        z = torch.complex(Z[..., :h], Z[..., h:]) * rot[:, None, :]
        return torch.cat([z.real, z.imag], -1)

    for l in range(cfg["n_layers"]):
        A = F.rms_norm(X, (H,), t(W["attn_norm"][l]), eps=cfg["rms_eps"])
        Q = rr((A @ t(W["wq"][l]).T).view(T, nq, hd))
        K = rr((A @ t(W["wk"][l]).T).view(T, nkv, hd))
        V = (A @ t(W["wv"][l]).T).view(T, nkv, hd)
        if kv_bf16:
            K = K.float().to(torch.bfloat16).double()
            V = V.float().to(torch.bfloat16).double()
        o = F.scaled_dot_product_attention(Q.transpose(0, 1), K.transpose(0, 1),
                                           V.transpose(0, 1), is_causal=True,
                                           enable_gqa=True)
        X = X + o.transpose(0, 1).reshape(T, nq * hd) @ t(W["wo"][l]).T
        B = F.rms_norm(X, (H,), t(W["ffn_norm"][l]), eps=cfg["rms_eps"])
        X = X + (F.silu(B @ t(W["w_gate"][l]).T) * (B @ t(W["w_up"][l]).T)) @ t(W["w_down"][l]).T
    Hn = F.rms_norm(X, (H,), t(W["final_norm"]), eps=cfg["rms_eps"])
    return (Hn @ t(W["lm_head"]).T).numpy()


def test_full_forward_matches_independent_torch_composition():
    cfg = TINY
    W, Wt = _tiny_weights(cfg, np.float64)
    toks = synth.make_prompt(12, cfg["vocab"]).tolist()
    ours = O.forward_full(Wt, cfg, toks, kv_bf16=False)
    ref = _torch_forward(W, cfg, toks)
    assert np.max(np.abs(ours - ref)) < 1e-9


def test_full_forward_bf16_kv_matches_torch_composition():
    """With the cache in bfloat16 the oracle rounds K and V from its float32
    working values; torch rounds its own float32 values with its own
    conversion.  A rounding decision could differ only where the two float32
    values differ across a rounding boundary; on this seed none does, so the
    logits agree to float32 accuracy, while skipping the rounding moves them
    by about 2e-3."""
    cfg = TINY
    W, Wt = _tiny_weights(cfg, np.float32)
    toks = synth.make_prompt(12, cfg["vocab"]).tolist()
    ours = O.forward_full(Wt, cfg, toks)
    ref = _torch_forward(W, cfg, toks, kv_bf16=True)
    assert np.max(np.abs(ours.astype(np.float64) - ref)) < 1e-5
    plain = O.forward_full(Wt, cfg, toks, kv_bf16=False).astype(np.float64)
    assert np.max(np.abs(plain - ref)) > 5e-4


def test_round_bf16_against_torch_and_ties():
    g = np.random.default_rng(7)
    x = np.concatenate([g.standard_normal(20000) * 10.0 ** g.integers(-30, 30, 20000),
                        -g.standard_normal(1000)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    assert np.array_equal(O.round_bf16(x), ref)
    # ties go to the even neighbour: 1 + 2^-8 lies halfway between 1 and
    # 1 + 2^-7 (even: 1); 1 + 3*2^-8 halfway between 1 + 2^-7 (odd) and
    # 1 + 2^-6 (even)
    t = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 3.0, 0.5 + 2.0 ** -10])
    want = np.array([1.0, 1 + 2.0 ** -6, -1.0, 3.0, 0.5])
    assert np.array_equal(O.round_bf16(t), want)
    assert np.array_equal(O.round_bf16(t.astype(np.float32)), want.astype(np.float32))
    # idempotent, and at most half a bf16 ulp away
    r = O.round_bf16(x)
    assert np.array_equal(O.round_bf16(r), r)
    m, e = np.frexp(x.astype(np.float64))
    assert np.all(np.abs(r.astype(np.float64) - x) <= np.ldexp(1.0, e - 9))


def test_fp32_oracle_error_bound_vs_fp64_shadow():
    cfg = TINY
    W, Wt32 = _tiny_weights(cfg, np.float32)
    Wt64 = O.OracleWeights(W, cfg, np.float64)
    toks = synth.make_prompt(39, cfg["vocab"]).tolist()
    # the arithmetic error of the fp32 working type alone (no KV rounding,
    # whose decisions could flip between the two precisions)
    c32 = O.KVCache(cfg, np.float32, kv_bf16=False)
    c64 = O.KVCache(cfg, np.float64, kv_bf16=False)
    worst = 0.0
    for p, t in enumerate(toks):
        a = O.decode_step(Wt32, cfg, c32, t, p)
        b = O.decode_step(Wt64, cfg, c64, t, p)
        worst = max(worst, float(np.max(np.abs(a.astype(np.float64) - b))))
    assert worst < 1e-4, worst


def test_argmax_ties_and_margin():
    lg = np.array([0.1, 0.7, 0.7, -1.0])
    assert O.greedy_argmax(lg) == 1
    assert O.top2_margin(lg) == 0.0
    assert abs(O.top2_margin(np.array([3.0, 1.0, 2.5])) - 0.5) < 1e-15


# ------------------------------------------------- forced MoE routing -------
# The forced branch of the oracle's MoE block re-runs a step with the expert
# ids the device chose where the device took a legitimate near-tie decision
# (the router's k-th and (k+1)-th logits nearly equal).  It is pinned here on
# its own, since ordinary runs never take it.
def _torch_moe_block(Wt, layer, b, ids):
    """Independent torch composition of one MoE block with a given expert
    set: router logits by torch, softmax over the chosen logits by torch,
    expert SwiGLU MLPs by torch, summed in ascending expert id (float64)."""
    bt = torch.from_numpy(np.asarray(b, dtype=np.float64))
    r = torch.from_numpy(Wt.get("router", layer)) @ bt
    ids = sorted(int(e) for e in ids)
    w = torch.softmax(r[torch.tensor(ids)], 0)
    y = torch.zeros_like(bt)
    for we, e in zip(w, ids):
        Wg = torch.from_numpy(Wt.get("e_gate", layer, e))
        Wu = torch.from_numpy(Wt.get("e_up", layer, e))
        Wd = torch.from_numpy(Wt.get("e_down", layer, e))
        y = y + we * (Wd @ (F.silu(Wg @ bt) * (Wu @ bt)))
    return y.numpy(), w.numpy()


def test_moe_forced_own_routing_reproduces_unforced_exactly():
    """Forcing the oracle's own expert ids, given in any order, must leave
    every logit bit-identical (the forced ids are sorted and weighted from
    the same router logits)."""
    cfg = dict(_tiny_moe_cfg(E=8, k=3), n_layers=2)
    W, Wt = _tiny_weights(cfg, np.float32)
    toks = synth.make_prompt(6, cfg["vocab"]).tolist()
    c0, c1 = O.KVCache(cfg), O.KVCache(cfg)
    g = np.random.default_rng(5)
    for p, t in enumerate(toks):
        info = []
        a = O.decode_step(Wt, cfg, c0, t, p, info=info)
        forced = {d["layer"]: g.permutation(d["ids"]).tolist() for d in info}
        info2 = []
        b = O.decode_step(Wt, cfg, c1, t, p, forced_experts=forced, info=info2)
        assert np.array_equal(a, b), p
        for d1, d2 in zip(info, info2):
            assert np.array_equal(d1["ids"], d2["ids"])
            assert np.array_equal(d1["w"], d2["w"])


def test_moe_forced_swap_matches_torch_composition():
    """One routed expert swapped for an unrouted one: the block output and
    the routing weights (softmax over the forced set's own router logits)
    equal an independent torch composition; and the result differs from the
    unforced block, so the override is not ignored."""
    cfg = _tiny_moe_cfg(E=8, k=3)
    W, Wt = _tiny_weights(cfg, np.float64)
    b = RNG.standard_normal(64)
    info = []
    y0 = O.model._ffn(Wt, cfg, 0, b, np.float64, info=info)
    own = info[0]["ids"].tolist()
    out = [e for e in range(8) if e not in own]
    for drop in range(3):
        forced = [e for i, e in enumerate(own) if i != drop] + [out[drop]]
        info = []
        y = O.model._ffn(Wt, cfg, 0, b, np.float64, forced=forced[::-1], info=info)
        ref, w_ref = _torch_moe_block(Wt, 0, b, forced)
        assert info[0]["ids"].tolist() == sorted(forced)
        assert np.allclose(info[0]["w"], w_ref, rtol=0, atol=1e-14)
        assert np.max(np.abs(y - ref)) < 1e-12
        assert np.max(np.abs(y - y0)) > 1e-6


def test_moe_forced_layer_only_changes_that_layer():
    """Forcing one layer's routing leaves the steps' earlier layers alone: a
    forced swap in the last layer changes the logits, one in a layer whose
    own ids are forced back unchanged does not."""
    cfg = dict(_tiny_moe_cfg(E=8, k=2), n_layers=2)
    W, Wt = _tiny_weights(cfg, np.float64)
    info = []
    base = O.decode_step(Wt, cfg, O.KVCache(cfg, np.float64), 3, 0, info=info)
    own1 = info[1]["ids"].tolist()
    swap = [own1[0], next(e for e in range(8) if e not in own1)]
    info2 = []
    got = O.decode_step(Wt, cfg, O.KVCache(cfg, np.float64), 3, 0,
                        forced_experts={1: swap}, info=info2)
    assert np.array_equal(info2[0]["ids"], info[0]["ids"])
    assert info2[1]["ids"].tolist() == sorted(swap)
    assert np.max(np.abs(got - base)) > 1e-6
    same = O.decode_step(Wt, cfg, O.KVCache(cfg, np.float64), 3, 0,
                         forced_experts={0: info[0]["ids"].tolist()})
    assert np.array_equal(same, base)


# ------------------------------------ 8B-shaped spot checks (2 layers) ------
@pytest.fixture(scope="module")
def llama8b_l2():
    """The Llama-3-8B shape truncated to 2 layers (real per-layer shapes and
    the full 128256-row LM head), generated on the CPU."""
    cfg = synth.truncated(synth.MODELS["llama8b"], 2)
    W = {k: synth.to_numpy_bf16(v) for k, v in synth.make_weights(cfg).items()}
    return cfg, W


@pytest.mark.slow
def test_incremental_equals_full_recompute_llama8b_2layer(llama8b_l2):
    """Incremental decode equals the full causal recompute on the 8B shape
    (two layers), at every position of a 6-token sequence.  In fp32 with an
    unrounded cache the two summation orders agree within 1e-4.  With the
    bf16 cache a key computed in a different order can round to the other
    bf16 neighbour (one such flip moves a logit by ~2e-4), so the bf16-cache
    check runs in float64, where both orders give the same rounding."""
    cfg, W = llama8b_l2
    toks = synth.make_prompt(6, cfg["vocab"]).tolist()
    for dtype, kv_bf16, tol in ((np.float32, False, 1e-4), (np.float64, True, 1e-9)):
        Wt = O.OracleWeights(W, cfg, dtype)
        full = O.forward_full(Wt, cfg, toks, kv_bf16=kv_bf16)
        cache = O.KVCache(cfg, dtype, kv_bf16=kv_bf16)
        for p, t in enumerate(toks):
            lg = O.decode_step(Wt, cfg, cache, t, p)
            assert np.max(np.abs(lg - full[p])) <= tol, (dtype, p)
        del Wt


@pytest.mark.slow
def test_fp32_oracle_error_bound_llama8b_2layer(llama8b_l2):
    """The fp32 oracle against its float64 shadow on the 8B shape (two
    layers), cache unrounded: the working type's own error stays below 1e-4
    in every logit, far under the 3e-2 parity bound."""
    cfg, W = llama8b_l2
    Wt32 = O.OracleWeights(W, cfg, np.float32)
    Wt64 = O.OracleWeights(W, cfg, np.float64)
    toks = synth.make_prompt(4, cfg["vocab"]).tolist()
    c32 = O.KVCache(cfg, np.float32, kv_bf16=False)
    c64 = O.KVCache(cfg, np.float64, kv_bf16=False)
    worst = 0.0
    for p, t in enumerate(toks):
        a = O.decode_step(Wt32, cfg, c32, t, p)
        b = O.decode_step(Wt64, cfg, c64, t, p)
        worst = max(worst, float(np.max(np.abs(a.astype(np.float64) - b))))
    assert worst < 1e-4, worst
