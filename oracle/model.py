"""Plain numpy definition of one transformer decode step (test infrastructure).

Weights are row-major [out_features, in_features] and a projection is W @ x.
Weights may be given as numpy uint16 arrays holding bf16 bit patterns (they are
upcast exactly on use) or as float arrays.

Citations name the page and its section: "Cohere" is the Cohere megakernel
article (aihirek.info), "MPK" is the Mirage Persistent Kernel summary
(news.hada.io).  The pages list the operations of a forward pass but print no
formulas; the readings of the open points are in each docstring.
"""
from __future__ import annotations

import numpy as np


# ----------------------------------------------------------------------------
# weights
# ----------------------------------------------------------------------------
def _up(a, dtype):
    """bf16 bit patterns (uint16) or floats -> `dtype`, exactly."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(dtype, copy=False)
    return a.astype(dtype, copy=False)


class OracleWeights:
    """Read-only view of a weight dictionary for the oracle.

    `W` maps names to arrays: embed [V,H], lm_head [V,H], final_norm [H],
    attn_norm/ffn_norm [L,H], wq/wk/wv/wo [L,...], w_gate/w_up/w_down [L,...]
    for dense layers or router [L,E,H], e_gate/e_up [L,E,Fe,H], e_down
    [L,E,H,Fe] for MoE layers.  Arrays are upcast to `dtype` when fetched;
    `cache=True` keeps the upcast copies (fast repeated use, more memory).
    """

    def __init__(self, W: dict, cfg: dict, dtype=np.float32, cache=True):
        self.W, self.cfg, self.dtype, self._cache = W, cfg, dtype, {} if cache else None

    def get(self, name, *idx):
        key = (name,) + idx
        if self._cache is not None and key in self._cache:
            return self._cache[key]
        a = self.W[name]
        for i in idx:
            a = a[i]
        a = _up(a, self.dtype)
        if self._cache is not None:
            self._cache[key] = a
        return a

    def embed_row(self, token):
        return _up(self.W["embed"][int(token)], self.dtype)


# ----------------------------------------------------------------------------
# primitives
# ----------------------------------------------------------------------------
def round_bf16(x):
    """Round to the nearest bfloat16 value (ties to even), kept in x's dtype.

    bfloat16 keeps 8 significant bits and fp32's exponent range.  With
    x = m * 2^e and 0.5 <= |m| < 1, the result is rint(m * 2^8) * 2^(e-8),
    where rint rounds half to even.  Values are assumed inside the normal
    range (|x| >= 2^-126), which holds for every cached key and value here.
    """
    x = np.asarray(x)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(m * 256.0), e - 8).astype(x.dtype, copy=False)


def rmsnorm(x, g, eps, dtype=np.float32):
    """RMSNorm: x / sqrt(mean(x^2) + eps) * g, over the last axis.

    The pages name the norm only as part of the layer list; this is the
    standard definition (reading: eps = 1e-5 and gains 1.0 for every model).
    """
    x = np.asarray(x, dtype=dtype)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + dtype(eps)) * np.asarray(g, dtype=dtype)


def rope_cos_sin(positions, head_dim, theta, dtype=np.float32):
    """cos/sin of the rotary angles p * theta^(-2i/head_dim), i < head_dim/2.

    Reading: angles and their cos/sin are computed in float64 and rounded once
    to `dtype`; no long-context frequency scaling.  Returns arrays of shape
    [len(positions), head_dim/2].
    """
    half = head_dim // 2
    i = np.arange(half, dtype=np.float64)
    inv_freq = np.power(np.float64(theta), -2.0 * i / head_dim)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv_freq[None, :]
    return np.cos(ang).astype(dtype), np.sin(ang).astype(dtype)


def rope(v, cos, sin):
    """Rotate-half rotary embedding of the last axis of v (length head_dim).

    Reading: element i pairs with i + head_dim/2:
      out_i          = v_i cos_i - v_{i+h} sin_i
      out_{i+h}      = v_i sin_i + v_{i+h} cos_i.
    `cos`/`sin` broadcast against v[..., :h].
    """
    h = v.shape[-1] // 2
    a, b = v[..., :h], v[..., h:]
    return np.concatenate([a * cos - b * sin, a * sin + b * cos], axis=-1)


def softmax(s, axis=-1):
    """Max-subtracted softmax along `axis`."""
    m = np.max(s, axis=axis, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=axis, keepdims=True)


def attention(q, K, V, n_kv_heads):
    """Scaled dot-product attention of one query position over T keys (GQA).

    q: [nq, hd] (already rotated); K, V: [T, nkv, hd].  Query head h reads KV
    head g = h // (nq / nkv) (contiguous groups).  Scale 1/sqrt(hd), no bias,
    no soft-cap.  Returns o: [nq, hd].
    """
    nq, hd = q.shape
    group = nq // n_kv_heads
    out = np.empty_like(q)
    scale = q.dtype.type(1.0 / np.sqrt(hd))
    for h in range(nq):
        g = h // group
        s = (K[:, g, :] @ q[h]) * scale          # [T]
        p = softmax(s)
        out[h] = p @ V[:, g, :]
    return out


def silu(z):
    """silu(z) = z / (1 + exp(-z))."""
    return z / (z.dtype.type(1.0) + np.exp(-z))


def swiglu(gate, up):
    """SwiGLU activation: silu(gate) * up."""
    return silu(gate) * up


def route_topk(r, k):
    """Softmax router with top-k selection and renormalised weights.

    Reading: softmax over all experts, keep the k largest, renormalise over
    those k.  That equals a softmax over the k selected logits, which is what
    is computed.  Ties break toward the lower expert index (stable sort).
    Returns (ids ascending, weights in the same order, boundary margin
    r_(k) - r_(k+1) between the k-th and (k+1)-th largest logits; +inf when
    k equals the number of experts).
    """
    order = np.argsort(-r, kind="stable")
    sel = order[:k]
    margin = np.inf if k >= r.shape[0] else float(r[order[k - 1]] - r[order[k]])
    ids = np.sort(sel)
    logit = r[ids]
    w = np.exp(logit - np.max(logit))
    w = w / np.sum(w)
    return ids, w, margin


def greedy_argmax(logits):
    """Index of the largest logit; the lowest index wins an exact tie."""
    return int(np.argmax(logits))


def top2_margin(logits):
    """Gap between the largest and the second largest logit."""
    part = np.partition(np.asarray(logits, dtype=np.float64), -2)[-2:]
    return float(part[1] - part[0])


# ----------------------------------------------------------------------------
# the model
# ----------------------------------------------------------------------------
class KVCache:
    """Per-layer cached keys/values of one sequence, [T, nkv, hd] each.

    Reading: the cache stores keys (after the rotary embedding) and values in
    bfloat16, the model's storage type (the pages keep the KV cache in paged
    HBM blocks and name no other format); attention reads the stored values,
    the current token's included.  With kv_bf16=True entries are rounded to
    bfloat16 when stored (held in the working dtype); kv_bf16=False keeps
    them unrounded.
    """

    def __init__(self, cfg, dtype=np.float32, K=None, V=None, kv_bf16=True):
        L = cfg["n_layers"]
        nkv, hd = cfg["n_kv_heads"], cfg["head_dim"]
        self.kv_bf16 = kv_bf16
        if K is None:
            self.K = [np.zeros((0, nkv, hd), dtype) for _ in range(L)]
            self.V = [np.zeros((0, nkv, hd), dtype) for _ in range(L)]
        else:
            self.K = [self._store(np.asarray(K[l], dtype=dtype)) for l in range(L)]
            self.V = [self._store(np.asarray(V[l], dtype=dtype)) for l in range(L)]

    def _store(self, a):
        return round_bf16(a) if self.kv_bf16 else a

    def length(self):
        return self.K[0].shape[0]

    def append(self, layer, k, v):
        self.K[layer] = np.concatenate([self.K[layer], self._store(k)[None]], axis=0)
        self.V[layer] = np.concatenate([self.V[layer], self._store(v)[None]], axis=0)


def _ffn(Wt, cfg, layer, b, dtype, forced=None, info=None):
    """The feed-forward block on the normalised input b: returns its output."""
    if cfg["n_experts"] == 0:
        g = Wt.get("w_gate", layer) @ b
        u = Wt.get("w_up", layer) @ b
        return Wt.get("w_down", layer) @ swiglu(g, u)
    r = Wt.get("router", layer) @ b
    ids, w, margin = route_topk(r, cfg["top_k"])
    if forced is not None:
        ids = np.sort(np.asarray(forced, dtype=np.int64))
        logit = r[ids]
        w = np.exp(logit - np.max(logit))
        w = w / np.sum(w)
    if info is not None:
        info.append(dict(layer=layer, ids=ids.copy(), w=w.copy(), margin=margin,
                         logits=r.copy()))
    y = np.zeros_like(b)
    for e, we in zip(ids, w):          # ascending expert id
        # per-expert slices are upcast on demand (the full MoE does not fit)
        Wg = _up(Wt.W["e_gate"][layer][e], dtype)
        Wu = _up(Wt.W["e_up"][layer][e], dtype)
        Wd = _up(Wt.W["e_down"][layer][e], dtype)
        y = y + dtype(we) * (Wd @ swiglu(Wg @ b, Wu @ b))
    return y


def decode_step(Wt: OracleWeights, cfg: dict, cache: KVCache, token: int,
                pos: int, forced_experts=None, info=None, return_hidden=False):
    """One incremental decode step: feed `token` at position `pos`.

    `pos` equals the cache length before the call (the token's 0-based index);
    its key and value are appended.  Returns the logits [vocab].
    `forced_experts` (MoE only): {layer: ids} routing override used to re-check
    a step where the device took a legitimate near-tie routing decision.
    `info`: optional list collecting per-layer router decisions.
    """
    dtype = Wt.dtype
    assert cache.length() == pos, (cache.length(), pos)
    L, eps = cfg["n_layers"], cfg["rms_eps"]
    nq, nkv, hd = cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    cos, sin = rope_cos_sin([pos], hd, cfg["rope_theta"], dtype)
    x = Wt.embed_row(token).astype(dtype)
    for l in range(L):
        a = rmsnorm(x, Wt.get("attn_norm", l), eps, dtype)
        q = (Wt.get("wq", l) @ a).reshape(nq, hd)
        k = (Wt.get("wk", l) @ a).reshape(nkv, hd)
        v = (Wt.get("wv", l) @ a).reshape(nkv, hd)
        q = rope(q, cos[0], sin[0])
        k = rope(k, cos[0], sin[0])
        cache.append(l, k, v)
        o = attention(q, cache.K[l], cache.V[l], nkv)
        x = x + Wt.get("wo", l) @ o.reshape(nq * hd)
        b = rmsnorm(x, Wt.get("ffn_norm", l), eps, dtype)
        forced = None if forced_experts is None else forced_experts.get(l)
        x = x + _ffn(Wt, cfg, l, b, dtype, forced, info)
    h = rmsnorm(x, Wt.get("final_norm"), eps, dtype)
    logits = Wt.get("lm_head") @ h
    return (logits, x) if return_hidden else logits


def causal_attention(Q, K, V, n_kv_heads):
    """Causal attention of T query positions over the same T positions (GQA).

    Q: [T, nq, hd] (rotated); K, V: [T, nkv, hd].  For every head the T x T
    score matrix (Q_h K_g^T) / sqrt(hd) is masked above the diagonal (position
    t sees keys 0..t), softmax is taken along each row and the rows weight V_g:
    the textbook masked-attention definition, in matrix form.  Returns
    [T, nq, hd].
    """
    T, nq, hd = Q.shape
    group = nq // n_kv_heads
    out = np.empty_like(Q)
    scale = Q.dtype.type(1.0 / np.sqrt(hd))
    future = np.triu(np.ones((T, T), dtype=bool), k=1)
    for h in range(nq):
        g = h // group
        s = (Q[:, h, :] @ K[:, g, :].T) * scale       # [T, T]
        s[future] = -np.inf
        out[:, h, :] = softmax(s, axis=-1) @ V[:, g, :]
    return out


def _ffn_tokens(Wt, cfg, layer, B, dtype):
    """The feed-forward block for every row of B [T, H] at once.

    Dense: the SwiGLU MLP as matrix products.  MoE: each token is routed by
    route_topk exactly as in the single-token block; then, expert by expert
    in ascending id, the tokens routed to that expert pass through its MLP
    together and their weighted outputs are added to their rows (so every
    row still sums its experts in ascending id)."""
    if cfg["n_experts"] == 0:
        G = B @ Wt.get("w_gate", layer).T
        U = B @ Wt.get("w_up", layer).T
        return swiglu(G, U) @ Wt.get("w_down", layer).T
    R = B @ Wt.get("router", layer).T                  # [T, E]
    T, E = R.shape
    W = np.zeros((T, E), dtype=dtype)
    chosen = np.zeros((T, E), dtype=bool)
    for t in range(T):
        ids, w, _ = route_topk(R[t], cfg["top_k"])
        W[t, ids] = w
        chosen[t, ids] = True
    Y = np.zeros_like(B)
    for e in range(E):
        rows = np.nonzero(chosen[:, e])[0]
        if rows.size == 0:
            continue
        Wg = _up(Wt.W["e_gate"][layer][e], dtype)
        Wu = _up(Wt.W["e_up"][layer][e], dtype)
        Wd = _up(Wt.W["e_down"][layer][e], dtype)
        Be = B[rows]
        Y[rows] += W[rows, e][:, None] * (swiglu(Be @ Wg.T, Be @ Wu.T) @ Wd.T)
    return Y


def forward_full(Wt: OracleWeights, cfg: dict, tokens, return_cache=False, kv_bf16=True,
                 last_only=False):
    """Full causal forward over a whole token sequence (no cache reuse).

    Position t attends to positions 0..t, reading keys and values in the
    cache's storage format (kv_bf16 as in KVCache).  Returns logits
    [T, vocab] ([1, vocab] of the last position with last_only).  This is
    the recompute that incremental decoding must reproduce.  With
    return_cache=True it also returns the rotated keys and values it
    computed, as a KVCache ready for incremental decoding from position T.
    """
    cache = KVCache(cfg, Wt.dtype, kv_bf16=kv_bf16) if return_cache else None
    dtype = Wt.dtype
    tokens = [int(t) for t in tokens]
    T = len(tokens)
    L, eps = cfg["n_layers"], cfg["rms_eps"]
    nq, nkv, hd = cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    cos, sin = rope_cos_sin(np.arange(T), hd, cfg["rope_theta"], dtype)
    X = np.stack([Wt.embed_row(t).astype(dtype) for t in tokens])       # [T, H]
    for l in range(L):
        A = rmsnorm(X, Wt.get("attn_norm", l), eps, dtype)
        Q = (A @ Wt.get("wq", l).T).reshape(T, nq, hd)
        Kx = (A @ Wt.get("wk", l).T).reshape(T, nkv, hd)
        Vx = (A @ Wt.get("wv", l).T).reshape(T, nkv, hd)
        Q = rope(Q, cos[:, None, :], sin[:, None, :])
        Kx = rope(Kx, cos[:, None, :], sin[:, None, :])
        if kv_bf16:
            Kx, Vx = round_bf16(Kx), round_bf16(Vx)
        if cache is not None:
            cache.K[l], cache.V[l] = Kx.copy(), Vx.copy()
        O = causal_attention(Q, Kx, Vx, nkv)
        X = X + O.reshape(T, nq * hd) @ Wt.get("wo", l).T
        B = rmsnorm(X, Wt.get("ffn_norm", l), eps, dtype)
        X = X + _ffn_tokens(Wt, cfg, l, B, dtype)
    Hn = rmsnorm(X[-1:] if last_only else X, Wt.get("final_norm"), eps, dtype)
    logits = Hn @ Wt.get("lm_head").T
    return (logits, cache) if return_cache else logits
