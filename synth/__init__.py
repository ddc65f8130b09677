"""Seeded synthetic inputs shared by the HIP path's harness and the CPU oracle.

This module only draws random numbers and lays them out; it holds none of the
decode step's arithmetic.  Every tensor is drawn from its own torch.Generator,
seeded from (weight seed, tensor kind, layer), so a layer's values do not depend
on how many layers are generated (a depth-truncated model has the same first
layers as the full one) nor on the order of generation.

Weights are N(0, 0.02^2) drawn in fp32 and rounded to bf16 with
round-to-nearest-even (torch's fp32 -> bf16 conversion).  Norm gains are 1.0.
Weight matrices are row-major [out_features, in_features]: y = W @ x.
"""
from __future__ import annotations

import torch

from .configs import (MODELS, WORKLOADS, PAGE_SIZE, WEIGHT_SEED, PROMPT_SEED,
                      KV_SEED, truncated)

__all__ = ["MODELS", "WORKLOADS", "PAGE_SIZE", "WEIGHT_SEED", "PROMPT_SEED",
           "KV_SEED", "truncated", "make_weights", "make_prompt",
           "make_kv_values", "weight_shapes", "tensor_seed", "bf16_to_f32_np",
           "to_numpy_bf16", "ragged_schedule"]

# kind index -> name; the index enters the per-tensor seed
_KINDS = ["embed", "lm_head", "wq", "wk", "wv", "wo", "w_gate", "w_up",
          "w_down", "router", "e_gate", "e_up", "e_down"]
_KIND_ID = {k: i for i, k in enumerate(_KINDS)}
STD = 0.02


def tensor_seed(seed: int, kind: str, layer: int = 0) -> int:
    return (int(seed) << 24) + (_KIND_ID[kind] << 16) + int(layer) + 1


def weight_shapes(cfg: dict) -> dict:
    """Per-layer shapes of every random tensor (global ones have layer 0)."""
    H, V = cfg["hidden"], cfg["vocab"]
    nq, nkv, hd = cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    s = {"embed": (V, H), "lm_head": (V, H),
         "wq": (nq * hd, H), "wk": (nkv * hd, H), "wv": (nkv * hd, H),
         "wo": (H, nq * hd)}
    if cfg["n_experts"] == 0:
        F = cfg["ffn_dim"]
        s.update(w_gate=(F, H), w_up=(F, H), w_down=(H, F))
    else:
        E, Fe = cfg["n_experts"], cfg["expert_ffn_dim"]
        s.update(router=(E, H), e_gate=(E, Fe, H), e_up=(E, Fe, H),
                 e_down=(E, H, Fe))
    return s


def _randn_bf16(shape, seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    t.mul_(STD)
    return t.to(torch.bfloat16)


def make_weights(cfg: dict, device="cpu", seed: int = WEIGHT_SEED) -> dict:
    """All weights of `cfg` as bf16 torch tensors on `device`.

    Per-layer tensors are stacked along a leading layer axis:
    wq [L, nq*hd, H], ..., e_gate [L, E, Fe, H].
    """
    L, H = cfg["n_layers"], cfg["hidden"]
    shapes = weight_shapes(cfg)
    W = {}
    for kind in ("embed", "lm_head"):
        W[kind] = _randn_bf16(shapes[kind], tensor_seed(seed, kind), device)
    ones = torch.ones(H, dtype=torch.bfloat16, device=device)
    W["final_norm"] = ones.clone()
    W["attn_norm"] = ones.repeat(L, 1)
    W["ffn_norm"] = ones.repeat(L, 1)
    for kind, shp in shapes.items():
        if kind in ("embed", "lm_head"):
            continue
        out = torch.empty((L,) + tuple(shp), dtype=torch.bfloat16, device=device)
        for l in range(L):
            out[l] = _randn_bf16(shp, tensor_seed(seed, kind, l), device)
        W[kind] = out
    return W


def make_prompt(n: int, vocab: int, seed: int = PROMPT_SEED) -> torch.Tensor:
    """n token ids uniform in [0, vocab), int32, on the CPU."""
    g = torch.Generator()
    g.manual_seed(int(seed))
    return torch.randint(0, vocab, (n,), generator=g, dtype=torch.int64).to(torch.int32)


def kv_std(cfg: dict) -> float:
    """Std of synthetic K/V entries: that of W x for W ~ N(0, 0.02^2) and an
    input of unit RMS, i.e. 0.02 * sqrt(hidden)."""
    return STD * float(cfg["hidden"]) ** 0.5


def make_kv_values(cfg: dict, n_tokens: int, seed: int = KV_SEED,
                   device="cpu", stream_id: int = 0):
    """Synthetic cached keys and values for one sequence of n_tokens tokens.

    Returns (K, V), each bf16 [n_layers, n_tokens, n_kv_heads, head_dim],
    N(0, kv_std^2) rounded to bf16.  `stream_id` separates sequences.
    """
    L, nkv, hd = cfg["n_layers"], cfg["n_kv_heads"], cfg["head_dim"]
    sd = kv_std(cfg)
    out = []
    for which in (0, 1):
        g = torch.Generator(device=device)
        g.manual_seed((int(seed) << 32) + (int(stream_id) << 1) + which + 7)
        t = torch.randn((L, n_tokens, nkv, hd), generator=g, device=device,
                        dtype=torch.float32)
        t.mul_(sd)
        out.append(t.to(torch.bfloat16))
    return out[0], out[1]


def to_numpy_bf16(t: torch.Tensor):
    """bf16 torch tensor -> numpy uint16 array holding the same bit patterns."""
    import numpy as np
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def bf16_to_f32_np(a):
    """numpy uint16 bf16 bit patterns -> float32 with identical values."""
    import numpy as np
    return (a.astype(np.uint32) << 16).view(np.float32)


def ragged_schedule(B: int, steps: int, ctx_lo: int = 128, ctx_hi: int = 16384,
                    retire_p: float = 1.0 / 32.0, seed: int = KV_SEED) -> dict:
    """Seeded continuous-batching schedule for B slots over `steps` steps.

    Every slot starts with a sequence whose cached context is uniform in
    [ctx_lo, ctx_hi] (inclusive).  Before each step after the first, every
    slot's sequence retires with probability retire_p and a new sequence with
    a fresh uniform context joins the same slot.  Each sequence has its own
    stream id (its synthetic KV draws: `make_kv_values(..., stream_id=sid)`).

    Returns {"ctx0": [B] initial contexts, "sid0": [B] stream ids,
    "joins": [steps] lists of (slot, context, stream id), "pos": [steps][B]
    the position each slot feeds at each step (its cached length)}.
    """
    g = torch.Generator()
    g.manual_seed((int(seed) << 20) + 0x5A17 + int(B))
    def draw_ctx():
        return int(torch.randint(ctx_lo, ctx_hi + 1, (1,), generator=g))
    ctx = [draw_ctx() for _ in range(B)]
    sid = list(range(B))
    nxt = B
    out = {"ctx0": list(ctx), "sid0": list(sid), "joins": [], "pos": []}
    for k in range(steps):
        joins = []
        if k > 0:
            u = torch.rand(B, generator=g)
            for b in range(B):
                if float(u[b]) < retire_p:
                    ctx[b] = draw_ctx()
                    sid[b] = nxt
                    nxt += 1
                    joins.append((b, ctx[b], sid[b]))
        out["joins"].append(joins)
        out["pos"].append(list(ctx))
        ctx = [c + 1 for c in ctx]
    return out
