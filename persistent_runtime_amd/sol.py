"""Speed-of-light arithmetic for the decode step (bytes per step / HBM rate).

The bound is the one the Cohere megakernel article states ("A szűk
keresztmetszet a memória-sávszélesség"): decode is bound by memory bandwidth,
so the fastest possible step reads every weight it needs plus the KV cache
once at the full HBM rate.  The MPK summary ("MPK का मुख्य मूल्य") uses the same
bound with weights only.

Algorithmic bytes counted per step: every layer weight actually used (for MoE
only the routed experts plus the router), norm gains, the full LM head, one
embedding row per active sequence, and the K and V of every attended position
(the cached ones plus the one being written).  The unread part of the
embedding table is not counted.
"""
from __future__ import annotations

HBM_PEAK_BYTES_PER_S = 8.0e12  # MI355X HBM3E, published peak


def layer_weight_bytes(cfg: dict, experts_used: int | None = None) -> int:
    H = cfg["hidden"]
    nq, nkv, hd = cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    b = 2 * H * 2                                   # attn_norm + ffn_norm gains
    b += (nq * hd + 2 * nkv * hd) * H * 2           # wq, wk, wv
    b += H * nq * hd * 2                            # wo
    if cfg["n_experts"] == 0:
        b += 3 * cfg["ffn_dim"] * H * 2
    else:
        k = cfg["top_k"] if experts_used is None else experts_used
        b += cfg["n_experts"] * H * 2               # router
        b += k * 3 * cfg["expert_ffn_dim"] * H * 2
    return b


def weight_bytes_per_step(cfg: dict, batch: int = 1, include_embed_table=False,
                          experts_used: int | None = None) -> int:
    H, V = cfg["hidden"], cfg["vocab"]
    b = cfg["n_layers"] * layer_weight_bytes(cfg, experts_used)
    b += V * H * 2 + H * 2                          # LM head + final norm
    b += (V * H * 2) if include_embed_table else batch * H * 2
    return b


def kv_bytes_per_token(cfg: dict) -> int:
    return cfg["n_layers"] * 2 * cfg["n_kv_heads"] * cfg["head_dim"] * 2


def step_bytes(cfg: dict, attended, experts_used: int | None = None) -> int:
    """Algorithmic bytes of one step; `attended[b]` = positions sequence b
    attends to (cached ones + the current one); 0 for an empty slot."""
    active = sum(1 for a in attended if a > 0)
    return (weight_bytes_per_step(cfg, max(active, 1), experts_used=experts_used)
            + kv_bytes_per_token(cfg) * int(sum(attended)))


def sol_seconds(nbytes: float, bw: float = HBM_PEAK_BYTES_PER_S) -> float:
    return float(nbytes) / float(bw)


def sol_tokens_per_s(nbytes: float, batch: int = 1,
                     bw: float = HBM_PEAK_BYTES_PER_S) -> float:
    return batch / sol_seconds(nbytes, bw)


def waves(n_tiles: int, n_units: int):
    """Static round-robin of n_tiles over n_units: (waves, tiles in the last
    wave, units idle during the last wave)."""
    w = -(-n_tiles // n_units)
    tail = n_tiles - (w - 1) * n_units
    return w, tail, n_units - tail
