"""CPU oracle for the transformer decode step (test infrastructure only).

A plain, slow, obviously correct numpy implementation of what one decode step
computes: the layer list RMSNorm -> QKV projection -> RoPE -> attention over
the cached keys/values -> O projection -> SwiGLU MLP (or softmax router + top-k
expert MLPs) -> final RMSNorm -> LM head -> argmax.  The pages name these
operations (Cohere megakernel article, "Egyetlen tartós kernelre épül a
kiszolgálás" and "Honnan jön a gyorsulás?"; Mirage MPK summary, "Part 2.
Runtime", Worker) but print no formulas, so each function below is the plain
textbook definition of its operation; readings of points the pages leave open
are stated in the function docstrings.

This package is test infrastructure.  Only the test suite, the smoke check and
the benchmark's CPU-baseline leg may import it.  It shares no code with the HIP
path (persistent_runtime_amd) and imports nothing from it; its only shared
input is the seeded generator package `synth`.

Every function takes a numpy dtype (float32 by default, float64 for the
shadow run that bounds the oracle's own rounding error).

Parity pins: every function here is pinned by tests/test_oracle_pins.py
(brute force, closed forms, invariants).  The model-level outputs themselves
(logits, tokens of a random-weight model) have no printed values anywhere on
the pages and are pinned only through those invariants, chiefly "incremental
decode with a KV cache equals full causal recompute".
"""
from .model import (rmsnorm, rope_cos_sin, rope, softmax, attention, causal_attention, silu,
                    swiglu, route_topk, KVCache, OracleWeights, decode_step,
                    forward_full, greedy_argmax, top2_margin, round_bf16)

__all__ = ["rmsnorm", "rope_cos_sin", "rope", "softmax", "attention", "causal_attention", "silu",
           "swiglu", "route_topk", "KVCache", "OracleWeights", "decode_step",
           "forward_full", "greedy_argmax", "top2_margin", "round_bf16"]
