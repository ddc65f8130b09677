"""Model shapes and workload recipes of the decode-step benchmarks.

Plain data: no arithmetic of the decode step lives here.  Both the HIP path
and the CPU oracle read these dictionaries.

Shapes follow the workloads described on the pages: the 39-token prompt with
greedy generation (Mirage MPK post summary, "MPK का मुख्य मूल्य"), the MoE with
30B total / 3.3B active parameters at 8K context and batch 1 (Cohere
megakernel article, "A szűk keresztmetszet a memória-sávszélesség"), ragged
continuous batching over paged attention (same article, "Folyamatos
batchkezelés"), and long contexts (same section, the 256K claim).
"""

PAGE_SIZE = 16  # tokens per KV page

# Fields not fixed by the pages (readings, stated in the design notes):
#   rms_eps = 1e-5 and norm gains = 1.0 everywhere; untied LM head;
#   MoE rope_theta = 1e6 (the usual value for this model family).
TINY = dict(
    name="tiny", n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2,
    head_dim=64, ffn_dim=1024, vocab=1024, rms_eps=1e-5, rope_theta=10000.0,
    n_experts=0, top_k=0, expert_ffn_dim=0,
)

LLAMA8B = dict(
    name="llama8b", n_layers=32, hidden=4096, n_q_heads=32, n_kv_heads=8,
    head_dim=128, ffn_dim=14336, vocab=128256, rms_eps=1e-5,
    rope_theta=500000.0, n_experts=0, top_k=0, expert_ffn_dim=0,
)

MOE30B = dict(
    name="moe30b", n_layers=48, hidden=2048, n_q_heads=32, n_kv_heads=4,
    head_dim=128, ffn_dim=0, vocab=151936, rms_eps=1e-5,
    rope_theta=1000000.0, n_experts=128, top_k=8, expert_ffn_dim=768,
)

LLAMA70B = dict(
    name="llama70b", n_layers=80, hidden=8192, n_q_heads=64, n_kv_heads=8,
    head_dim=128, ffn_dim=28672, vocab=128256, rms_eps=1e-5,
    rope_theta=500000.0, n_experts=0, top_k=0, expert_ffn_dim=0,
)

MODELS = {m["name"]: m for m in (TINY, LLAMA8B, MOE30B, LLAMA70B)}

# Workloads (prompt length, decode steps, batch).
WORKLOADS = {
    "tiny": dict(model="tiny", prompt_len=39, steps=16, batch=1),
    "llama8b": dict(model="llama8b", prompt_len=39, steps=512, batch=1),
    "moe30b": dict(model="moe30b", context=8192, steps=256, batch=1),
    "ragged": dict(model="llama8b", batches=(1, 4, 16, 64), ctx_lo=128,
                   ctx_hi=16384, steps=128, retire_p=1.0 / 32.0),
    "llama70b": dict(model="llama70b", prompt_len=39, steps=512, batch=1),
    "longctx": dict(model="llama8b", context=131072, steps=64, batch=1),
}

# Seeds (recorded with every run).
WEIGHT_SEED = 0
PROMPT_SEED = 1
KV_SEED = 2


def truncated(cfg, n_layers):
    """The same per-layer shapes with fewer layers (depth-truncated model)."""
    c = dict(cfg)
    c["n_layers"] = int(n_layers)
    c["name"] = f"{cfg['name']}_L{n_layers}"
    return c
