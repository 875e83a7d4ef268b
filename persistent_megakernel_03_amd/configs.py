"""Model shapes and workloads.

The pages name no architecture (they give only total and active parameter
counts, "Cohere Publishes One-Kernel Server for North Mini Code, Claims 1.58x
vLLM Speedup", section "The delay is between operations"); the two shapes
below are synthetic stand-ins: a tiny decoder that a CPU reference finishes in
seconds, and a 30B-total / 3.3B-active MoE whose per-token weight stream is
close to the pages' 6.6 GB.
"""

TINY = dict(
    n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
    n_experts=8, top_k=2, moe_inter=128, vocab=1024, page_size=16,
    rms_eps=1e-6, rope_theta=10000.0,
)

A3B = dict(
    n_layers=48, hidden=2048, n_q_heads=32, n_kv_heads=4, head_dim=128,
    n_experts=128, top_k=8, moe_inter=768, vocab=151936, page_size=16,
    rms_eps=1e-6, rope_theta=10000.0,
)

# A micro shape small enough for pure-Python brute force.
MICRO = dict(
    n_layers=1, hidden=8, n_q_heads=2, n_kv_heads=1, head_dim=4,
    n_experts=4, top_k=2, moe_inter=4, vocab=16, page_size=2,
    rms_eps=1e-6, rope_theta=10000.0,
)

WORKLOADS = {
    # tiny decoder, 64 cached tokens in 16-token pages, 16 greedy steps
    "tiny_b1_ctx64": dict(model="TINY", batch=1, context=64, steps=16),
    # 30B-A3B, batch 1 at 8K context: the throughput workload
    "a3b_b1_ctx8k": dict(model="A3B", batch=1, context=8192, steps=128),
    # batch sweep at 8K with a shuffled page table
    "a3b_b4_ctx8k": dict(model="A3B", batch=4, context=8192, steps=128),
    "a3b_b16_ctx8k": dict(model="A3B", batch=16, context=8192, steps=128),
    "a3b_b64_ctx8k": dict(model="A3B", batch=64, context=8192, steps=128),
    # long context, batch 1
    "a3b_b1_ctx32k": dict(model="A3B", batch=1, context=32768, steps=32),
    "a3b_b1_ctx128k": dict(model="A3B", batch=1, context=131072, steps=32),
    "a3b_b1_ctx256k": dict(model="A3B", batch=1, context=262144, steps=32),
}


def dims_of(name: str) -> dict:
    return {"TINY": TINY, "A3B": A3B, "MICRO": MICRO}[name].copy()
