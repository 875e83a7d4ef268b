"""Closed-form algorithmic bytes of one decode step, and speed-of-light rates.

The pages price a decode step as the bytes it must move divided by HBM
bandwidth: about 6.6 GB of BF16 weights plus about 0.5 GB of KV cache at 8K
context, against 3.35 TB/s, for a ceiling near 470 tok/s ("Inside the
Megakernel Serving Engine for North Mini Code", paragraph 2; "Cohere fuses an
entire decode step into one GPU program", paragraph 3). Here the same model
is written out for this build's shapes: only the bytes the step has to touch
count (routed experts only, looked-up embedding rows only).
"""

from __future__ import annotations

from typing import Iterable, Sequence

MI355X_HBM_BYTES_PER_S = 8.0e12


def step_bytes(dims: dict, contexts: Sequence[int], distinct_experts: Sequence[int],
               distinct_tokens: int | None = None, router_bias: bool = False) -> int:
    """Bytes one decode step must read or write.

    contexts[b] is the number of tokens sequence b has cached before the step
    (its new token goes to that position); distinct_experts[l] is the number of
    different experts layer l routes to over the batch; distinct_tokens is the
    number of different input tokens (embedding rows), default the batch size.
    """
    L, H, V = dims["n_layers"], dims["hidden"], dims["vocab"]
    hq, hkv, D = dims["n_q_heads"], dims["n_kv_heads"], dims["head_dim"]
    E, I = dims["n_experts"], dims["moe_inter"]
    B = len(contexts)
    if distinct_tokens is None:
        distinct_tokens = B
    if len(distinct_experts) != L:
        raise ValueError("one distinct-expert count per layer")
    dense = L * 2 * (H * (hq + 2 * hkv) * D + hq * D * H + E * H + 2 * H)
    if router_bias:
        dense += L * 4 * E
    experts = 2 * 3 * H * I * int(sum(distinct_experts))
    head = 2 * V * H + 2 * H + 2 * H * int(distinct_tokens)
    kv_token = L * 2 * hkv * D * 2
    kv_read = sum((int(t) + 1) * kv_token for t in contexts)
    kv_write = B * kv_token
    logits = B * V * 4
    return int(dense + experts + head + kv_read + kv_write + logits)


def forward_step_bytes(dims: dict, runs: Sequence[tuple], distinct_experts: Sequence[int],
                       distinct_tokens: int | None = None, router_bias: bool = False) -> int:
    """Bytes a multi-token step must move. runs[i] = (first position, rows)
    of one sequence: the run reads that sequence's cache once (the cached
    prefix and its own new entries, positions 0 .. first + rows - 1), writes
    one KV slot and one logits row per row. Dense weights, routed experts and
    the LM head count once, as in step_bytes."""
    L, V = dims["n_layers"], dims["vocab"]
    kv_token = L * 2 * dims["n_kv_heads"] * dims["head_dim"] * 2
    rows = sum(int(n) for _, n in runs)
    if distinct_tokens is None:
        distinct_tokens = rows
    base = step_bytes(dims, [], distinct_experts, distinct_tokens, router_bias)
    kv_read = sum((int(p0) + int(n)) * kv_token for p0, n in runs)
    return int(base + kv_read + rows * kv_token + rows * V * 4)


def weight_bytes(dims: dict, distinct_experts: Sequence[int]) -> int:
    """The weight part of step_bytes (dense, routed experts, LM head)."""
    return step_bytes(dims, [], distinct_experts, 0) - 0


def sol_tokens_per_s(bytes_per_step: float, batch: int, bandwidth: float = MI355X_HBM_BYTES_PER_S) -> float:
    """Speed-of-light decode rate: batch tokens per (bytes / bandwidth)."""
    return batch * bandwidth / float(bytes_per_step)
