"""Sizing arithmetic of the Paged Experts scheme.

[PE] "A preflight script before you turn it on" gives the formulas, and prints
their results for three setups (the worked example pinned in
tests/golden/preflight.json):
  slot cost (all layers)       = per-expert bytes x MoE layers
  batch cap (one wave)         = K // top_k
  bytes per token if all miss  = layers x top_k x per-expert bytes
  highest miss rate a measured = link bandwidth / (tok/s x all-miss bytes)
    speed allows
  miss rate without reuse      = 1 - K / E
  verdict                      = "reuse implied" when the highest allowed miss
                                 rate is below 0.8 x the no-reuse rate, else
                                 "inconclusive"
[PE] "What does a resident slot cost in context length?": a slot costs the
per-expert bytes times the layers, against a bf16 KV cache of
2 x layers x kv_heads x head_dim x 2 bytes per token.
[PE] "Why do short prompts get slower first tokens?": a prefill pages in every
expert that is not resident, once: (E - K) x slot cost.
[PE] "FAQ": the pinned host store holds every expert of every layer.
"""


def slots_for_budget(record_bytes, experts, layers, budget_bytes):
    """Slots per layer that a device-memory budget holds, the same K in every
    layer. [LRU] "How to use it": the expert cache is given as one budget (in
    MiB); [PE] "What does a resident slot cost in context length?": a slot
    costs its record bytes in each MoE layer. So K is the largest count with
    K x layers x record bytes within the budget, and never more than E."""
    return min(experts, budget_bytes // (layers * record_bytes))


def kv_bytes_per_token(layers=48, kv_heads=4, head_dim=128, elem_bytes=2):
    return 2 * layers * kv_heads * head_dim * elem_bytes


def preflight(layers, experts, top_k, expert_mb, K, link_gbps, tok_s, kv_bytes):
    slot_mb = expert_mb * layers
    all_miss_gb = layers * top_k * expert_mb / 1e3
    max_miss = link_gbps / (tok_s * all_miss_gb)
    random_miss = 1.0 - K / experts
    return {
        "slot_mb": slot_mb,
        "kv_tokens_per_slot": slot_mb * 1e6 / kv_bytes,
        "batch_cap": K // top_k,
        "all_miss_gb_per_token": all_miss_gb,
        "max_miss": max_miss,
        "random_miss": random_miss,
        "verdict": "reuse implied" if max_miss < 0.8 * random_miss else "inconclusive",
    }


def prefill_page_in_gb(experts, K, slot_mb):
    """Bytes a prefill touching every expert pages in, in GB."""
    return (experts - K) * slot_mb / 1e3


def host_store_gb(experts, layers, expert_mb):
    return experts * layers * expert_mb / 1e3


def link_needed_gbps(all_miss_gb, tok_s):
    """Link bandwidth needed if every activation missed at a measured speed."""
    return all_miss_gb * tok_s


def uniform_miss_rate(E, K):
    """Expected miss rate per activation after warm-up when each step's experts
    are drawn independently of the past: a drawn expert is resident with
    probability K / E ([PE] "Why is it fast ...", the no-reuse column)."""
    return 1.0 - K / E
