"""Seeded synthetic inputs for the Paged Experts hot path.

This module is the only code shared by the HIP path's tests/bench and the
oracle. It draws numbers and packs them into the agreed byte layouts; it holds
none of the method's arithmetic (no routing, no slot planning, no expert
math, no decoding).

Workloads (the shapes of Qwen3-30B-A3B as given in [PE] "What does Paged
Experts actually do?": 128 experts, 8 per token, hidden 2048, MoE
intermediate 768, 48 layers):

  1 tiny     f32,  E=8 k=2 H=64 I=32, K=4, 16 decode steps at batch 1, cold
  2 bf16     one layer, E=128 k=8 H=2048 I=768, K=40, 256 steps at batch 1, cold,
             correlated routing p=0.75
  3 fp8      as 2, block-FP8 e4m3 with 128x128 fp32 scales, batch 1,2,4,5,6,8
  4 int4     48 layers, int4 asym g128, K=92, 256 tokens at batch 1, correlated
             routing p=0.75, plus a uniform-routing control
  5 prefill  one 2048-token chunk through 48 bf16 layers, K=92, warm table
             (experts 0..91 resident), uniform routing

Routing processes ([PE] "Why is it fast when experts keep crossing PCIe?"
infers that consecutive tokens reuse experts; [LRU] "The observation" names
the same locality):
  correlated: each of the previous step's k experts is kept independently
              with probability p; the set is refilled to k by drawing without
              replacement, uniformly, from the experts not kept; step 0 is a
              uniform k of E. One chain per sequence (batch row) and per layer.
  uniform:    a fresh uniform k of E per token, layer and step.
  The target set S becomes router logits z + 16 * [e in S] with z ~ N(0,1),
  so the router still selects S (checked when drawn).

Weights ~ N(0, sigma) are drawn by inverse-CDF lookup of 16-bit uniform
integers (a 65536-entry quantile table of the normal distribution), which is
fast enough for stores of 10^9 weights. A 48-layer store is built from one
layer's worth of E independently drawn records: layer l's expert e is record
perm_l[e] of that pool, with perm_l a seeded permutation per layer. Within a
layer every expert is distinct, which is what the slot table can confuse.
"""
from .gen import (CONFIGS, Config, streams, normal_table_f32, draw_normal_f32,
                  f32_to_bf16_bits, bf16_bits_to_f32, encode_record, record_stride,
                  expert_store, layer_permutation, correlated_sets, uniform_sets,
                  logits_from_sets, normal_logits, hidden_states)

__all__ = ["CONFIGS", "Config", "streams", "normal_table_f32", "draw_normal_f32",
           "f32_to_bf16_bits", "bf16_bits_to_f32", "encode_record", "record_stride",
           "expert_store", "layer_permutation", "correlated_sets", "uniform_sets",
           "logits_from_sets", "normal_logits", "hidden_states"]
