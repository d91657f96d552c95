"""CPU oracle for the Paged Experts hot path.

THIS PACKAGE IS TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import or run it. The product
(``expert_weight_paging_amd``) never imports it, and this package imports
nothing from the product: the only code both sides share is the seeded input
generator in ``workloads`` (which holds none of the method's arithmetic).

Sources, cited by title and section:

  [PE]  "Running an MoE Model Larger Than Your VRAM: SGLang Paged Experts, the
        PCIe Math, and the 4-Request Cliff" (a post on the sgl-project feed page).
  [LRU] "Locality of reference helped 94GB Qwen3.8-Flash-Next runs at 68 tok/s
        on one RTX 5090" (a post on the same feed page).
  [SRV] "Mastering the LLM Inference Serving Engine SGLang".

What the method computes (and so what the oracle computes):

  * a router picks top_k of E experts per token ([PE] "What does Paged Experts
    actually do?");
  * each layer keeps K experts in a slot table, copies in only the routed
    experts that are not resident, and evicts the least recently used one
    ([PE] "TL;DR", "What does Paged Experts actually do?"; [LRU] "The fix");
  * a step whose distinct experts do not fit the table runs in several waves,
    each with its own page-in ([PE] "What happens with more than one request?");
  * the expert math (SwiGLU FFN and the weighted top-k combine) is the ordinary
    MoE layer; paging does not change its result ([PE] "Can paging change the
    model's outputs?").

All floating point is float64 (numpy) for parity; ``PagedLayer(dtype=float32)``
takes the same steps in single precision and is the variant timed as the
CPU baseline. Integer results (top-k ids, slot
assignments, miss lists, wave counts, table state) are unique under the tie
rules stated in ``router`` and ``lru``.

Pins (tests/test_oracle_*.py, all ``-m "not gpu"``):
  router  -- pairwise brute-force check of the top-k tie rule, torch.topk on
             tie-free input, closed-form softmax identities;
  lru     -- an independent move-to-front list model over every routing
             sequence on tiny E, the LRU eviction property, K=E => zero misses
             after warm-up, misses <= B*top_k, one wave iff distinct <= K,
             uniform-routing miss rate 1-K/E and the correlated-routing closed
             form;
  formats -- all 256 FP8 e4m3fn codes against torch.float8_e4m3fn, bf16 against
             torch.bfloat16, hand-packed int4 words; the sixteen E2M1 values and
             the E8M0 scale bytes of MXFP4 listed, a byte-by-byte MXFP4 record;
  expert  -- SwiGLU against torch.nn.functional.silu / F.linear in float64;
  layer   -- paged output == unpaged output bitwise;
  stack   -- bf16 round-to-nearest-even against torch.bfloat16 conversion;
             run_stack against an independent chain of unpaged layers and
             torch's bf16 rounding (bitwise, over warm tables), and against a
             torch-built MoE per layer; x0-fed, residual-free and
             last-output-only compositions shown to differ;
  float32 -- the single-precision variant against float64: same plans, outputs
             within the float32 tolerance on every format;
  sizing  -- the worked example the [PE] preflight section prints, reproduced;
             slots for a memory budget against a brute-force search.
No oracle function is "parity unpinned".
"""
