"""GPU parity of the native stack driver (moe_stack_forward), strict order and
with lookahead: a stack run by the driver must give bitwise the hidden state,
output, plans and table state of a twin stack run layer by layer, where every
layer is checked against the oracle (tests/stack_check.py: plans and state
exact, each layer's output within tolerance on its own input, residual exact
up to rare flips, hidden state within the accumulated bound of an independent
oracle chain)."""
import numpy as np
import pytest
import torch

import expert_weight_paging_amd as ewp
import workloads as W
from workloads import gen

from gpu_harness import say
from stack_check import StackPair

pytestmark = pytest.mark.gpu


def _run(cfg, n_layers, T, steps, lookahead, initial_fill, tokens_salt=0):
    streams = lambda: (torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream())
    A = StackPair(cfg, n_layers, T, initial_fill, streams(), keep_refs=False)   # the driver
    B = StackPair(cfg, n_layers, T, initial_fill, streams())                    # layer by layer
    rng = np.random.default_rng(11 + tokens_salt)
    E = cfg.E
    worst = {}
    for step in range(steps):
        sets = np.stack([np.stack([np.sort(rng.choice(E, cfg.top_k, replace=False)) for _ in range(T)])
                         for _ in range(n_layers)])
        logits = gen.logits_from_sets(rng, sets, E)                     # [L][T][E]
        x0 = gen.f32_to_bf16_bits(rng.standard_normal((T, cfg.H)).astype(np.float32))
        x = torch.from_numpy(x0.view(np.int16)).cuda()
        out = torch.empty(T, cfg.H, dtype=torch.float32, device="cuda")
        ewp.stack_forward(A.layers, A.plans, torch.from_numpy(logits).cuda(), x, out, lookahead=lookahead)
        torch.cuda.synchronize()
        xb, ob, summ = B.run_token(logits, x0, "host", chain=slice(None))
        assert torch.equal(x, xb) and torch.equal(out, ob), step
        for l in range(n_layers):
            for u, v in zip(A.plans[l].read(), B.plans[l].read()):
                assert np.array_equal(u, v), (step, l)
            for u, v in zip(A.layers[l].get_state(), B.layers[l].get_state()):
                assert np.array_equal(np.asarray(u), np.asarray(v)), (step, l)
        for k, v in summ.items():
            worst[k] = max(worst.get(k, 0.0), v)
    A.close()
    B.close()
    return worst


@pytest.mark.parametrize("lookahead", [False, True])
def test_int4_decode_stack(lookahead):
    cfg = W.CONFIGS[4]
    say("case: int4 stack 4 layers x 12 tokens at batch 1, lookahead=%s" % lookahead)
    say("worst: %s" % _run(cfg, 4, 1, 12, lookahead, False))


@pytest.mark.parametrize("lookahead", [False, True])
def test_bf16_prefill_stack(lookahead):
    cfg = W.CONFIGS[5]
    say("case: bf16 prefill stack 2 layers x 256 tokens, warm, lookahead=%s" % lookahead)
    say("worst: %s" % _run(cfg, 2, 256, 2, lookahead, True, tokens_salt=1))
