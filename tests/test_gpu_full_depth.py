"""Full-depth parity of the two 48-layer workloads, every layer checked
(tests/stack_check.py): plan and table state bit-exact, each layer's MoE
output within the format's tolerance of the oracle on that layer's GPU input,
the residual exact up to rare one-ulp flips, and the hidden state within the
accumulated bound of an independent oracle chain. The product paths the
benchmark times (a HIP graph of device-resolved steps per decode token, the
strict-order stack driver for the prefill chunk; for the decode stack also
the graph with lookahead) must then give bitwise the same hidden states as
the checked layer-by-layer runs.

[PE] "What does Paged Experts actually do?": 48 MoE layers of 128 experts,
8 per token."""
import numpy as np
import pytest
import torch

import expert_weight_paging_amd as ewp
import workloads as W
from workloads import gen

from gpu_harness import say
from stack_check import StackPair

pytestmark = pytest.mark.gpu


def _stats(layers):
    tot = {}
    for L in layers:
        for k, v in L.stats().items():
            tot[k] = tot.get(k, 0) + v
    return tot


@pytest.mark.timeout(900)
def test_int4_stack_48_layers_every_layer():
    cfg = W.CONFIGS[4]
    tokens = 8
    say("case: int4 stack, 48 layers, K=92, %d correlated tokens from cold tables, every layer" % tokens)
    compute, copy = torch.cuda.Stream(), torch.cuda.Stream()
    pair = StackPair(cfg, cfg.layers, 1, False, (compute, copy, compute))
    logits, x0 = gen.stack_inputs(cfg, steps=tokens)        # [t][48][1][E], [t][1][H]
    finals, lasts = [], []
    with torch.cuda.stream(compute):
        for t in range(tokens):
            x, out, summ = pair.run_token(logits[t], x0[t], "device", chain=slice(None))
            say("token %d: %s" % (t, {k: round(v, 5) for k, v in summ.items()}))
            finals.append(x.clone())
            lasts.append(out.clone())
    s1 = _stats(pair.layers)
    # the benchmark's path: one HIP graph of the 48 device-resolved layers per token
    pair.reset()
    lg_buf = torch.zeros(cfg.layers, 1, cfg.E, dtype=torch.float32, device="cuda")
    xg = torch.zeros(1, cfg.H, dtype=torch.int16, device="cuda")
    og = torch.zeros(1, cfg.H, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=compute):
        ewp.stack_forward_device(pair.layers, pair.plans, lg_buf, xg, og)
    torch.cuda.synchronize()
    lg_all = torch.from_numpy(logits).cuda()
    x0_all = torch.from_numpy(np.ascontiguousarray(x0).view(np.int16)).cuda()
    for t in range(tokens):
        with torch.cuda.stream(compute):
            lg_buf.copy_(lg_all[t])
            xg.copy_(x0_all[t])
            g.replay()
        torch.cuda.synchronize()
        assert torch.equal(xg, finals[t]) and torch.equal(og, lasts[t]), t
    s2 = _stats(pair.layers)
    assert {k: s2[k] - s1[k] for k in s1} == s1
    say("graph replays equal the checked layer-by-layer run; stats %s" % s1)
    del g
    # the same with lookahead (copies of layer l + 1 beside layer l's math,
    # routing two layers ahead): the same plans, so the same bits and counters
    pair.reset()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=compute):
        ewp.stack_forward_device(pair.layers, pair.plans, lg_buf, xg, og, lookahead=True)
    torch.cuda.synchronize()
    for t in range(tokens):
        with torch.cuda.stream(compute):
            lg_buf.copy_(lg_all[t])
            xg.copy_(x0_all[t])
            g.replay()
        torch.cuda.synchronize()
        assert torch.equal(xg, finals[t]) and torch.equal(og, lasts[t]), t
    s3 = _stats(pair.layers)
    assert {k: s3[k] - s2[k] for k in s1} == s1
    say("lookahead graph replays equal the checked run too")
    del g
    pair.close()


@pytest.mark.timeout(900)
def test_prefill_chunk_48_layers_every_layer():
    cfg = W.CONFIGS[5]
    say("case: bf16 prefill, one 2048-token chunk through 48 layers, K=92 warm, every layer")
    s = (torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream())
    pair = StackPair(cfg, cfg.layers, cfg.tokens, True, s, keep_refs=False)
    logits, x0 = gen.prefill_inputs(cfg)                      # [48][2048][E], [2048][H]
    # the benchmark's path first: the strict-order stack driver
    x = torch.from_numpy(np.ascontiguousarray(x0).view(np.int16)).cuda()
    out = torch.empty(cfg.tokens, cfg.H, dtype=torch.float32, device="cuda")
    ewp.stack_forward(pair.layers, pair.plans, torch.from_numpy(logits).cuda(), x, out, lookahead=False)
    torch.cuda.synchronize()
    xa, oa = x.clone(), out.clone()
    s1 = _stats(pair.layers)
    pair.reset()
    rows = np.arange(0, cfg.tokens, 32)                      # independent chain on 64 tokens
    xb, ob, summ = pair.run_token(logits, x0, "host", chain=rows)
    say("prefill chunk: %s" % {k: round(v, 5) for k, v in summ.items()})
    assert torch.equal(xa, xb) and torch.equal(oa, ob)
    s2 = _stats(pair.layers)
    assert {k: s2[k] - s1[k] for k in s1} == s1
    assert s1["misses"] == 48 * 36 and s1["waves"] == 48 * 2
    pair.close()
