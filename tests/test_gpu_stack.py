"""GPU parity of the native stack driver (moe_stack_forward): per-layer slot
plans and table state exact, per-layer MoE outputs within tolerance, final
hidden state within the bf16 bound, in strict order and with lookahead."""
import numpy as np
import pytest
import torch

import expert_weight_paging_amd as ewp
import workloads as W
from oracle.layer import PagedLayer, bf16_rne
from workloads import gen

from gpu_harness import TOL, rel_err, say, x_values

pytestmark = pytest.mark.gpu


def _stack(cfg, n_layers, max_tokens, initial_fill, streams):
    rec = ewp.record_bytes(cfg.fmt, cfg.H, cfg.I)
    pool = gen.pool_records(cfg)
    hosts, layers, plans, refs = [], [], [], []
    for l in range(n_layers):
        h = ewp.HostStore(cfg.E, rec)
        gen.fill_layer_store(cfg, l, h.array, pool)
        slots, state = ewp.alloc_layer_buffers(cfg.E, cfg.K, rec, "cuda")
        L = ewp.Layer(cfg.E, cfg.top_k, cfg.H, cfg.I, cfg.K, cfg.fmt, h, slots, state, *streams,
                      initial_fill=initial_fill)
        hosts.append(h)
        layers.append(L)
        plans.append(ewp.Plan(L, max_tokens))
        refs.append(PagedLayer(h.array, cfg.fmt, cfg.E, cfg.top_k, cfg.H, cfg.I, cfg.K,
                               initial_fill=initial_fill))
    return hosts, layers, plans, refs


def _check_layer(plan, layer, ref, ids_ref, p_ref):
    info = plan.info()
    assert info["num_waves"] == p_ref.n_waves
    for w, wv in enumerate(p_ref.waves):
        ex, sl, misses = plan.wave(w)
        assert (ex, sl, misses) == (wv.experts, wv.slots, wv.misses)
    ids, _, sid, _ = plan.read()
    assert np.array_equal(ids, ids_ref) and np.array_equal(sid, p_ref.slot_ids)
    se, es, st, clk = layer.get_state()
    rse, res, rst, rclk = ref.table.state()
    assert np.array_equal(se, rse) and np.array_equal(st, rst) and clk == rclk


def _run(cfg, n_layers, T, steps, lookahead, initial_fill, tokens_salt=0):
    s = (torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream())
    hosts, layers, plans, refs = _stack(cfg, n_layers, T, initial_fill, s)
    rng = np.random.default_rng(11 + tokens_salt)
    E = cfg.E
    worst_out, worst_hidden = 0.0, 0.0
    for step in range(steps):
        sets = np.stack([np.stack([np.sort(rng.choice(E, cfg.top_k, replace=False)) for _ in range(T)])
                         for _ in range(n_layers)])
        logits = gen.logits_from_sets(rng, sets, E)                     # [L][T][E]
        x0 = gen.f32_to_bf16_bits(rng.standard_normal((T, cfg.H)).astype(np.float32))
        x = torch.from_numpy(x0.view(np.int16)).cuda()
        out = torch.empty(T, cfg.H, dtype=torch.float32, device="cuda")
        ewp.stack_forward(layers, plans, torch.from_numpy(logits).cuda(), x, out, lookahead=lookahead)
        torch.cuda.synchronize()
        # oracle, layer by layer; the last layer's MoE output is what `out` holds
        xv = x_values(x0, cfg.fmt)
        for l in range(n_layers):
            o, ids_ref, w_ref, p_ref = refs[l].step(logits[l], xv)
            _check_layer(plans[l], layers[l], refs[l], ids_ref, p_ref)
            xv_next = bf16_rne(xv + o)
            if l == n_layers - 1:
                e = rel_err(out.cpu().numpy(), o)
                worst_out = max(worst_out, e)
                assert e <= TOL[cfg.fmt], (step, e)
            xv = xv_next
        got = gen.bf16_bits_to_f32(x.cpu().numpy().view(np.uint16)).astype(np.float64)
        d = np.abs(got - xv)
        bound = TOL[cfg.fmt] * np.sqrt(np.mean(o ** 2)) + n_layers * np.exp2(
            np.floor(np.log2(np.maximum(np.abs(xv), 2.0 ** -126))) - 7)
        worst_hidden = max(worst_hidden, float((d / bound).max()))
        assert np.all(d <= bound)
    for p in plans:
        p.close()
    for L in layers:
        L.close()
    for h in hosts:
        h.free()
    return worst_out, worst_hidden


@pytest.mark.parametrize("lookahead", [False, True])
def test_int4_decode_stack(lookahead):
    cfg = W.CONFIGS[4]
    say("case: int4 stack 4 layers x 12 tokens at batch 1, lookahead=%s" % lookahead)
    wo, wh = _run(cfg, 4, 1, 12, lookahead, False)
    say("worst last-layer output err %.3g, hidden/bound %.3g" % (wo, wh))


@pytest.mark.parametrize("lookahead", [False, True])
def test_bf16_prefill_stack(lookahead):
    cfg = W.CONFIGS[5]
    say("case: bf16 prefill stack 2 layers x 256 tokens, warm, lookahead=%s" % lookahead)
    wo, wh = _run(cfg, 2, 256, 2, lookahead, True, tokens_salt=1)
    say("worst last-layer output err %.3g, hidden/bound %.3g" % (wo, wh))
