"""Oracle expert math and layer pins: SwiGLU vs torch, the full MoE layer vs a
torch-built one, paged == unpaged bitwise, bf16 rounding vs torch."""
import numpy as np
import torch
import torch.nn.functional as F

import workloads as W
from oracle import formats
from oracle.expert import silu, swiglu_expert
from oracle.layer import PagedLayer, bf16_rne, run_stack
from workloads import gen


def test_silu_and_swiglu_vs_torch():
    rng = np.random.default_rng(0)
    H, I = 48, 20                                     # non-square: catches transposes
    wg, wu = rng.standard_normal((I, H)), rng.standard_normal((I, H))
    wd = rng.standard_normal((H, I))
    x = rng.standard_normal((5, H))
    a = rng.standard_normal(1000) * 10
    assert np.allclose(silu(a), F.silu(torch.from_numpy(a)).numpy(), rtol=1e-14, atol=1e-300)
    t = lambda v: torch.from_numpy(v)
    ref = F.linear(F.silu(F.linear(t(x), t(wg))) * F.linear(t(x), t(wu)), t(wd)).numpy()
    assert np.allclose(swiglu_expert(wg, wu, wd, x), ref, rtol=1e-12, atol=1e-14)


def _torch_moe(store, fmt, k, H, I, logits, x):
    """Plain MoE layer in torch float64 on tie-free logits (torch.topk order)."""
    lg = torch.from_numpy(logits.astype(np.float64))
    p = torch.softmax(lg, dim=-1)
    w, ids = torch.topk(p, k, dim=-1)
    w = w / w.sum(-1, keepdim=True)
    out = torch.zeros(x.shape[0], H, dtype=torch.float64)
    xt = torch.from_numpy(np.asarray(x, np.float64))
    for b in range(x.shape[0]):
        for j in range(k):
            g, u, d = (torch.from_numpy(a) for a in formats.decode_record(store[int(ids[b, j])], fmt, H, I))
            out[b] += w[b, j] * F.linear(F.silu(F.linear(xt[b], g)) * F.linear(xt[b], u), d)
    return out.numpy()


def test_layer_vs_torch_moe_tiny():
    cfg = W.CONFIGS[1]
    store = gen.expert_store(cfg)
    logits, x = gen.decode_inputs(cfg, 1)
    lay = PagedLayer(store, cfg.fmt, cfg.E, cfg.top_k, cfg.H, cfg.I, cfg.K)
    for t in range(cfg.steps):
        out, ids, w, plan = lay.step(logits[t], x[t])
        ref = _torch_moe(store, cfg.fmt, cfg.top_k, cfg.H, cfg.I, logits[t], x[t])
        assert np.allclose(out, ref, rtol=1e-12, atol=1e-15)


def _multiwave_layer(fmt=formats.BF16, K=3):
    E, k, H, I = 12, 4, 128, 128
    rng = np.random.default_rng(5)
    store = np.stack([gen.encode_record(fmt, (rng.standard_normal((2 * I, H)) * 0.05).astype(np.float32),
                                        (rng.standard_normal((H, I)) * 0.05).astype(np.float32))
                      for _ in range(E)])
    return PagedLayer(store, fmt, E, k, H, I, K), rng


def test_paged_equals_unpaged_bitwise_multiwave():
    for fmt in (formats.F32, formats.BF16, formats.FP8, formats.INT4):
        lay, rng = _multiwave_layer(fmt)
        for _ in range(12):
            B = int(rng.integers(1, 4))
            logits = rng.standard_normal((B, lay.E)).astype(np.float32)
            x = gen.bf16_bits_to_f32(gen.f32_to_bf16_bits(rng.standard_normal((B, lay.H)).astype(np.float32)))
            ref = lay.unpaged_forward(logits, x)
            out, ids, w, plan = lay.step(logits, x)
            assert plan.n_waves >= 1
            assert np.array_equal(out, ref)


def test_stale_slot_would_be_caught():
    """A paged-in expert computed from another expert's bytes changes the output
    ([PE] 'Can paging change the model's outputs?'): the oracle computes from
    its slots, so a wrong copy is visible."""
    lay, rng = _multiwave_layer(formats.BF16, K=4)
    logits = rng.standard_normal((1, lay.E)).astype(np.float32)
    x = rng.standard_normal((1, lay.H))
    ref = lay.unpaged_forward(logits, x)
    orig = lay._page_in
    lay._page_in = lambda e, s: orig((e + 1) % lay.E, s)        # planted mistake
    out, *_ = lay.step(logits, x)
    assert not np.allclose(out, ref)


def test_bf16_rne_vs_torch():
    rng = np.random.default_rng(1)
    v = (rng.standard_normal(100000) * np.exp2(rng.integers(-20, 20, 100000))).astype(np.float32)
    # exact ties: a bf16 value plus half an ulp, both parities
    base = gen.bf16_bits_to_f32(gen.f32_to_bf16_bits(rng.standard_normal(1000).astype(np.float32)))
    ulp = np.exp2(np.floor(np.log2(np.abs(base))) - 7)
    ties = (base + ulp / 2).astype(np.float32)
    v = np.concatenate([v, ties, -ties]).astype(np.float64)
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(bf16_rne(v), ref)


def test_stack_residual():
    cfg = W.CONFIGS[1]
    store = gen.expert_store(cfg)
    layers = [PagedLayer(store, cfg.fmt, cfg.E, cfg.top_k, cfg.H, cfg.I, cfg.K) for _ in range(3)]
    rng = np.random.default_rng(2)
    logits = [rng.standard_normal((1, cfg.E)).astype(np.float32) for _ in range(3)]
    x0 = bf16_rne(rng.standard_normal((1, cfg.H)))
    xf, outs, plans = run_stack(layers, logits, x0)
    x = x0
    for o in outs:
        x = bf16_rne(x + o)
    assert np.array_equal(x, xf)
    assert len(plans) == 3
