"""Oracle expert math and layer pins: SwiGLU vs torch, the full MoE layer vs a
torch-built one, paged == unpaged bitwise, bf16 rounding vs torch."""
import numpy as np
import torch
import torch.nn.functional as F

import workloads as W
from oracle import formats
from oracle.expert import silu, swiglu_expert
from oracle.layer import RMS_EPS, PagedLayer, bf16_rne, rms_norm, run_stack
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


def _torch_bf16(v):
    """float64 -> bfloat16 -> float64 through torch's own conversion."""
    return torch.from_numpy(np.asarray(v, np.float64)).to(torch.bfloat16).to(torch.float64).numpy()


def _torch_norm(v):
    """Unit-gain RMSNorm through torch's own routine, float64."""
    t = torch.from_numpy(np.asarray(v, np.float64))
    return F.rms_norm(t, (t.shape[-1],), eps=RMS_EPS).numpy()


def test_rms_norm_vs_torch_and_closed_forms():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((7, 96)) * np.exp2(rng.integers(-8, 8, (7, 1)))
    assert np.allclose(rms_norm(x), _torch_norm(x), rtol=1e-14, atol=0)
    c = 3.0                                            # a constant row c: c / sqrt(c^2 + eps)
    assert np.allclose(rms_norm(np.full((1, 64), c)), c / np.sqrt(c * c + RMS_EPS), rtol=1e-15)
    big = x * 1e3                                      # norm(c x, c^2 eps) = norm(x, eps)
    assert np.allclose(rms_norm(big, eps=1e6 * RMS_EPS), rms_norm(x), rtol=1e-13)
    assert np.allclose(np.mean(rms_norm(x, eps=0.0) ** 2, axis=-1), 1.0, rtol=1e-13)
    assert np.array_equal(rms_norm(np.zeros((1, 8))), np.zeros((1, 8)))


def _tiny_stack_layers(cfg, n):
    """n layers of the tiny workload whose stores differ (layer l: pool record
    perm_l[e] for expert e), each with a cold table."""
    stores = [gen.expert_store(cfg)[np.random.default_rng(70 + l).permutation(cfg.E)] for l in range(n)]
    return stores, [PagedLayer(s, cfg.fmt, cfg.E, cfg.top_k, cfg.H, cfg.I, cfg.K) for s in stores]


def test_stack_against_independent_chain():
    """run_stack pinned against a chain built without it: torch's RMSNorm and
    bfloat16 rounding of the layer input, fresh layers' unpaged_forward
    (itself pinned to a torch-built MoE above), torch's bfloat16 rounding of
    x + out, layer by layer and over two tokens (the second through warm
    tables). Bitwise: both sum each layer in the same wave/expert order. A
    stack that fed x0 to every layer, skipped the residual or the norm, or
    reused one layer's output is shown to give a different answer, so the
    comparison can fail for those mistakes."""
    cfg = W.CONFIGS[1]
    n = 3
    _, layers = _tiny_stack_layers(cfg, n)
    stores, chain = _tiny_stack_layers(cfg, n)
    assert not all(np.array_equal(stores[0], s) for s in stores[1:])
    rng = np.random.default_rng(2)
    for tok in range(2):
        logits = [rng.standard_normal((1, cfg.E)).astype(np.float32) for _ in range(n)]
        x0 = _torch_bf16(rng.standard_normal((1, cfg.H)))
        xf, outs, plans = run_stack(layers, logits, x0)
        assert len(outs) == n and len(plans) == n
        # independent chain: unpaged math of each layer, then advance the
        # chain layer's table exactly as a step does (its output is not used)
        x, ref_outs = x0, []
        for l in range(n):
            a = _torch_bf16(_torch_norm(x))
            o = chain[l].unpaged_forward(logits[l], a)
            _, _, _, p = chain[l].step(logits[l], a, compute=False)
            assert p.n_waves == plans[l].n_waves and p.waves[0].misses == plans[l].waves[0].misses
            ref_outs.append(o)
            x = _torch_bf16(x + o)
        for l in range(n):
            assert np.array_equal(outs[l], ref_outs[l]), (tok, l)
        assert np.array_equal(xf, x), tok
        # also against the torch-built MoE on the same hidden states (tie-free logits)
        xl = x0
        for l in range(n):
            t = _torch_moe(stores[l], cfg.fmt, cfg.top_k, cfg.H, cfg.I, logits[l], _torch_bf16(_torch_norm(xl)))
            assert np.allclose(outs[l], t, rtol=1e-12, atol=1e-15)
            xl = _torch_bf16(xl + t)
        # negative controls: plausible composition mistakes change the result
        fresh = _tiny_stack_layers(cfg, n)[1]
        a0 = _torch_bf16(_torch_norm(x0))
        wrong_x0 = _torch_bf16(x0 + sum(fresh[l].unpaged_forward(logits[l], a0) for l in range(n)))
        assert not np.array_equal(wrong_x0, xf)
        no_residual = x0
        for l in range(n):
            no_residual = _torch_bf16(fresh[l].unpaged_forward(logits[l], _torch_bf16(_torch_norm(no_residual))))
        assert not np.array_equal(no_residual, xf)
        no_norm = x0
        for l in range(n):
            no_norm = _torch_bf16(no_norm + fresh[l].unpaged_forward(logits[l], no_norm))
        assert not np.array_equal(no_norm, xf)
        assert not np.array_equal(_torch_bf16(x0 + outs[-1]), xf)


def test_float32_variant_matches_float64():
    """The float32 oracle (timed as the CPU baseline) takes the same steps:
    identical ids and plans, outputs within the float32 tolerance of the
    float64 oracle, on every format and multi-wave steps."""
    for fmt in (formats.F32, formats.BF16, formats.FP8, formats.INT4, formats.MXFP4):
        lay64, rng = _multiwave_layer(fmt)
        lay32 = PagedLayer(lay64.store, fmt, lay64.E, lay64.top_k, lay64.H, lay64.I, lay64.K,
                           dtype=np.float32)
        for _ in range(8):
            B = int(rng.integers(1, 4))
            logits = rng.standard_normal((B, lay64.E)).astype(np.float32)
            x = gen.bf16_bits_to_f32(gen.f32_to_bf16_bits(rng.standard_normal((B, lay64.H)).astype(np.float32)))
            o64, i64, w64, p64 = lay64.step(logits, x)
            o32, i32, w32, p32 = lay32.step(logits, x)
            assert o32.dtype == np.float32
            assert np.array_equal(i64, i32) and np.array_equal(p64.slot_ids, p32.slot_ids)
            assert [w.misses for w in p64.waves] == [w.misses for w in p32.waves]
            rms = np.sqrt(np.mean(o64 ** 2))
            assert np.abs(o32 - o64).max() <= 1e-5 * rms, fmt


def test_shared_decode_cache_changes_nothing():
    """Layers sharing a decode memo (records keyed by a hash of their bytes)
    give bitwise the outputs of layers that decode every slot themselves, and
    a planted copy of the wrong record is still visible through the memo."""
    cfg = W.CONFIGS[1]
    stores, plain = _tiny_stack_layers(cfg, 3)
    memo = {}
    cached = [PagedLayer(s, cfg.fmt, cfg.E, cfg.top_k, cfg.H, cfg.I, cfg.K, decode_cache=memo)
              for s in stores]
    rng = np.random.default_rng(9)
    for _ in range(6):
        logits = [rng.standard_normal((2, cfg.E)).astype(np.float32) for _ in range(3)]
        x0 = bf16_rne(rng.standard_normal((2, cfg.H)))
        a = run_stack(plain, logits, x0)
        b = run_stack(cached, logits, x0)
        assert np.array_equal(a[0], b[0]) and all(np.array_equal(u, v) for u, v in zip(a[1], b[1]))
    assert 0 < len(memo) <= cfg.E                  # the three layers hold permutations of one pool
    lay = PagedLayer(stores[0], cfg.fmt, cfg.E, cfg.top_k, cfg.H, cfg.I, cfg.K, decode_cache=memo)
    logits = rng.standard_normal((1, cfg.E)).astype(np.float32)
    x = rng.standard_normal((1, cfg.H))
    ref = lay.unpaged_forward(logits, x)
    orig = lay._page_in
    lay._page_in = lambda e, s: orig((e + 1) % lay.E, s)        # planted mistake
    out, *_ = lay.step(logits, x)
    assert not np.allclose(out, ref)
