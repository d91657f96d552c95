"""GPU parity of the decode path (route -> slot plan -> page-in -> GEMV FFN)
against the oracle, through the C ABI, on the seeded workloads."""
import numpy as np
import pytest

import workloads as W
from workloads import gen

from gpu_harness import PairedLayer, say

pytestmark = pytest.mark.gpu


def _layer(cfg, B, K=None, **kw):
    K = cfg.K if K is None else K
    return PairedLayer(cfg.E, cfg.top_k, cfg.H, cfg.I, K, cfg.fmt,
                       lambda a: gen.expert_store(cfg, out=a), max_tokens=B, **kw)


def test_tiny_f32_all_steps():
    cfg = W.CONFIGS[1]
    say("case: tiny f32 E=8 k=2 H=64 I=32 K=4, 16 steps")
    p = _layer(cfg, 1)
    logits, x = gen.decode_inputs(cfg, 1)
    worst = p.run(logits, x, check_state_every=1)
    say("tiny f32 worst rel err", worst)
    st = p.gpu.stats()
    assert st["steps"] == 16 and st["hits"] + st["misses"] == st["refs"]
    p.close()


def test_bf16_layer_256_steps():
    cfg = W.CONFIGS[2]
    say("case: bf16 layer E=128 k=8 H=2048 I=768 K=40, 256 steps at batch 1")
    p = _layer(cfg, 1)
    logits, x = gen.decode_inputs(cfg, 1)
    worst = p.run(logits, x, sample=lambda t: t % 16 == 0 or t == cfg.steps - 1)
    st = p.gpu.stats()
    say("bf16 worst rel err", worst, "stats", st)
    assert st["steps"] == 256 and st["misses"] + st["hits"] == st["refs"]
    p.close()


@pytest.mark.parametrize("B", [3, 8])
def test_bf16_layer_batches(B):
    """Several tokens per expert (the bf16 up kernel shares each pair's
    activation row through LDS, pair after pair); B=8 gives multi-wave steps."""
    cfg = W.CONFIGS[2]
    say("case: bf16 layer K=40, 24 steps at batch %d" % B)
    p = _layer(cfg, B)
    logits, x = gen.decode_inputs(cfg, B, steps=24)
    worst = p.run(logits, x, sample=lambda t: t % 4 == 3)
    say("bf16 B=%d worst rel err" % B, worst)
    p.close()


@pytest.mark.parametrize("B", [1, 2, 4, 5, 6, 8])
def test_fp8_layer_batches(B):
    cfg = W.CONFIGS[3]
    say("case: fp8 layer K=40 B=%d, 48 steps" % B)
    p = _layer(cfg, B)
    logits, x = gen.decode_inputs(cfg, B, steps=48)
    worst = p.run(logits, x, sample=lambda t: t % 8 == 0 or t == 47)
    st = p.gpu.stats()
    say("fp8 B=%d worst rel err %.3g waves %d steps %d" % (B, worst, st["waves"], st["steps"]))
    if B <= cfg.K // cfg.top_k:
        assert st["waves"] == st["steps"]        # batch cap: always one wave
    p.close()


def test_int4_layer():
    cfg = W.CONFIGS[4]
    say("case: int4 layer E=128 K=92, 64 steps at batch 1")
    p = _layer(cfg, 1)
    logits, x = gen.decode_inputs(cfg, 1, steps=64)
    worst = p.run(logits, x, sample=lambda t: t % 8 == 0 or t == 63)
    say("int4 worst rel err", worst)
    p.close()


@pytest.mark.parametrize("B", [1, 4])
def test_mxfp4_layer(B):
    cfg = W.CONFIGS[6]
    steps = 64 if B == 1 else 24
    say("case: mxfp4 layer E=128 k=8 H=2048 I=768 K=40, B=%d, %d steps" % (B, steps))
    p = _layer(cfg, B)
    logits, x = gen.decode_inputs(cfg, B, steps=steps)
    worst = p.run(logits, x, sample=lambda t: t % 8 == 0 or t == steps - 1)
    st = p.gpu.stats()
    say("mxfp4 B=%d worst rel err %.3g stats %s" % (B, worst, st))
    assert st["steps"] == steps and st["misses"] + st["hits"] == st["refs"]
    p.close()


def test_mxfp4_small_ragged_shape():
    """H and I multiples of the 32-value scale block but not of 64 or 128:
    a partial wavefront of chunks in the up projection and a short down row."""
    E, k, H, I, K, B = 8, 2, 96, 160, 4, 3
    say("case: mxfp4 E=8 k=2 H=96 I=160 K=4 B=3, 12 steps")
    rng = np.random.default_rng(11)
    recs = [gen.encode_record(gen.MXFP4, (rng.standard_normal((2 * I, H)) * 0.1).astype(np.float32),
                              (rng.standard_normal((H, I)) * 0.1).astype(np.float32)) for _ in range(E)]

    def fill(a):
        for e in range(E):
            a[e] = recs[e]
    p = PairedLayer(E, k, H, I, K, gen.MXFP4, fill, max_tokens=B)
    logits = rng.standard_normal((12, B, E)).astype(np.float32)
    x = gen.f32_to_bf16_bits(rng.standard_normal((12, B, H)).astype(np.float32))
    worst = p.run(logits, x, check_state_every=1)
    say("mxfp4 small worst rel err %.3g" % worst)
    p.close()


@pytest.mark.parametrize("fmt", [gen.INT4, gen.FP8, gen.MXFP4, gen.BF16])
def test_activation_range_extremes(fmt):
    """Activations over the whole bf16 range the layers accept: magnitudes
    near 7e4 (beyond fp16's largest finite value) mixed with values near 1e-6
    (below fp16's normal range) and ordinary ones, at batch 1 and 3, against
    the oracle. The expert kernels keep activations in bf16 or fp32, so
    nothing is clamped or flushed."""
    E, k, H, I, K = 16, 2, 256, 256, 8
    say("case: fmt %d activations near 7e4 and 1e-6" % fmt)
    rng = np.random.default_rng(90 + fmt)
    recs = [gen.encode_record(fmt, (rng.standard_normal((2 * I, H)) * 0.02).astype(np.float32),
                              (rng.standard_normal((H, I)) * 0.02).astype(np.float32)) for _ in range(E)]

    def fill(a):
        for e in range(E):
            a[e] = recs[e]
    for B in (1, 3):
        p = PairedLayer(E, k, H, I, K, fmt, fill, max_tokens=B)
        steps = 6
        logits = rng.standard_normal((steps, B, E)).astype(np.float32)
        v = rng.standard_normal((steps, B, H))
        pick = rng.integers(0, 3, (steps, B, H))
        v = np.where(pick == 0, np.sign(v) * rng.uniform(6e4, 7.5e4, v.shape),
                     np.where(pick == 1, v * 1e-6, v))
        x = gen.f32_to_bf16_bits(v.astype(np.float32))
        worst = p.run(logits, x, check_state_every=1)
        say("fmt %d B=%d worst rel err %.3g" % (fmt, B, worst))
        p.close()
