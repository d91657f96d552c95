"""GPU parity of the decode route kernel across table shapes: one, two and four
experts per planning lane (E <= 64, <= 128, <= 256), odd E and odd K (the
padded pairwise reads), single-token steps (top-k ranks split over the
workgroup) and multi-token steps, single- and multi-wave steps, and logits
with many exact ties. Host-driven steps check the published plan, the wave
lists and the table state after every step; device-resolved steps check the
plan left on the device and the counters."""
import numpy as np
import pytest
import torch

from workloads import gen

from gpu_harness import TOL, PairedLayer, rel_err, say, x_values

pytestmark = pytest.mark.gpu

H, I = 64, 32


def _fill(E, seed):
    rng = np.random.default_rng(seed)
    recs = [gen.encode_record(gen.F32, (rng.standard_normal((2 * I, H)) * 0.05).astype(np.float32),
                              (rng.standard_normal((H, I)) * 0.05).astype(np.float32)) for _ in range(E)]

    def fill(a):
        for e in range(E):
            a[e] = recs[e]
    return fill


def _inputs(E, B, steps, seed):
    """Logits N(0,1) with a third of them rounded to multiples of 0.5 (many
    exact ties, incl. +0 and -0), x N(0,1)."""
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((steps, B, E)).astype(np.float32)
    tie = rng.random((steps, B, E)) < 1 / 3
    logits[tie] = np.round(logits[tie] * 2) / 2
    x = rng.standard_normal((steps, B, H)).astype(np.float32)
    return logits, x


@pytest.mark.parametrize("E,k,K,B", [(64, 4, 64, 1), (65, 4, 13, 5), (200, 8, 24, 6),
                                     (255, 6, 101, 3), (256, 8, 77, 1), (256, 8, 256, 16)])
def test_host_steps_across_table_shapes(E, k, K, B):
    say("case: host-driven route, E=%d k=%d K=%d B=%d, 12 steps" % (E, k, K, B))
    p = PairedLayer(E, k, H, I, K, gen.F32, _fill(E, E + K), max_tokens=B)
    logits, x = _inputs(E, B, 12, E * 7 + K)
    worst = p.run(logits, x, check_state_every=1)
    say("worst rel err %.3g stats %s" % (worst, p.gpu.stats()))
    if B * k > K:
        assert p.gpu.stats()["waves"] > 12
    p.close()


@pytest.mark.parametrize("E,k,K,B", [(256, 8, 77, 1), (255, 6, 101, 3), (65, 4, 13, 3), (64, 8, 64, 8),
                                     (256, 8, 256, 4)])
def test_device_steps_across_table_shapes(E, k, K, B):
    say("case: device-resolved route, E=%d k=%d K=%d B=%d, 16 steps" % (E, k, K, B))
    assert B * k <= K
    p = PairedLayer(E, k, H, I, K, gen.F32, _fill(E, E + 3 * K), max_tokens=B)
    logits, x = _inputs(E, B, 16, E * 11 + K)
    lg = torch.from_numpy(logits).cuda()
    xd = torch.from_numpy(x).cuda()
    out = torch.empty(B, H, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    hits = misses = 0
    for t in range(16):
        p.gpu.step_device(p.plan, lg[t], xd[t], out)
        o_ref, ids_ref, w_ref, p_ref = p.ref.step(logits[t], x_values(x[t], p.fmt))
        assert p_ref.n_waves == 1
        hits += len(p_ref.hits)
        misses += len(p_ref.missed)
        ids, wts, sid, wof = p.plan.read()
        assert np.array_equal(ids, ids_ref), (t, ids, ids_ref)
        assert np.array_equal(sid, p_ref.slot_ids), (t, sid, p_ref.slot_ids)
        assert np.array_equal(wof, p_ref.wave_of)
        assert np.allclose(wts, w_ref, rtol=2e-6, atol=1e-7)
        torch.cuda.synchronize()
        e = rel_err(out.cpu().numpy(), o_ref)
        assert e <= TOL[gen.F32], (t, e)
        p.check_state()
    st = p.gpu.stats()
    assert st["steps"] == 16 and st["hits"] == hits and st["misses"] == misses and st["waves"] == 16
    p.close()
