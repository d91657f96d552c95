"""GPU parity of the device-resolved path (moe_step_device and
moe_stack_forward_device: route, slot plan, kernel page-in and FFN with no host
synchronisation; one wave, or several when T * top_k > K) against the oracle,
its interleaving with host-driven steps, and its HIP-graph capture against
eager runs, all through the C ABI."""
import numpy as np
import pytest
import torch

import expert_weight_paging_amd as ewp
import workloads as W
from oracle.layer import PagedLayer, bf16_rne
from workloads import gen

from stack_check import StackPair
from gpu_harness import TOL, PairedLayer, rel_err, say, x_values

pytestmark = pytest.mark.gpu


def _layer(cfg, B, K=None, **kw):
    K = cfg.K if K is None else K
    return PairedLayer(cfg.E, cfg.top_k, cfg.H, cfg.I, K, cfg.fmt,
                       lambda a: gen.expert_store(cfg, out=a), max_tokens=B, **kw)


def _dev(a):
    a = np.ascontiguousarray(a)
    return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).cuda()


def _check_device_plan(p, ids_ref, w_ref, p_ref):
    ids, wts, sid, wof = p.plan.read()
    assert np.array_equal(ids, ids_ref), (ids, ids_ref)
    assert np.array_equal(sid, p_ref.slot_ids)
    assert np.array_equal(wof, p_ref.wave_of)
    assert np.allclose(wts, w_ref, rtol=2e-6, atol=1e-7)


def _run_device(p, logits, x, sample, host_every=0):
    """Device-resolved steps (every host_every-th one host-driven instead);
    returns the worst output error and the oracle's hit and miss totals."""
    steps, B = logits.shape[0], logits.shape[1]
    lg, xd = _dev(logits), _dev(x)
    out = torch.empty(B, p.H, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()  # inputs in place before the layer's streams read them
    worst, hits, misses = 0.0, 0, 0
    for t in range(steps):
        comp = bool(sample(t))
        host = host_every and t % host_every == host_every - 1
        if host:
            info = p.gpu.route(p.plan, lg[t])
            for w in range(info["num_waves"]):
                p.gpu.page_in(p.plan, w)
                p.gpu.forward(p.plan, w, xd[t], out)
        else:
            p.gpu.step_device(p.plan, lg[t], xd[t], out)
        o_ref, ids_ref, w_ref, p_ref = p.ref.step(logits[t], x_values(x[t], p.fmt), compute=comp)
        hits += len(p_ref.hits)
        misses += len(p_ref.missed)
        if host:
            p.check_plan(ids_ref, w_ref, p_ref, B)
        else:
            _check_device_plan(p, ids_ref, w_ref, p_ref)
            with pytest.raises(ewp.MoeError):
                p.plan.info()  # the host view is not updated by a device step
        if comp:
            torch.cuda.synchronize()
            e = rel_err(out.cpu().numpy(), o_ref)
            worst = max(worst, e)
            assert e <= TOL[p.fmt], (t, e)
        if (t + 1) % 8 == 0:
            p.check_state()
    torch.cuda.synchronize()
    p.check_state()
    return worst, hits, misses


def test_tiny_f32_device_steps():
    cfg = W.CONFIGS[1]
    say("case: device steps, tiny f32 E=8 k=2 K=4, 16 steps")
    p = _layer(cfg, 1)
    logits, x = gen.decode_inputs(cfg, 1)
    worst, hits, misses = _run_device(p, logits, x, sample=lambda t: True)
    st = p.gpu.stats()
    say("worst rel err %.3g stats %s" % (worst, st))
    assert st["steps"] == 16 and st["hits"] == hits and st["misses"] == misses
    assert st["bytes_paged"] == misses * ewp.record_bytes(cfg.fmt, cfg.H, cfg.I)
    p.close()


@pytest.mark.parametrize("split", [False, True])
def test_bf16_device_steps(split):
    cfg = W.CONFIGS[2]
    # the benchmark's decode workload as it times it: 32 warm-up and 256 timed
    # steps from a cold table, every plan checked, outputs sampled
    n = 288 if not split else 64
    say("case: device steps, bf16 layer K=40, %d steps at batch 1, own copy stream=%s" % (n, split))
    streams = None
    if split:  # a layer with a copy stream of its own: device steps stay on the compute stream
        c = torch.cuda.Stream()
        streams = (c, torch.cuda.Stream(), c)
    p = _layer(cfg, 1, streams=streams)
    logits, x = gen.decode_inputs(cfg, 1, steps=n)
    worst, hits, misses = _run_device(p, logits, x, sample=lambda t: t % 16 == 0 or t == n - 1)
    st = p.gpu.stats()
    say("worst rel err %.3g hits %d misses %d" % (worst, hits, misses))
    assert st["hits"] == hits and st["misses"] == misses and st["waves"] == n
    p.close()


@pytest.mark.parametrize("B", [1, 2, 5])
def test_fp8_device_steps(B):
    cfg = W.CONFIGS[3]
    say("case: device steps, fp8 layer K=40, B=%d, 24 steps" % B)
    p = _layer(cfg, B)
    logits, x = gen.decode_inputs(cfg, B, steps=24)
    worst, _, _ = _run_device(p, logits, x, sample=lambda t: t % 4 == 0 or t == 23)
    say("worst rel err %.3g" % worst)
    p.close()


def test_mxfp4_device_steps():
    cfg = W.CONFIGS[6]
    say("case: device steps, mxfp4 layer K=40, 32 steps at batch 1")
    p = _layer(cfg, 1)
    logits, x = gen.decode_inputs(cfg, 1, steps=32)
    worst, hits, misses = _run_device(p, logits, x, sample=lambda t: t % 4 == 0 or t == 31)
    st = p.gpu.stats()
    say("worst rel err %.3g hits %d misses %d" % (worst, hits, misses))
    assert st["hits"] == hits and st["misses"] == misses
    p.close()


@pytest.mark.parametrize("cid,B,K", [(1, 5, 4), (3, 6, 40), (3, 8, 40), (3, 4, 24)])
def test_token_waves(cid, B, K):
    """Batches beyond one wave as groups of K // top_k tokens, each a
    device-resolved single-wave step, against the oracle's token waves."""
    cfg = W.CONFIGS[cid]
    steps = 16
    say("case: token waves, %s B=%d K=%d, %d steps" % (cfg.name, B, K, steps))
    p = _layer(cfg, B, K=K)
    G = p.gpu.group_tokens(p.plan)
    assert G == K // cfg.top_k
    logits, x = gen.decode_inputs(cfg, B, steps=steps)
    lg, xd = _dev(logits), _dev(x)
    out = torch.empty(B, p.H, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    hits = misses = 0
    worst = 0.0
    for t in range(steps):
        comp = t % 3 == 0 or t == steps - 1
        p.gpu.step_token_waves(p.plan, lg[t], xd[t], out)
        o_ref, ids_ref, w_ref, plans = p.ref.step_token_waves(logits[t], x_values(x[t], p.fmt), G, compute=comp)
        assert len(plans) == -(-B // G)
        hits += sum(len(q.hits) for q in plans)
        misses += sum(len(q.missed) for q in plans)
        last = (len(plans) - 1) * G
        _check_device_plan(p, ids_ref[last:], w_ref[last:], plans[-1])
        if comp:
            torch.cuda.synchronize()
            e = rel_err(out.cpu().numpy(), o_ref)
            worst = max(worst, e)
            assert e <= TOL[p.fmt], (t, e)
        if (t + 1) % 4 == 0:
            p.check_state()
    torch.cuda.synchronize()
    p.check_state()
    st = p.gpu.stats()
    say("worst rel err %.3g hits %d misses %d" % (worst, hits, misses))
    assert st["hits"] == hits and st["misses"] == misses
    p.close()


def test_int4_device_steps_interleaved_with_host_steps():
    cfg = W.CONFIGS[4]
    say("case: int4 layer K=92, 40 steps, every third one host-driven")
    p = _layer(cfg, 1)
    logits, x = gen.decode_inputs(cfg, 1, steps=40)
    worst, hits, misses = _run_device(p, logits, x, sample=lambda t: t % 4 == 0 or t == 39, host_every=3)
    st = p.gpu.stats()
    say("worst rel err %.3g stats %s" % (worst, st))
    assert st["steps"] == 40 and st["hits"] == hits and st["misses"] == misses
    p.close()


@pytest.mark.parametrize("cid,B,K,steps", [(3, 6, 40, 32), (3, 8, 40, 32), (1, 5, 4, 16), (2, 1, 4, 12),
                                           (3, 8, 24, 16)])
def test_multi_wave_device_steps(cid, B, K, steps):
    """Batches whose routed experts can exceed K ([PE] "What happens with more
    than one request?"): device-resolved expert waves, each wave's misses paged
    in before its experts run; every step's plan (ids, weights, slot and wave of
    each pair), the table state and sampled outputs against the oracle, with
    every fifth step host-driven. Covers B * top_k just past K (B = 6), well
    past it (B = 8, K = 24: up to three waves), one token with K < top_k, and
    the tiny f32 layer (up to three waves of four)."""
    cfg = W.CONFIGS[cid]
    say("case: multi-wave device steps, %s B=%d K=%d, %d steps" % (cfg.name, B, K, steps))
    p = _layer(cfg, B, K=K)
    logits, x = gen.decode_inputs(cfg, B, steps=steps)
    worst, hits, misses = _run_device(p, logits, x, sample=lambda t: t % 4 == 0 or t == steps - 1,
                                      host_every=5)
    st = p.gpu.stats()
    say("worst rel err %.3g hits %d misses %d waves %d" % (worst, hits, misses, st["waves"]))
    assert st["hits"] == hits and st["misses"] == misses and st["waves"] > steps
    p.close()


def test_device_step_rejects_too_many_waves():
    cfg = W.CONFIGS[3]
    say("case: device step that may need more than 16 waves is rejected")
    p = _layer(cfg, 9, K=4)  # min(9 * 8, 128) / 4 = 18 possible waves
    logits, x = gen.decode_inputs(cfg, 9, steps=1)
    out = torch.empty(9, cfg.H, dtype=torch.float32, device="cuda")
    with pytest.raises(ewp.MoeError) as ei:
        p.gpu.step_device(p.plan, _dev(logits[0]), _dev(x[0]), out)
    assert ei.value.status == -1  # MOE_ERR_INVALID_ARG
    p.close()


def _int4_stack(cfg, n_layers, s, c):
    rec = ewp.record_bytes(cfg.fmt, cfg.H, cfg.I)
    pool = gen.pool_records(cfg)
    hosts, layers, plans, refs = [], [], [], []
    for l in range(n_layers):
        h = ewp.HostStore(cfg.E, rec)
        gen.fill_layer_store(cfg, l, h.array, pool)
        slots, state = ewp.alloc_layer_buffers(cfg.E, cfg.K, rec, "cuda")
        L = ewp.Layer(cfg.E, cfg.top_k, cfg.H, cfg.I, cfg.K, cfg.fmt, h, slots, state, s, c, s)
        hosts.append(h)
        layers.append(L)
        plans.append(ewp.Plan(L, 1))
        refs.append(PagedLayer(h.array, cfg.fmt, cfg.E, cfg.top_k, cfg.H, cfg.I, cfg.K))
    return hosts, layers, plans, refs


def _close_stack(hosts, layers, plans):
    for p in plans:
        p.close()
    for L in layers:
        L.close()
    for h in hosts:
        h.free()


@pytest.mark.parametrize("lookahead", [False, True])
def test_int4_stack_device(lookahead):
    """moe_stack_forward_device against a twin stack stepped layer by layer
    with every layer checked against the oracle (tests/stack_check.py): the
    hidden state, output, plans and table state must be bitwise equal."""
    cfg = W.CONFIGS[4]
    n_layers, steps = 4, 12
    say("case: int4 stack %d layers x %d tokens, device-resolved, lookahead=%s" % (n_layers, steps, lookahead))
    s, c = torch.cuda.Stream(), torch.cuda.Stream()
    A = StackPair(cfg, n_layers, 1, False, (s, c, s), keep_refs=False)
    sb = torch.cuda.Stream()
    B = StackPair(cfg, n_layers, 1, False, (sb, torch.cuda.Stream(), sb))
    rng = np.random.default_rng(5)
    worst = {}
    for step in range(steps):
        sets = np.stack([np.sort(rng.choice(cfg.E, cfg.top_k, replace=False))[None] for _ in range(n_layers)])
        logits = gen.logits_from_sets(rng, sets, cfg.E)                      # [L][1][E]
        x0 = gen.f32_to_bf16_bits(rng.standard_normal((1, cfg.H)).astype(np.float32))
        x = _dev(x0)
        out = torch.empty(1, cfg.H, dtype=torch.float32, device="cuda")
        lg = _dev(logits)
        torch.cuda.synchronize()  # inputs are in place before the stack's stream reads them
        ewp.stack_forward_device(A.layers, A.plans, lg, x, out, lookahead=lookahead)
        torch.cuda.synchronize()
        xb, ob, summ = B.run_token(logits, x0, "device", chain=slice(None))
        assert torch.equal(x, xb) and torch.equal(out, ob), step
        for l in range(n_layers):
            for u, v in zip(A.plans[l].read(), B.plans[l].read()):
                assert np.array_equal(u, v), (step, l)
            for u, v in zip(A.layers[l].get_state(), B.layers[l].get_state()):
                assert np.array_equal(np.asarray(u), np.asarray(v)), (step, l)
        for k, v in summ.items():
            worst[k] = max(worst.get(k, 0.0), v)
    say("worst: %s" % worst)
    A.close()
    B.close()


def test_int4_stack_device_lookahead_graph_replays_match_eager():
    """A token through a 3-layer int4 stack with device lookahead (the next
    layer routed and paged in by the up launch of the layer before) captured in a HIP graph;
    6 replays, with eager input copies and synchronisations between them,
    must equal an eager twin stack bit for bit (x, out, plans, table state)."""
    cfg = W.CONFIGS[4]
    n_layers, steps = 3, 6
    say("case: int4 stack %d layers, device lookahead captured in a graph, %d replays" % (n_layers, steps))
    sa, ca, sb, cb = (torch.cuda.Stream() for _ in range(4))
    A = _int4_stack(cfg, n_layers, sa, ca)
    B = _int4_stack(cfg, n_layers, sb, cb)
    rng = np.random.default_rng(9)
    sets = np.stack([np.stack([np.sort(rng.choice(cfg.E, cfg.top_k, replace=False))[None]
                               for _ in range(n_layers)]) for _ in range(steps)])
    logits = _dev(gen.logits_from_sets(rng, sets, cfg.E))                 # [steps][L][1][E]
    x0 = _dev(gen.f32_to_bf16_bits(rng.standard_normal((steps, 1, cfg.H)).astype(np.float32)))
    lg_buf = torch.zeros_like(logits[0])
    xa = torch.zeros(1, cfg.H, dtype=torch.int16, device="cuda")
    xb = torch.zeros_like(xa)
    oa = torch.zeros(1, cfg.H, dtype=torch.float32, device="cuda")
    ob = torch.zeros_like(oa)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=sb):
        ewp.stack_forward_device(B[1], B[2], lg_buf, xb, ob, lookahead=True)
    torch.cuda.synchronize()
    for t in range(steps):
        lg_buf.copy_(logits[t])
        xb.copy_(x0[t])
        xa.copy_(x0[t])
        torch.cuda.synchronize()
        g.replay()
        ewp.stack_forward_device(A[1], A[2], logits[t], xa, oa, lookahead=True)
        torch.cuda.synchronize()
        assert torch.equal(xa, xb) and torch.equal(oa, ob), t
        for l in range(n_layers):
            for u, v in zip(A[2][l].read(), B[2][l].read()):
                assert np.array_equal(u, v), (t, l)
            for u, v in zip(A[1][l].get_state(), B[1][l].get_state()):
                assert np.array_equal(np.asarray(u), np.asarray(v)), (t, l)
    del g
    _close_stack(A[0], A[1], A[2])
    _close_stack(B[0], B[1], B[2])


@pytest.mark.parametrize("cid,B", [(2, 1), (3, 6)], ids=["bf16-one-wave", "fp8-B6-waves"])
def test_device_step_graph_replays_match_eager(cid, B):
    """One device-resolved step captured in a HIP graph, replayed for 10
    decode steps with eager input copies and synchronisations between the
    replays; every replay's output, plan and table state must equal an eager
    twin layer's bit for bit. At B = 6 (48 pairs, K = 40) the graph holds the
    launches of two possible waves."""
    cfg = W.CONFIGS[cid]
    steps = 10
    say("case: %s device step at B=%d captured in a graph, %d replays vs eager" % (cfg.name, B, steps))
    rec = ewp.record_bytes(cfg.fmt, cfg.H, cfg.I)
    host = ewp.HostStore(cfg.E, rec)
    gen.expert_store(cfg, out=host.array)
    s_eager, s_cap = torch.cuda.Stream(), torch.cuda.Stream()
    mk = []
    for s in (s_eager, s_cap):
        # a copy stream of its own (device steps keep to the compute stream)
        slots, state = ewp.alloc_layer_buffers(cfg.E, cfg.K, rec, "cuda")
        L = ewp.Layer(cfg.E, cfg.top_k, cfg.H, cfg.I, cfg.K, cfg.fmt, host, slots, state, s,
                      torch.cuda.Stream(), s)
        mk.append((L, ewp.Plan(L, B), slots, state))
    (La, Pa, _, _), (Lb, Pb, _, _) = mk
    logits, x = gen.decode_inputs(cfg, B, steps=steps)
    lg, xd = _dev(logits), _dev(x)
    lg_buf = torch.zeros(B, cfg.E, dtype=torch.float32, device="cuda")
    x_buf = torch.zeros(B, cfg.H, dtype=torch.int16, device="cuda")
    out_b = torch.zeros(B, cfg.H, dtype=torch.float32, device="cuda")
    out_a = torch.zeros(B, cfg.H, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s_cap):
        Lb.step_device(Pb, lg_buf, x_buf, out_b)
    torch.cuda.synchronize()
    for t in range(steps):
        lg_buf.copy_(lg[t])
        x_buf.copy_(xd[t])
        g.replay()
        with torch.cuda.stream(s_eager):
            La.step_device(Pa, lg[t], xd[t], out_a)
        torch.cuda.synchronize()
        assert torch.equal(out_a, out_b), t
        ra, rb = Pa.read(), Pb.read()
        for u, v in zip(ra, rb):
            assert np.array_equal(u, v), t
        for u, v in zip(La.get_state(), Lb.get_state()):
            assert np.array_equal(np.asarray(u), np.asarray(v)), t
    assert La.stats() == Lb.stats()
    say("replays equal eager; stats %s" % Lb.stats())
    del g
    for L, P, _, _ in mk:
        P.close()
        L.close()
    host.free()


def test_multi_wave_device_step_applies_the_residual_once():
    """x_res on a device step that may need two waves (B = 6, 48 pairs, K = 40):
    the residual is applied exactly once, by the launch holding the step's
    last expert, to the final out: x_res == bf16_rne(x + out) computed in fp32
    from the GPU's own out, bit for bit; out itself within the oracle's
    tolerance. Steps with one and with two actual waves both occur."""
    cfg = W.CONFIGS[3]
    B, steps = 6, 12
    say("case: multi-wave device steps with the stack residual, fp8 B=%d K=40, %d steps" % (B, steps))
    p = _layer(cfg, B)
    logits, x = gen.decode_inputs(cfg, B, steps=steps)
    lg, xd = _dev(logits), _dev(x)
    out = torch.empty(B, cfg.H, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    waves_seen = set()
    for t in range(steps):
        xr = xd[t].clone()
        w0 = p.gpu.stats()["waves"]
        p.gpu.step_device(p.plan, lg[t], xd[t], out, x_res=xr)
        torch.cuda.synchronize()
        waves_seen.add(p.gpu.stats()["waves"] - w0)
        o = out.cpu().numpy()
        xs = gen.bf16_bits_to_f32(x[t]).astype(np.float32)
        want = gen.f32_to_bf16_bits(xs + o)
        assert np.array_equal(xr.cpu().numpy().view(np.uint16), want), t
        o_ref, ids_ref, w_ref, p_ref = p.ref.step(logits[t], x_values(x[t], p.fmt))
        _check_device_plan(p, ids_ref, w_ref, p_ref)
        assert rel_err(o, o_ref) <= TOL[p.fmt], t
    say("waves per step seen: %s" % sorted(waves_seen))
    assert waves_seen == {1, 2}
    p.check_state()
    p.close()
