"""GPU edge cases of the boundary: empty steps, K < top_k, K = E, the largest
E and top_k, error codes, the startup self-check, ordering under separate
streams (NaN canary in victim slots), and bitwise reproducibility."""
import ctypes

import numpy as np
import pytest
import torch

import expert_weight_paging_amd as ewp
import workloads as W
from workloads import gen

from gpu_harness import PairedLayer, say

pytestmark = pytest.mark.gpu


def _tiny_fill(E, H, I, fmt=gen.F32, seed=0):
    rng = np.random.default_rng(seed)
    recs = [gen.encode_record(fmt, (rng.standard_normal((2 * I, H)) * 0.05).astype(np.float32),
                              (rng.standard_normal((H, I)) * 0.05).astype(np.float32)) for _ in range(E)]

    def fill(a):
        for e in range(E):
            a[e] = recs[e]
    return fill


def _seq(E, B, steps, seed):
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((steps, B, E)).astype(np.float32)
    x = rng.standard_normal((steps, B, 64)).astype(np.float32)
    return logits, x


def test_empty_step_then_normal():
    say("case: T=0 route")
    p = PairedLayer(8, 2, 64, 32, 4, gen.F32, _tiny_fill(8, 64, 32), max_tokens=4)
    lg = torch.zeros(0, 8, dtype=torch.float32, device="cuda")
    info = p.gpu.route(p.plan, lg, num_tokens=0)
    assert info["num_waves"] == 0 and info["num_distinct"] == 0
    logits, x = _seq(8, 3, 6, 1)
    p.run(logits, x, check_state_every=1)
    p.close()


@pytest.mark.parametrize("K", [1, 2, 3, 8])
def test_small_and_full_tables(K):
    say("case: E=8 k=3 K=%d B=2 (K < top_k gives multi-wave steps)" % K)
    p = PairedLayer(8, 3, 64, 32, K, gen.F32, _tiny_fill(8, 64, 32, seed=K), max_tokens=2)
    logits, x = _seq(8, 2, 20, K)
    p.run(logits, x, check_state_every=1)
    st = p.gpu.stats()
    if K == 8:
        # K = E: after every expert has been seen there are no more misses
        assert st["misses"] <= 8
    if K < 3:
        assert st["waves"] > st["steps"]
    p.close()


def test_largest_e_and_top_k():
    E, k = 1024, 32
    say("case: E=1024 k=32 K=100 B=3")
    p = PairedLayer(E, k, 64, 32, 100, gen.F32, _tiny_fill(E, 64, 32), max_tokens=3)
    rng = np.random.default_rng(5)
    logits = rng.standard_normal((5, 3, E)).astype(np.float32)
    logits[:, :, :50] = np.round(logits[:, :, :50])         # plenty of exact ties
    x = rng.standard_normal((5, 3, 64)).astype(np.float32)
    p.run(logits, x, check_state_every=1)
    p.close()


def test_gemv_launch_past_512_experts():
    """A GEMV wave of about 650 distinct experts (E = K = 1024, 32 tokens of
    top-32): each down wavefront takes more than 64 experts, so the kernel's
    per-lane expert metadata needs its second register; ties included."""
    E, k, T = 1024, 32, 32
    say("case: E=K=1024 k=32 B=32, one wave of ~650 experts")
    p = PairedLayer(E, k, 64, 32, E, gen.F32, _tiny_fill(E, 64, 32, seed=11), max_tokens=T)
    rng = np.random.default_rng(12)
    logits = rng.standard_normal((3, T, E)).astype(np.float32)
    logits[:, :, :40] = np.round(logits[:, :, :40])
    x = rng.standard_normal((3, T, 64)).astype(np.float32)
    seen = []

    def count(pl, t, info):
        seen.append((info["num_distinct"], info["num_hits"]))
    p.run(logits, x, check_state_every=1, on_step=count)
    # the first step (cold table) is one launch of all its experts
    assert seen[0][1] == 0 and seen[0][0] > 8 * 64, seen
    p.close()


@pytest.mark.parametrize("fmt", [gen.F32, gen.FP8, gen.INT4])
def test_one_token_more_than_8_experts(fmt):
    """One token of top-16: 16 experts in one launch, two per down wavefront
    (the kernel variant that prefetches the next expert), on one token."""
    E, k, K, H, I = 64, 16, 32, 256, 128
    say("case: E=64 k=16 K=32 B=1 fmt=%d" % fmt)
    p = PairedLayer(E, k, H, I, K, fmt, _tiny_fill(E, H, I, fmt=fmt, seed=13), max_tokens=1)
    rng = np.random.default_rng(14)
    logits = rng.standard_normal((12, 1, E)).astype(np.float32)
    v = rng.standard_normal((12, 1, H)).astype(np.float32)
    x = v if fmt == gen.F32 else gen.f32_to_bf16_bits(v)
    p.run(logits, x, check_state_every=4)
    p.close()


def test_separate_streams_and_nan_canary():
    """Compute, copy and route on three streams; before each page-in the victim
    slots are filled with NaN on the copy stream. A forward that read a slot
    before its copy landed would produce NaN."""
    cfg = W.CONFIGS[2]
    say("case: bf16 layer on 3 streams with NaN-poisoned victims, 24 steps")
    s = (torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream())
    p = PairedLayer(cfg.E, cfg.top_k, cfg.H, cfg.I, cfg.K, cfg.fmt,
                    lambda a: gen.expert_store(cfg, out=a), max_tokens=1, streams=s)
    logits, x = gen.decode_inputs(cfg, 1, steps=24)
    rec = p.gpu.record_bytes
    slots = p.slots.view(cfg.K, rec)

    def poison(pl, t, info):
        # after the previous forward (compute stream), before this page-in (copy stream)
        ev = torch.cuda.Event()
        ev.record(s[0])
        s[1].wait_event(ev)
        for w in range(info["num_waves"]):
            _, _, misses = pl.plan.wave(w)
            with torch.cuda.stream(s[1]):
                for e, sl in misses:
                    slots[sl].fill_(0xFF)
    p.run(logits, x, on_step=poison, sample=lambda t: t % 6 == 5)
    p.close()


def test_bitwise_reproducible():
    cfg = W.CONFIGS[3]
    say("case: fp8 B=6 run twice -> identical bits")
    outs = []
    logits, x = gen.decode_inputs(cfg, 6, steps=6)
    for _ in range(2):
        p = PairedLayer(cfg.E, cfg.top_k, cfg.H, cfg.I, cfg.K, cfg.fmt,
                        lambda a: gen.expert_store(cfg, out=a), max_tokens=6)
        lg = torch.from_numpy(logits).cuda()
        xd = torch.from_numpy(x.view(np.int16)).cuda()
        out = torch.empty(6, cfg.H, dtype=torch.float32, device="cuda")
        res = []
        for t in range(6):
            p.gpu.step(p.plan, lg[t], xd[t], out)
            res.append(out.cpu().numpy().copy())
        outs.append(np.stack(res))
        p.close()
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))


def test_self_check_pass_and_fail():
    say("case: startup independence check")
    E, H, I = 8, 64, 32
    fill = _tiny_fill(E, H, I)
    p = PairedLayer(E, 2, H, I, 4, gen.F32, fill, max_tokens=1, self_check=True)
    p.close()

    def aliased(a):                       # expert 1's record is a copy of expert 0's
        fill(a)
        a[1] = a[0]
    with pytest.raises(ewp.MoeError) as ei:
        PairedLayer(E, 2, H, I, 4, gen.F32, aliased, max_tokens=1, self_check=True)
    assert ei.value.name == "MOE_ERR_SELFCHECK"


def _desc(E=8, k=2, H=64, I=32, K=4, fmt=0, rb=None, host=None, slots=None, state=None):
    rb = ewp.record_bytes(fmt, H, I) if rb is None else rb
    return ewp._Desc(E, k, H, I, K, fmt, rb, ctypes.c_void_p(host), ctypes.c_void_p(slots),
                     ctypes.c_void_p(state), 0, 0)


def _init(d):
    h = ctypes.c_void_p()
    return ewp.lib().moe_layer_init(ctypes.byref(d), None, None, None, ctypes.byref(h)), h


def test_error_codes():
    say("case: error codes")
    E, H, I, K = 8, 64, 32, 4
    rb = ewp.record_bytes(0, H, I)
    host = ewp.HostStore(E, rb)
    slots, state = ewp.alloc_layer_buffers(E, K, rb, "cuda")
    args = dict(host=host.ptr, slots=slots.data_ptr(), state=state.data_ptr())
    assert _init(_desc(K=0, **args))[0] == -1
    assert _init(_desc(K=9, **args))[0] == -1
    assert _init(_desc(k=9, **args))[0] == -1
    assert _init(_desc(rb=rb + 256, **args))[0] == -3
    assert _init(_desc(fmt=7, **args))[0] == -3
    assert _init(_desc(fmt=2, **args))[0] == -3          # FP8 needs multiples of 128
    pageable = np.zeros(E * rb, dtype=np.uint8)
    a2 = dict(args, host=pageable.ctypes.data)
    assert _init(_desc(**a2))[0] == -2
    st, h = _init(_desc(**args))
    assert st == 0
    layer = ewp.Layer.__new__(ewp.Layer)
    layer.handle, layer.top_k, layer.E, layer.K = h, 2, E, K
    with pytest.raises(ewp.MoeError) as ei:        # f32 layers stay on the GEMV path (<= 64 tokens)
        ewp.Plan(layer, 65)
    assert ei.value.name == "MOE_ERR_INVALID_ARG"
    plan = ewp.Plan(layer, 2)
    x = torch.zeros(2, H, device="cuda")
    out = torch.zeros(2, H, device="cuda")
    lg = torch.randn(2, E, device="cuda")
    with pytest.raises(ewp.MoeError) as ei:
        ewp._check(ewp.lib().moe_forward(h, plan.handle, 0, ctypes.c_void_p(x.data_ptr()),
                                         ctypes.c_void_p(out.data_ptr())))
    assert ei.value.name == "MOE_ERR_STATE"
    ewp._check(ewp.lib().moe_route(h, ctypes.c_void_p(lg.data_ptr()), 2, plan.handle))
    with pytest.raises(ewp.MoeError) as ei:       # route again before the waves ran
        ewp._check(ewp.lib().moe_route(h, ctypes.c_void_p(lg.data_ptr()), 2, plan.handle))
    assert ei.value.name == "MOE_ERR_STATE"
    with pytest.raises(ewp.MoeError) as ei:       # forward before page-in
        ewp._check(ewp.lib().moe_forward(h, plan.handle, 0, ctypes.c_void_p(x.data_ptr()),
                                         ctypes.c_void_p(out.data_ptr())))
    assert ei.value.name == "MOE_ERR_STATE"
    with pytest.raises(ewp.MoeError) as ei:       # more tokens than the plan holds
        ewp._check(ewp.lib().moe_route(h, ctypes.c_void_p(lg.data_ptr()), 3, plan.handle))
    assert ei.value.name in ("MOE_ERR_INVALID_ARG", "MOE_ERR_STATE")
    plan.close()
    layer.close()                                  # destroys h exactly once
    host.free()


def test_self_check_needs_two_slots_and_odd_k_passes():
    """The check places each expert in two different slots: K = 1 is refused at
    init, odd K (where a mirrored placement would keep the middle expert in
    its slot) passes."""
    say("case: self-check with K = 1 and K = 3")
    E, H, I = 8, 64, 32
    fill = _tiny_fill(E, H, I, seed=3)
    p = PairedLayer(E, 2, H, I, 3, gen.F32, fill, max_tokens=1, self_check=True)
    p.close()
    with pytest.raises(ewp.MoeError) as ei:
        PairedLayer(E, 1, H, I, 1, gen.F32, fill, max_tokens=1, self_check=True)
    assert ei.value.name == "MOE_ERR_INVALID_ARG"


class _PtrAttr(ctypes.Structure):
    _fields_ = [("type", ctypes.c_int), ("device", ctypes.c_int), ("devicePointer", ctypes.c_void_p),
                ("hostPointer", ctypes.c_void_p), ("isManaged", ctypes.c_int),
                ("allocationFlags", ctypes.c_uint)]


def _is_host_pinned(hip, addr):
    a = _PtrAttr()
    if hip.hipPointerGetAttributes(ctypes.byref(a), ctypes.c_void_p(addr)) != 0:
        hip.hipGetLastError()
        return False
    return a.type == 1


def test_store_with_unpinned_middle_is_refused():
    """A store whose first and last bytes are page-locked but whose middle is
    not (two pinned allocations with a gap between them) is refused with
    MOE_ERR_NOT_PINNED ([PE] "A rollout checklist": the whole store must be
    pinned, refused at startup); a store inside one allocation is accepted."""
    say("case: host store spanning two pinned allocations with an unpinned gap")
    H, I, K = 64, 32, 4
    rb = ewp.record_bytes(0, H, I)
    hip = ctypes.CDLL("libamdhip64.so.7")
    L = ewp.lib()
    bufs = [L.moe_host_alloc(1 << 20) for _ in range(6)]
    assert all(bufs)
    try:
        def extent(ptr):               # [base, base + size) of the allocation holding ptr
            base, size = ctypes.c_void_p(), ctypes.c_size_t()
            assert hip.hipPointerGetAttribute(ctypes.byref(base), 11, ctypes.c_void_p(ptr)) == 0
            assert hip.hipPointerGetAttribute(ctypes.byref(size), 12, ctypes.c_void_p(ptr)) == 0
            return base.value, base.value + size.value
        order = sorted(bufs)
        pick = None
        for a, c in zip(order, order[1:]):
            a_end = extent(a)[1]
            c_end = extent(c)[1]
            E = -(-(c - a + 1) // rb)
            if (c > a_end and E <= 1024 and a + E * rb <= c_end and
                    not _is_host_pinned(hip, a_end) and not _is_host_pinned(hip, c - 1)):
                pick = (a, E)
                break
        if pick is None:
            pytest.skip("no two pinned allocations with an unpinned gap within 1024 records")
        a, E = pick
        slots, state = ewp.alloc_layer_buffers(E, K, rb, "cuda")
        assert _is_host_pinned(hip, a) and _is_host_pinned(hip, a + E * rb - 1)
        st, h = _init(_desc(E=E, K=K, host=a, slots=slots.data_ptr(), state=state.data_ptr()))
        assert st == -2, (st, L.moe_last_error())
        # the same layer over one allocation is fine
        st, h = _init(_desc(E=8, K=K, host=a, slots=slots.data_ptr(), state=state.data_ptr()))
        assert st == 0, L.moe_last_error()
        L.moe_layer_destroy(h)
    finally:
        for b in bufs:
            L.moe_host_free(b)


def test_host_step_bits_do_not_depend_on_copy_progress():
    """A host-driven decode step gives the same bits whether its copies are
    still in flight when the forward is enqueued or already complete: the
    resident-first split is decided from the plan, not from timing."""
    cfg = W.CONFIGS[2]
    say("case: bf16 layer, 16 host-driven steps, copies complete vs in flight")
    logits, x = gen.decode_inputs(cfg, 1, steps=16)
    outs = []
    for sync_copies in (False, True):
        s = (torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream())
        p = PairedLayer(cfg.E, cfg.top_k, cfg.H, cfg.I, cfg.K, cfg.fmt,
                        lambda a: gen.expert_store(cfg, out=a), max_tokens=1, streams=s)
        lg = torch.from_numpy(logits).cuda()
        xd = torch.from_numpy(x.view(np.int16)).cuda()
        out = torch.empty(1, cfg.H, dtype=torch.float32, device="cuda")
        res = []
        for t in range(16):
            info = p.gpu.route(p.plan, lg[t])
            for w in range(info["num_waves"]):
                p.gpu.page_in(p.plan, w)
                if sync_copies:
                    torch.cuda.synchronize()
                p.gpu.forward(p.plan, w, xd[t], out)
            torch.cuda.synchronize()
            res.append(out.cpu().numpy().copy())
        outs.append(np.stack(res))
        p.close()
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))


@pytest.mark.parametrize("fmt", [gen.FP8, gen.INT4])
def test_zeroed_scale_block_is_flagged(fmt):
    """[PE] "Can paging change the model's outputs?": an expert that runs with
    the wrong scale tensor gives wrong outputs silently. Plant that failure in
    the GPU's host store (one 128x128 FP8 scale block, or the int4 gate/up
    scale table, of an expert the first step routes, set to zero) and check that
    parity against the oracle of the clean store flags it, while the plans
    stay exact (paging itself is not what is wrong)."""
    from oracle.layer import PagedLayer
    from oracle.router import route
    say("case: zeroed %s must fail parity" % {gen.FP8: "FP8 128x128 scale block", gen.INT4: "int4 W13 scales"}[fmt])
    E, k, H, I, K = 16, 2, 256, 256, 8
    rng = np.random.default_rng(77)
    recs = [gen.encode_record(fmt, (rng.standard_normal((2 * I, H)) * 0.02).astype(np.float32),
                              (rng.standard_normal((H, I)) * 0.02).astype(np.float32)) for _ in range(E)]
    clean = np.stack(recs)
    logits = rng.standard_normal((6, 1, E)).astype(np.float32)
    x = gen.f32_to_bf16_bits(rng.standard_normal((6, 1, H)).astype(np.float32))
    victim = int(route(logits[0], k)[0][0, 0])                 # the first step's top expert
    if fmt == gen.FP8:
        s13 = 2 * I * H + H * I                                # after both code matrices
        bad = slice(s13, s13 + 4)                              # W13 scale block (0, 0), float32
    else:
        s13 = (2 * I * H + H * I) // 2                         # after both packed code matrices
        bad = slice(s13, s13 + 2 * (2 * I) * (H // 128))       # every W13 group scale, float16

    def fill(a):
        a[:] = clean
        a[victim, bad] = 0
    p = PairedLayer(E, k, H, I, K, fmt, fill, max_tokens=1)
    assert p.host.array[victim, bad].max() == 0 and clean[victim, bad].max() > 0
    p.ref = PagedLayer(clean, fmt, E, k, H, I, K)              # the oracle reads the clean bytes
    with pytest.raises(AssertionError) as ei:
        p.run(logits, x, check_state_every=1)
    step, err, tol = ei.value.args[0]                          # the output check, not a plan check
    say("flagged at step %d: rel err %.3g > %.3g" % (step, err, tol))
    assert err > tol
    p.close()
