"""moe_step_device_static, the entry point that allocates nothing (its step
workspace is the library's fixed device array), against moe_step_device on
the same inputs through the C ABI: identical outputs, residual, table state
and counters on two calls in a row, the second with fewer tokens; each also
within tolerance of the oracle. A step whose workspace exceeds the fixed
array is refused."""
import numpy as np
import pytest
import torch

import expert_weight_paging_amd as ewp
import workloads as W
from oracle.layer import PagedLayer, bf16_rne
from workloads import gen

from gpu_harness import TOL, rel_err, say, x_values

pytestmark = pytest.mark.gpu


def test_static_step_matches_device_step():
    cfg = W.CONFIGS[3]                                     # FP8 layer, E=128 k=8 K=40
    say("case: moe_step_device_static vs moe_step_device, FP8 layer, T=4 then T=2")
    rec = ewp.record_bytes(cfg.fmt, cfg.H, cfg.I)
    host = ewp.HostStore(cfg.E, rec)
    gen.expert_store(cfg, out=host.array)
    layers = []
    for _ in range(2):
        slots, state = ewp.alloc_layer_buffers(cfg.E, cfg.K, rec, "cuda")
        layers.append((ewp.Layer(cfg.E, cfg.top_k, cfg.H, cfg.I, cfg.K, cfg.fmt, host, slots, state), slots,
                       state))
    A, B = layers[0][0], layers[1][0]
    plan = ewp.Plan(A, 4)
    ref = PagedLayer(host.array, cfg.fmt, cfg.E, cfg.top_k, cfg.H, cfg.I, cfg.K)
    logits, x = gen.decode_inputs(cfg, 4, steps=2)
    for call, T in enumerate((4, 2)):
        lg = torch.from_numpy(np.ascontiguousarray(logits[call, :T])).cuda()
        xd = torch.from_numpy(np.ascontiguousarray(x[call, :T]).view(np.int16)).cuda()
        out_a = torch.full((T, cfg.H), float("nan"), dtype=torch.float32, device="cuda")
        out_b = torch.full((T, cfg.H), float("nan"), dtype=torch.float32, device="cuda")
        xr_a, xr_b = xd.clone(), xd.clone()
        A.step_device(plan, lg, xd, out_a, x_res=xr_a if call else None)
        B.step_device_static(lg, xd, out_b, x_res=xr_b if call else None)
        torch.cuda.synchronize()
        oa, ob = out_a.cpu().numpy(), out_b.cpu().numpy()
        assert np.array_equal(oa.view(np.uint32), ob.view(np.uint32)), call
        assert torch.equal(xr_a, xr_b)
        o_ref, ids_ref, _, p_ref = ref.step(logits[call, :T], x_values(x[call, :T], cfg.fmt))
        e = rel_err(ob, o_ref)
        say("call %d T=%d: bitwise equal, rel err vs oracle %.3g" % (call, T, e))
        assert e <= TOL[cfg.fmt]
        ids, _, sid, _ = plan.read()
        assert np.array_equal(ids, ids_ref) and np.array_equal(sid, p_ref.slot_ids)
        if call:
            xv = bf16_rne(x_values(x[call, :T], cfg.fmt) + ob.astype(np.float64))
            got = gen.bf16_bits_to_f32(xr_b.cpu().numpy().view(np.uint16)).astype(np.float64)
            # one bf16 ulp where the fp32 and fp64 sums straddle a rounding boundary
            ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(xv), 2.0 ** -126))) - 7)
            assert np.all(np.abs(got - xv) <= ulp)
        sa, sb = A.get_state(), B.get_state()
        for u, v in zip(sa, sb):
            assert np.array_equal(np.asarray(u), np.asarray(v))
        rse, res, rst, rclk = ref.table.state()
        assert np.array_equal(sb[0], rse) and np.array_equal(sb[2], rst) and sb[3] == rclk
        assert A.stats() == B.stats()
    plan.close()
    for L, _, _ in layers:
        L.close()
    host.free()


def test_static_step_refuses_oversized_workspace():
    """T * top_k * I * 4 bytes of h beyond the fixed array: refused before any
    launch, and the layer still takes a step that fits."""
    E, k, H, I = 256, 8, 32, 4096
    say("case: moe_step_device_static workspace limit, mxfp4 E=K=%d k=%d H=%d I=%d" % (E, k, H, I))
    rec = ewp.record_bytes(gen.MXFP4, H, I)
    host = ewp.HostStore(E, rec)
    host.array[:] = 0
    slots, state = ewp.alloc_layer_buffers(E, E, rec, "cuda")
    L = ewp.Layer(E, k, H, I, E, gen.MXFP4, host, slots, state)
    lg = torch.randn(32, E, device="cuda")
    x = torch.zeros(32, H, dtype=torch.int16, device="cuda")
    out = torch.empty(32, H, device="cuda")
    with pytest.raises(ewp.MoeError) as ei:                # 256 pairs x 4096 x 4 B = 4 MiB of h alone
        L.step_device_static(lg, x, out)
    assert ei.value.name == "MOE_ERR_INVALID_ARG"
    L.step_device_static(lg[:8], x[:8], out[:8])           # 64 pairs: fits
    torch.cuda.synchronize()
    assert torch.all(out[:8] == 0)                         # all-zero experts
    st = L.stats()
    assert st["steps"] == 1 and st["misses"] == st["refs"] > 0
    L.close()
    host.free()
