"""GPU parity of the prefill path (token-grouped MFMA GEMMs + combine) against
the oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import expert_weight_paging_amd as ewp
import workloads as W
from oracle.layer import PagedLayer, bf16_rne, run_stack
from workloads import gen

from gpu_harness import TOL, PairedLayer, rel_err, say, x_values

pytestmark = pytest.mark.gpu


def _prefill_layer_check(p, logits, x, tol=2e-2):
    T = logits.shape[0]
    dev = p.dev
    lg = torch.from_numpy(np.ascontiguousarray(logits)).to(dev)
    xd = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev)
    out = torch.empty(T, p.H, dtype=torch.float32, device=dev)
    info = p.gpu.route(p.plan, lg)
    for w in range(info["num_waves"]):
        p.gpu.page_in(p.plan, w)
        p.gpu.forward(p.plan, w, xd, out)
    o_ref, ids_ref, w_ref, p_ref = p.ref.step(logits, x_values(x, p.fmt))
    p.check_plan(ids_ref, w_ref, p_ref, T)
    torch.cuda.synchronize()
    e = rel_err(out.cpu().numpy(), o_ref)
    say("prefill T=%d waves=%d misses=%d rel err %.3g" % (T, info["num_waves"], info["num_misses"], e))
    assert e <= tol
    p.check_state()
    return info


def test_prefill_qwen_layer_2048_tokens():
    cfg = W.CONFIGS[5]
    say("case: prefill bf16 layer E=128 k=8 H=2048 I=768 K=92 warm, 2048 tokens")
    p = PairedLayer(cfg.E, cfg.top_k, cfg.H, cfg.I, cfg.K, cfg.fmt,
                    lambda a: gen.expert_store(cfg, out=a), max_tokens=2048, initial_fill=True)
    logits, x0 = gen.prefill_inputs(cfg, layers=1)
    info = _prefill_layer_check(p, logits[0], x0)
    assert info["num_waves"] == 2 and info["num_misses"] == 36
    p.close()


@pytest.mark.parametrize("H,I", [(256, 384), (640, 256), (2176, 128)])
@pytest.mark.parametrize("fmt", [gen.FP8, gen.INT4, gen.MXFP4])
def test_prefill_quantised_formats(fmt, H, I):
    """More than 64 tokens with FP8, int4 and MXFP4 experts through the MFMA
    GEMMs (two waves per step), the records read in place. H = 640 leaves the
    down GEMM a last tile of 128 columns (its weight and scale rows past H are
    clamped); H = 2176 gives the 4-bit formats 68 bytes of scales (and zero
    points) per up row, past the GEMM's LDS scale region, so their records
    take the expansion pass to bf16 instead."""
    T, E, k, K = 300, 16, 2, 12
    say("case: prefill %s T=%d E=%d k=%d H=%d I=%d K=%d" % ({gen.FP8: "fp8", gen.INT4: "int4", gen.MXFP4: "mxfp4"}[fmt], T, E, k, H, I, K))
    rng = np.random.default_rng(40 + fmt + H)
    recs = [gen.encode_record(fmt, (rng.standard_normal((2 * I, H)) * 0.02).astype(np.float32),
                              (rng.standard_normal((H, I)) * 0.02).astype(np.float32)) for _ in range(E)]

    def fill(a):
        for e in range(E):
            a[e] = recs[e]
    p = PairedLayer(E, k, H, I, K, fmt, fill, max_tokens=T)
    for step in range(2):
        logits = rng.standard_normal((T, E)).astype(np.float32)
        x = gen.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
        info = _prefill_layer_check(p, logits, x, tol=TOL[fmt])
        assert info["num_waves"] == 2
    p.close()


def test_prefill_mxfp4_qwen_layer_2048_tokens():
    cfg = W.CONFIGS[6]
    K = 92
    say("case: prefill mxfp4 layer E=128 k=8 H=2048 I=768 K=92 warm, 2048 tokens")
    p = PairedLayer(cfg.E, cfg.top_k, cfg.H, cfg.I, K, cfg.fmt,
                    lambda a: gen.expert_store(cfg, out=a), max_tokens=2048, initial_fill=True)
    rng = np.random.default_rng(2048)
    logits = rng.standard_normal((2048, cfg.E)).astype(np.float32)
    x = gen.f32_to_bf16_bits(rng.standard_normal((2048, cfg.H)).astype(np.float32))
    info = _prefill_layer_check(p, logits, x, tol=TOL[cfg.fmt])
    assert info["num_waves"] == 2
    p.close()


@pytest.mark.parametrize("T,E,k,H,I,K", [(1000, 64, 4, 512, 256, 20), (65, 32, 8, 256, 128, 12),
                                         (300, 16, 2, 768, 384, 16)])
def test_prefill_ragged(T, E, k, H, I, K):
    say("case: prefill ragged T=%d E=%d k=%d H=%d I=%d K=%d" % (T, E, k, H, I, K))
    rng = np.random.default_rng(T + E)
    recs = [gen.encode_record(gen.BF16, (rng.standard_normal((2 * I, H)) * 0.02).astype(np.float32),
                              (rng.standard_normal((H, I)) * 0.02).astype(np.float32)) for _ in range(E)]

    def fill(a):
        for e in range(E):
            a[e] = recs[e]
    p = PairedLayer(E, k, H, I, K, gen.BF16, fill, max_tokens=T)
    for step in range(2):
        logits = rng.standard_normal((T, E)).astype(np.float32)
        x = gen.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
        _prefill_layer_check(p, logits, x)
    p.close()


def test_prefill_stack_residual():
    """Three bf16 layers at full shape with the device norm and residual,
    against the oracle's stack run from the same x0 (each layer reads the
    unit-gain RMSNorm of the residual stream). Each layer's MoE output must meet the
    bf16 output tolerance. The hidden state is bf16, so where the two sides'
    sums straddle a rounding boundary they differ by one bf16 ulp; element-wise
    the final hidden state may differ by the last layer's output tolerance plus
    one ulp of each intermediate hidden value, and such flips must be rare."""
    cfg = W.CONFIGS[5]
    L, T = 3, 512
    say("case: prefill stack of %d bf16 layers, %d tokens" % (L, T))
    logits, x0 = gen.prefill_inputs(cfg, layers=L, tokens=T, salt=7)
    pool = gen.expert_store(cfg)
    layers, refs = [], []
    for l in range(L):
        perm = gen.layer_permutation(cfg, l)
        p = PairedLayer(cfg.E, cfg.top_k, cfg.H, cfg.I, cfg.K, cfg.fmt,
                        lambda a, perm=perm: a.__setitem__(slice(None), pool[perm]),
                        max_tokens=T, initial_fill=True)
        layers.append(p)
        refs.append(p.ref)
    dev = "cuda:0"
    x = torch.from_numpy(np.ascontiguousarray(x0).view(np.int16)).to(dev)
    out = torch.empty(T, cfg.H, dtype=torch.float32, device=dev)
    lg = torch.from_numpy(logits).to(dev)
    outs = []
    a = torch.empty_like(x)
    for l, p in enumerate(layers):
        ewp.rmsnorm_bf16(x, a)
        info = p.gpu.route(p.plan, lg[l])
        for w in range(info["num_waves"]):
            p.gpu.page_in(p.plan, w)
            p.gpu.forward(p.plan, w, a, out)
        outs.append(out.cpu().numpy().copy())
        ewp.residual_bf16(x, out, x)
    torch.cuda.synchronize()
    xf_ref, outs_ref, plans = run_stack(refs, [logits[l] for l in range(L)], x_values(x0, cfg.fmt))
    for l in range(L):
        e = rel_err(outs[l], outs_ref[l])
        say("layer %d MoE output rel err %.3g" % (l, e))
        assert e <= 2e-2
    got = gen.bf16_bits_to_f32(x.cpu().numpy().view(np.uint16)).astype(np.float64)
    # bound per element: the output tolerance of the last layer plus one bf16
    # ulp of every intermediate hidden value the rounding may have flipped
    xl, bound = x_values(x0, cfg.fmt), 2e-2 * np.sqrt(np.mean(outs_ref[-1] ** 2))
    for o in outs_ref:
        xl = bf16_rne(xl + o)
        bound = bound + np.exp2(np.floor(np.log2(np.maximum(np.abs(xl), 2.0 ** -126))) - 7)
    d = np.abs(got - xf_ref)
    say("hidden: max diff / bound %.3g, %.2e of elements differ" % ((d / bound).max(), (d > 0).mean()))
    assert np.all(d <= bound)
    assert (d > 0).mean() < 2e-2
    for p in layers:
        p.check_state()
        p.close()


def test_residual_kernel_exact():
    rng = np.random.default_rng(3)
    n = 4096 * 3 + 2                                   # ragged tail

    def mag(v):                                        # |v| in [1/16, 8): sums of two stay exact in fp32
        return np.where(np.abs(v) < 1 / 16, np.sign(v + 1e-30) / 16, v)
    xb = gen.f32_to_bf16_bits(mag(rng.uniform(-8, 8, n)).astype(np.float32))
    # out values whose fp32 sum with x is exact, so both sides round the same value
    o = gen.bf16_bits_to_f32(gen.f32_to_bf16_bits(mag(rng.uniform(-8, 8, n)).astype(np.float32)))
    dev = "cuda:0"
    xd = torch.from_numpy(xb.view(np.int16)).to(dev)
    od = torch.from_numpy(o.astype(np.float32)).to(dev)
    yd = torch.empty_like(xd)
    ewp.residual_bf16(xd, od, yd)
    torch.cuda.synchronize()
    ref = bf16_rne(gen.bf16_bits_to_f32(xb).astype(np.float64) + o.astype(np.float64))
    got = gen.bf16_bits_to_f32(yd.cpu().numpy().view(np.uint16)).astype(np.float64)
    assert np.array_equal(got, ref)


def test_rmsnorm_kernel():
    """The unit-gain RMSNorm of a stack layer's input against the oracle's
    float64 norm, rounded to bf16: equal up to one bf16 ulp where float32 and
    float64 straddle a rounding boundary (rare); rows of very different
    scales, a zero row, H not a multiple of the workgroup's 2048 values, and
    in place."""
    rng = np.random.default_rng(12)
    from oracle.layer import rms_norm
    for T, H in ((7, 2048), (3, 520), (65, 8)):
        v = rng.standard_normal((T, H)) * np.exp2(rng.integers(-30, 30, (T, 1)))
        v[0] = 0.0
        xb = gen.f32_to_bf16_bits(v.astype(np.float32))
        xd = torch.from_numpy(xb.view(np.int16)).cuda()
        ad = torch.empty_like(xd)
        ewp.rmsnorm_bf16(xd, ad)
        torch.cuda.synchronize()
        got = gen.bf16_bits_to_f32(ad.cpu().numpy().view(np.uint16)).astype(np.float64)
        ref = bf16_rne(rms_norm(gen.bf16_bits_to_f32(xb).astype(np.float64)))
        ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -126))) - 7)
        d = np.abs(got - ref)
        say("norm T=%d H=%d: %d of %d values one ulp apart" % (T, H, int((d > 0).sum()), d.size))
        assert np.all(d <= ulp) and (d > 0).mean() < 1e-2
        assert np.all(got[0] == 0.0)
        ewp.rmsnorm_bf16(xd, xd)                        # in place
        torch.cuda.synchronize()
        assert torch.equal(xd, ad)


@pytest.mark.parametrize("cid", [3, 4, 6], ids=["fp8", "int4", "mxfp4"])
def test_prefill_quantised_qwen_layer_reads_records_in_place(cid):
    """FP8, int4 and MXFP4 prefill at the 2048-token Qwen shape (K=92 warm,
    two waves): the GEMMs read the records in place and widen each weight to
    bf16 in registers (value times its block scale, or (q - z) times s, in
    fp32, rounded to nearest even). Against the oracle to the format's tolerance, and bitwise against a
    bf16 layer whose records hold exactly those bf16 values (the expansion a
    separate pass would have written): the same matrix-core inputs in the
    same order."""
    from oracle import formats
    cfg = W.CONFIGS[cid]
    K, T = 92, 2048
    say("case: prefill %s layer E=128 k=8 H=2048 I=768 K=92 warm, 2048 tokens, in place vs expanded bf16"
        % cfg.name)
    ql = PairedLayer(cfg.E, cfg.top_k, cfg.H, cfg.I, K, cfg.fmt, lambda a: gen.expert_store(cfg, out=a),
                     max_tokens=T, initial_fill=True)

    def expanded(a):
        for e in range(cfg.E):
            g, u, d = formats.decode_record(ql.host.array[e], cfg.fmt, cfg.H, cfg.I)
            w13 = np.concatenate([g, u]).astype(np.float32)       # exact products rounded to fp32
            a[e] = gen.encode_record(gen.BF16, w13, d.astype(np.float32))
    bf = PairedLayer(cfg.E, cfg.top_k, cfg.H, cfg.I, K, gen.BF16, expanded, max_tokens=T, initial_fill=True)
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((T, cfg.E)).astype(np.float32)
    x = gen.f32_to_bf16_bits(rng.standard_normal((T, cfg.H)).astype(np.float32))
    lg = torch.from_numpy(logits).cuda()
    xd = torch.from_numpy(x.view(np.int16)).cuda()
    outs = []
    for p in (ql, bf):
        out = torch.empty(T, cfg.H, dtype=torch.float32, device="cuda")
        info = p.gpu.route(p.plan, lg)
        assert info["num_waves"] == 2 and info["num_misses"] == 36
        for w in range(info["num_waves"]):
            p.gpu.page_in(p.plan, w)
            p.gpu.forward(p.plan, w, xd, out)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
    o_ref, ids_ref, w_ref, p_ref = ql.ref.step(logits, x_values(x, cfg.fmt))
    ql.check_plan(ids_ref, w_ref, p_ref, T)
    e = rel_err(outs[0], o_ref)
    say("%s in place == expanded bf16 bitwise; rel err vs oracle %.3g" % (cfg.name, e))
    assert e <= TOL[cfg.fmt]
    ql.close()
    bf.close()
