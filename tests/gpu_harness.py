"""Shared helpers of the GPU parity tests: run the HIP path and the oracle
side by side on the same seeded inputs and compare.

Integer results (top-k ids, slot of each pair, wave of each pair, wave
expert lists, miss lists, table state) must be bit-exact; outputs within
max|gpu - oracle| / rms(oracle) of the format's tolerance.
"""
import sys

import numpy as np
import torch

import expert_weight_paging_amd as ewp
from oracle.layer import PagedLayer
from workloads import gen

TOL = {gen.F32: 1e-5, gen.BF16: 2e-2, gen.FP8: 5e-2, gen.INT4: 5e-2, gen.MXFP4: 5e-2}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_err(got, ref):
    rms = float(np.sqrt(np.mean(np.asarray(ref, np.float64) ** 2)))
    return float(np.abs(np.asarray(got, np.float64) - ref).max()) / max(rms, 1e-30)


def x_values(x, fmt):
    return x.astype(np.float64) if fmt == gen.F32 else gen.bf16_bits_to_f32(x).astype(np.float64)


class PairedLayer:
    """A GPU layer and the oracle layer over the same pinned store bytes."""

    def __init__(self, E, k, H, I, K, fmt, store_fill, max_tokens, initial_fill=False,
                 self_check=False, streams=None, dev="cuda:0"):
        self.E, self.k, self.H, self.I, self.K, self.fmt = E, k, H, I, K, fmt
        rec = ewp.record_bytes(fmt, H, I)
        assert rec == gen.record_stride(fmt, H, I)
        self.host = ewp.HostStore(E, rec)
        store_fill(self.host.array)
        self.slots, self.state = ewp.alloc_layer_buffers(E, K, rec, dev)
        s = streams or (None, None, None)
        self.gpu = ewp.Layer(E, k, H, I, K, fmt, self.host, self.slots, self.state,
                             s[0], s[1], s[2], initial_fill=initial_fill, self_check=self_check)
        self.plan = ewp.Plan(self.gpu, max_tokens)
        self.ref = PagedLayer(self.host.array, fmt, E, k, H, I, K, initial_fill=initial_fill)
        self.dev = dev

    def close(self):
        self.plan.close()
        self.gpu.close()
        self.host.free()

    def check_plan(self, ids_ref, w_ref, p_ref, T):
        info = self.plan.info()
        assert info["num_tokens"] == T
        assert info["num_waves"] == p_ref.n_waves, (info, p_ref.n_waves)
        assert info["num_distinct"] == len(p_ref.distinct)
        assert info["num_hits"] == len(p_ref.hits)
        for w, wv in enumerate(p_ref.waves):
            ex, sl, misses = self.plan.wave(w)
            assert ex == wv.experts, (w, ex, wv.experts)
            assert sl == wv.slots, (w, sl, wv.slots)
            assert misses == wv.misses, (w, misses, wv.misses)
        ids, wts, sid, wof = self.plan.read()
        assert np.array_equal(ids, ids_ref), (ids, ids_ref)
        assert np.array_equal(sid, p_ref.slot_ids)
        assert np.array_equal(wof, p_ref.wave_of)
        if T:
            assert np.allclose(wts, w_ref, rtol=2e-6, atol=1e-7), (wts, w_ref)
        return info

    def check_state(self):
        se, es, st, clk = self.gpu.get_state()
        rse, res, rst, rclk = self.ref.table.state()
        assert np.array_equal(se, rse), (se, rse)
        assert np.array_equal(es, res)
        assert np.array_equal(st, rst), (st, rst)
        assert clk == rclk

    def run(self, logits, x, sample=lambda t: True, check_state_every=16, tol=None,
            on_step=None):
        """logits [steps][B][E] float32, x [steps][B][H] (f32 or bf16 bits).
        Returns the worst relative output error over the sampled steps."""
        tol = TOL[self.fmt] if tol is None else tol
        steps, B = logits.shape[0], logits.shape[1]
        lg_d = torch.from_numpy(np.ascontiguousarray(logits)).to(self.dev)
        xd = torch.from_numpy(np.ascontiguousarray(x.view(np.int16) if x.dtype == np.uint16 else x)).to(self.dev)
        out = torch.empty(B, self.H, dtype=torch.float32, device=self.dev)
        worst = 0.0
        for t in range(steps):
            comp = bool(sample(t))
            info = self.gpu.route(self.plan, lg_d[t])
            if on_step is not None:
                on_step(self, t, info)
            for w in range(info["num_waves"]):
                self.gpu.page_in(self.plan, w)
                self.gpu.forward(self.plan, w, xd[t], out)
            o_ref, ids_ref, w_ref, p_ref = self.ref.step(logits[t], x_values(x[t], self.fmt), compute=comp)
            self.check_plan(ids_ref, w_ref, p_ref, B)
            if comp:
                torch.cuda.synchronize()
                e = rel_err(out.cpu().numpy(), o_ref)
                worst = max(worst, e)
                assert e <= tol, (t, e, tol)
            if check_state_every and (t + 1) % check_state_every == 0:
                self.check_state()
        torch.cuda.synchronize()
        self.check_state()
        return worst
