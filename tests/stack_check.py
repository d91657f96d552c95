"""Layer-by-layer parity of a stack of paged MoE layers on the GPU.

A stack layer reads the residual stream through a unit-gain RMSNorm:
a_l = bf16_rne(rms_norm(x_l)), out_l = MoE_l(a_l), x_{l+1} = bf16_rne(x_l + out_l).
The GPU's a_l is checked against the oracle's norm of the GPU's own x_l (equal
up to one bf16 ulp where float32 and float64 straddle a rounding boundary, and
such flips rare). Each GPU layer's MoE output is checked against the oracle
layer stepped on the a_l that GPU layer actually received (so every layer is
held to the format's output tolerance on its own input, however deep it
sits), its plan and table state bit-exact, and the residual against the GPU's
own x_l and out_l (up to one bf16 ulp, rare).

End to end, the GPU hidden state is compared with an independent oracle chain
from x0 (norm included). Along the chain, every layer may contribute its
output tolerance and one bf16 flip of the hidden state it writes, so after
layer L the bound per element is sum over l <= L of
(tol * rms(out_l) + ulp(x_{l+1})). This assumes that a difference in a
layer's input moves its output by no more than itself (the norm divides by
rms(x) >= 1 here), which the measured ratios (printed) confirm.
"""
import numpy as np
import torch

import expert_weight_paging_amd as ewp
from oracle import formats
from oracle.expert import swiglu_expert
from oracle.layer import PagedLayer, bf16_rne, rms_norm
from oracle.router import route
from workloads import gen

from gpu_harness import TOL, rel_err, say, x_values


_POOLS, _MEMOS = {}, {}      # per workload: its record pool and decoded records, built once


def ulp_bf16(v):
    return np.exp2(np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** -126))) - 7)


def moe_unpaged(store, fmt, k, H, I, logits, x, memo):
    """The plain MoE layer from the store (no table), float64, decodes memoised
    by record bytes in `memo` (a dict shared with the oracle layers)."""
    dec = _Decoder(fmt, H, I, memo)
    ids, w = route(logits, k)
    out = np.zeros((x.shape[0], H))
    for e in np.unique(ids):
        rows, cols = np.nonzero(ids == e)
        g, u, d = dec(store[e])
        out[rows] += w[rows, cols][:, None] * swiglu_expert(g, u, d, x[rows])
    return out


class _Decoder(PagedLayer):
    """Only the oracle layer's memoised record decoder."""

    def __init__(self, fmt, H, I, memo):
        self.fmt, self.H, self.I, self.dtype, self.decode_cache = fmt, H, I, np.float64, memo

    def __call__(self, rec):
        return self._decode(rec)


class StackPair:
    """n GPU layers of a stack workload (layer l's store: pool record
    perm_l[e] for expert e) and their oracle twins stepped on the GPU's inputs.
    keep_refs=False creates each oracle layer when its GPU layer is checked
    and drops it afterwards (one step per layer, e.g. one prefill chunk)."""

    def __init__(self, cfg, n_layers, max_tokens, initial_fill, streams, keep_refs=True, dev="cuda"):
        self.cfg, self.n, self.initial_fill, self.keep_refs = cfg, n_layers, initial_fill, keep_refs
        self.streams = streams
        rec = ewp.record_bytes(cfg.fmt, cfg.H, cfg.I)
        if cfg.cid not in _POOLS:
            _POOLS[cfg.cid] = gen.pool_records(cfg)
        self.pool = _POOLS[cfg.cid]
        self.memo = _MEMOS.setdefault(cfg.cid, {})
        self.hosts, self.layers, self.plans, self.refs = [], [], [], []
        for l in range(n_layers):
            h = ewp.HostStore(cfg.E, rec)
            gen.fill_layer_store(cfg, l, h.array, self.pool)
            slots, state = ewp.alloc_layer_buffers(cfg.E, cfg.K, rec, dev)
            L = ewp.Layer(cfg.E, cfg.top_k, cfg.H, cfg.I, cfg.K, cfg.fmt, h, slots, state, *streams,
                          initial_fill=initial_fill)
            self.hosts.append(h)
            self.layers.append(L)
            self.plans.append(ewp.Plan(L, max_tokens))
            self.refs.append(self._ref(l) if keep_refs else None)

    def _ref(self, l):
        c = self.cfg
        return PagedLayer(self.hosts[l].array, c.fmt, c.E, c.top_k, c.H, c.I, c.K,
                          initial_fill=self.initial_fill, max_cached=16, decode_cache=self.memo)

    def reset(self):
        for L in self.layers:
            L.reset()

    def close(self):
        for p in self.plans:
            p.close()
        for L in self.layers:
            L.close()
        for h in self.hosts:
            h.free()

    def run_token(self, logits, x0, kind, chain=None):
        """One step (T tokens) through every layer, layer by layer, with the
        checks above. logits float32 [n][T][E]; x0 bf16 bits [T][H].
        kind: "device" (moe_step_device with the fused residual) or "host"
        (route, page-in and forward per wave, then the residual kernel).
        chain: None, or the token rows for which the independent oracle chain
        is computed (all rows: slice(None)). Returns (x_final bf16 tensor,
        last layer's out tensor, summary dict)."""
        c = self.cfg
        tol = TOL[c.fmt]
        T = x0.shape[0]
        x = torch.from_numpy(np.ascontiguousarray(x0).view(np.int16)).cuda()
        out = torch.empty(T, c.H, dtype=torch.float32, device="cuda")
        lg = torch.from_numpy(np.ascontiguousarray(logits)).cuda()
        worst_out, flips, n_res, nflips = 0.0, 0, 0, 0
        a = torch.empty_like(x)
        xo = x_values(x0, c.fmt)[chain] if chain is not None else None
        bound = 0.0
        for l in range(self.n):
            L, P = self.layers[l], self.plans[l]
            x_in = x_values(x.cpu().numpy().view(np.uint16), c.fmt)
            ewp.rmsnorm_bf16(x, a, stream=self.streams[0])
            if kind == "device":
                L.step_device(P, lg[l], a, out, x_res=x)
            else:
                info = L.route(P, lg[l])
                for w in range(info["num_waves"]):
                    L.page_in(P, w)
                    L.forward(P, w, a, out)
                ewp.residual_bf16(x, out, x, stream=self.streams[0])   # after the forward, same stream
            torch.cuda.synchronize()
            a_in = x_values(a.cpu().numpy().view(np.uint16), c.fmt)
            a_ref = bf16_rne(rms_norm(x_in))
            da = np.abs(a_in - a_ref)
            assert np.all(da <= ulp_bf16(a_ref)), l
            nflips += int((da > 0).sum())
            o_gpu = out.cpu().numpy().astype(np.float64)
            x_out = x_values(x.cpu().numpy().view(np.uint16), c.fmt)
            ref = self.refs[l] if self.keep_refs else self._ref(l)
            o_ref, ids_ref, _, p_ref = ref.step(logits[l], a_in)
            ids, _, sid, _ = P.read()
            assert np.array_equal(ids, ids_ref), l
            assert np.array_equal(sid, p_ref.slot_ids), l
            if kind == "host":
                info = P.info()
                assert info["num_waves"] == p_ref.n_waves, l
                for w, wv in enumerate(p_ref.waves):
                    assert P.wave(w) == (wv.experts, wv.slots, wv.misses), (l, w)
            se, es, st, clk = L.get_state()
            rse, res, rst, rclk = ref.table.state()
            assert np.array_equal(se, rse) and np.array_equal(es, res), l
            assert np.array_equal(st, rst) and clk == rclk, l
            e = rel_err(o_gpu, o_ref)
            worst_out = max(worst_out, e)
            assert e <= tol, (l, e, tol)
            # residual against the GPU's own input and output
            want = bf16_rne(x_in + o_gpu)
            d = np.abs(x_out - want)
            assert np.all(d <= ulp_bf16(want)), l
            flips += int((d > 0).sum())
            n_res += d.size
            if not self.keep_refs:
                del ref
            if chain is not None:
                oc = moe_unpaged(self.hosts[l].array, c.fmt, c.top_k, c.H, c.I, logits[l][chain],
                                 bf16_rne(rms_norm(xo)), self.memo)
                xo = bf16_rne(xo + oc)
                bound = bound + tol * np.sqrt(np.mean(oc ** 2)) + ulp_bf16(xo)
        summary = {"worst_layer_out": worst_out, "residual_flip_frac": flips / max(n_res, 1),
                   "norm_flip_frac": nflips / max(n_res, 1)}
        assert summary["residual_flip_frac"] < 1e-2 and summary["norm_flip_frac"] < 1e-2
        if chain is not None:
            got = x_values(x.cpu().numpy().view(np.uint16), c.fmt)[chain]
            ratio = float((np.abs(got - xo) / bound).max())
            summary["drift_over_bound"] = ratio
            summary["drift_max_abs"] = float(np.abs(got - xo).max())
            assert ratio <= 1.0, summary
        return x, out, summary
