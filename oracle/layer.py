"""One paged MoE layer and a stack of them, float64.

[PE] "What does Paged Experts actually do?": per step, the routed experts that
are missing are copied from the pinned host store into slots (least recently
used out), then the MoE math runs over the slots. [PE] "Can paging change the
model's outputs?": the paged layer must return what the unpaged layer returns,
and a paged-in expert must never run with another expert's bytes.

The oracle therefore keeps a CPU copy of the slot store, copies whole records
into it exactly as the planner says, and computes every expert FROM ITS SLOT,
so that a planner or copy mistake shows up in the output. ``unpaged_forward``
computes from the store directly; the two agree bitwise.

Stack reading (attention omitted): every layer reads the residual stream
through a unit-gain RMSNorm, as the MoE block of the model the pages run
(Qwen3-30B-A3B, [PE] "What does Paged Experts actually do?") does, and adds
its output back: a = bf16_rne(rms_norm(x)), x_next = bf16_rne(x + moe(a)).
Without the norm the SwiGLU experts make the hidden state grow about
quadratically per layer, past every 16- and 32-bit range within 48 layers.
"""
import numpy as np
import xxhash

from . import formats
from .expert import swiglu_expert
from .lru import SlotTable
from .router import route


def bf16_rne(v):
    """float64 -> nearest bfloat16 value (ties to even), returned as float64.

    With v = m * 2^e, 0.5 <= |m| < 1, a bfloat16 keeps 8 significant bits, so
    the result is rint(m * 2^8) * 2^(e-8) with rint rounding half to even.
    Normal-range inputs only (the hidden states here are O(1)).
    """
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)


RMS_EPS = 1e-6


def rms_norm(x, eps=RMS_EPS):
    """Unit-gain RMSNorm over the last axis, float64: x / sqrt(mean(x^2) + eps)."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def bf16_bits(v):
    """float64 values that are exact bf16 -> uint16 bit patterns."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


class PagedLayer:
    """host_store: uint8 [E][stride]. Keeps its own CPU slot store [K][stride].

    dtype: float64 (parity) or float32 (the same steps in single precision,
    the variant timed as the CPU baseline; routing and the plan are the same).
    """

    def __init__(self, host_store, fmt, E, top_k, H, I, K, initial_fill=False, max_cached=48,
                 dtype=np.float64, decode_cache=None):
        self.dtype = dtype
        # optional dict shared by several layers: decoded weights keyed by a
        # 128-bit hash of the record bytes (decoding is a function of those
        # bytes alone), so a record that several layers hold is decoded once
        self.decode_cache = decode_cache
        self.store = np.asarray(host_store, dtype=np.uint8)
        self.max_cached = max_cached
        self.fmt, self.E, self.top_k, self.H, self.I, self.K = fmt, E, top_k, H, I, K
        self.stride = formats.record_stride(fmt, H, I)
        assert self.store.shape == (E, self.stride)
        self.table = SlotTable(E, K, initial_fill)
        self.slots = np.zeros((K, self.stride), dtype=np.uint8)
        self._cache = {}
        self.reset()

    def reset(self):
        self.table.reset()
        self.slots[:] = 0
        if self.table.initial_fill:
            self.slots[:] = self.store[:self.K]
        self._cache = {}

    def _page_in(self, e, s):
        self.slots[s] = self.store[e]
        self._cache.pop(s, None)

    def _decode(self, rec):
        """Weights (gate, up, down) of one record's bytes, in the layer's dtype;
        through the shared memo when there is one."""
        key = None
        if self.decode_cache is not None:
            key = (xxhash.xxh3_128_digest(rec), np.dtype(self.dtype).str, self.fmt, self.H, self.I)
            if key in self.decode_cache:
                return self.decode_cache[key]
        w = tuple(np.asarray(m, dtype=self.dtype) for m in formats.decode_record(rec, self.fmt, self.H, self.I))
        if key is not None:
            self.decode_cache[key] = w
        return w

    def _slot_weights(self, s):
        # decoded from the slot's bytes; invalidated on every page-in into s
        if s not in self._cache:
            if len(self._cache) >= self.max_cached:
                self._cache.pop(next(iter(self._cache)))
            self._cache[s] = self._decode(self.slots[s])
        return self._cache[s]

    def step(self, logits, x, compute=True):
        """logits float32 [B,E], x [B,H] (values) -> (out float64 [B,H], ids, w, plan).

        Per wave, the wave's experts are taken in wave order; each one is
        decoded from ITS SLOT and applied to all tokens routed to it in this
        wave, out[t] += w_tj * y. compute=False plans and pages in exactly the
        same way but skips the expert math (out is None), for long sequences
        checked on samples.
        """
        ids, w = route(logits, self.top_k)
        plan = self.table.plan(ids, on_page_in=None)
        # replay the page-ins in wave order: a later wave may reuse a slot that
        # an earlier wave of the same step computed from
        x = np.asarray(x, dtype=self.dtype)
        out = np.zeros((x.shape[0], self.H), dtype=self.dtype) if compute else None
        for wave in plan.waves:
            for e, s in wave.misses:
                self._page_in(e, s)
            if compute:
                for e, s in zip(wave.experts, wave.slots):
                    self._apply(self._slot_weights(s), e, ids, w, x, out)
        return out, ids, w, plan

    def step_token_waves(self, logits, x, group, compute=True):
        """Token-partitioned waves. [PE] "What happens with more than one
        request?": a decode step is one wave when tokens x top_k <= K, so up to
        K // top_k tokens always fit one; a larger batch is served here as
        consecutive groups of `group` (<= K // top_k) tokens in token order,
        each group a step of its own (own routing of its rows, own LRU tick,
        own page-ins). Returns (out [B,H] or None, ids [B,k], w [B,k],
        list of the groups' plans)."""
        if not 1 <= group <= self.K // self.top_k:
            raise ValueError("group must be in 1..K // top_k")
        B = np.asarray(logits).shape[0]
        outs, ids, ws, plans = [], [], [], []
        for t0 in range(0, B, group):
            o, i, w, p = self.step(logits[t0:t0 + group], x[t0:t0 + group], compute)
            outs.append(o)
            ids.append(i)
            ws.append(w)
            plans.append(p)
        out = np.concatenate(outs) if compute else None
        return out, np.concatenate(ids), np.concatenate(ws), plans

    @staticmethod
    def _apply(weights, e, ids, w, x, out):
        """out[t] += w_tj * expert_e(x_t) for every (t, j) routed to expert e."""
        rows, cols = np.nonzero(ids == e)          # each token routes to e at most once
        if rows.size == 0:
            return
        wg, wu, wd = weights
        y = swiglu_expert(wg, wu, wd, x[rows], dtype=out.dtype)
        out[rows] += w[rows, cols][:, None].astype(out.dtype) * y

    def unpaged_forward(self, logits, x):
        """The same layer computed straight from the host store (no slots),
        in the same order as step(); the wave of each expert only depends on
        the table, so it is taken from a dry run of the planner."""
        ids, w = route(logits, self.top_k)
        x = np.asarray(x, dtype=np.float64)
        out = np.zeros((x.shape[0], self.H), dtype=np.float64)
        dry = SlotTable(self.E, self.K, self.table.initial_fill)
        dry.slot_expert, dry.expert_slot = self.table.slot_expert.copy(), self.table.expert_slot.copy()
        dry.stamp, dry.clock = self.table.stamp.copy(), self.table.clock
        plan = dry.plan(ids)
        for wave in plan.waves:
            for e in wave.experts:
                self._apply(self._decode(self.store[e]), e, ids, w, x, out)
        return out


def run_stack(layers, logits_per_layer, x0):
    """Stack of paged layers: a_l = bf16_rne(rms_norm(x_l)),
    x_{l+1} = bf16_rne(x_l + out_l) with out_l the layer's MoE output on a_l.

    logits_per_layer: list of float32 [B,E]; x0: values [B,H] (bf16-exact).
    Returns (x_final, per-layer outputs, per-layer plans).
    """
    x = np.asarray(x0, dtype=np.float64)
    outs, plans = [], []
    for layer, logits in zip(layers, logits_per_layer):
        out, _, _, plan = layer.step(logits, bf16_rne(rms_norm(x)))
        outs.append(out)
        plans.append(plan)
        x = bf16_rne(x + out)
    return x, outs, plans
