"""Python binding of libmoepage (Paged Experts hot path on MI355X).

Argument marshalling only: every step of the path (routing, slot planning,
page-in, expert math) runs in the HIP library. PyTorch provides device memory
and streams. There is no CPU fallback: if the library is not built, every
call raises.

Names follow the C ABI in include/moepage.h.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoepage.so")

FMT_F32, FMT_BF16, FMT_FP8, FMT_INT4, FMT_MXFP4 = 0, 1, 2, 3, 4
MAX_GEMV_TOKENS = 64
TIMERS = ("route", "ffn_up", "ffn_down", "gemm_up", "gemm_down", "combine", "page_in")

_STATUS = {0: "MOE_OK", -1: "MOE_ERR_INVALID_ARG", -2: "MOE_ERR_NOT_PINNED", -3: "MOE_ERR_FORMAT",
           -4: "MOE_ERR_HIP", -5: "MOE_ERR_SELFCHECK", -6: "MOE_ERR_STATE", -7: "MOE_ERR_TIMEOUT"}


class MoeError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__("%s: %s" % (_STATUS.get(status, status), msg))
        self.status = status
        self.name = _STATUS.get(status, str(status))


class _Desc(ctypes.Structure):
    _fields_ = [("num_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("hidden", ctypes.c_int32), ("intermediate", ctypes.c_int32),
                ("num_slots", ctypes.c_int32), ("format", ctypes.c_int32),
                ("record_bytes", ctypes.c_size_t), ("host_store", ctypes.c_void_p),
                ("slot_store", ctypes.c_void_p), ("state", ctypes.c_void_p),
                ("initial_fill", ctypes.c_int32), ("self_check", ctypes.c_int32)]


class _PlanInfo(ctypes.Structure):
    _fields_ = [("num_tokens", ctypes.c_int32), ("num_distinct", ctypes.c_int32),
                ("num_hits", ctypes.c_int32), ("num_misses", ctypes.c_int32),
                ("num_waves", ctypes.c_int32)]


class _WaveInfo(ctypes.Structure):
    _fields_ = [("num_experts", ctypes.c_int32), ("num_misses", ctypes.c_int32),
                ("experts", ctypes.POINTER(ctypes.c_int32)), ("slots", ctypes.POINTER(ctypes.c_int32)),
                ("miss_experts", ctypes.POINTER(ctypes.c_int32)),
                ("miss_slots", ctypes.POINTER(ctypes.c_int32))]


class _Stats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in
                ("steps", "refs", "activations", "hits", "misses", "waves", "bytes_paged")]


class _Timing(ctypes.Structure):
    _fields_ = [("count", ctypes.c_int64 * 7), ("ms", ctypes.c_double * 7),
                ("bytes", ctypes.c_double * 7), ("flops", ctypes.c_double * 7)]


EXPORTS = {
    "moe_record_bytes": (ctypes.c_size_t, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]),
    "moe_state_bytes": (ctypes.c_size_t, [ctypes.c_int32, ctypes.c_int32]),
    "moe_layer_init": (ctypes.c_int, [ctypes.POINTER(_Desc), ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.POINTER(ctypes.c_void_p)]),
    "moe_layer_reset": (ctypes.c_int, [ctypes.c_void_p]),
    "moe_layer_destroy": (None, [ctypes.c_void_p]),
    "moe_plan_create": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(ctypes.c_void_p)]),
    "moe_plan_destroy": (None, [ctypes.c_void_p]),
    "moe_route": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]),
    "moe_plan_get_info": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(_PlanInfo)]),
    "moe_plan_get_wave": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(_WaveInfo)]),
    "moe_plan_read": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_void_p]),
    "moe_page_in": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32]),
    "moe_forward": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                   ctypes.c_void_p, ctypes.c_void_p]),
    "moe_rmsnorm_bf16": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_void_p]),
    "moe_residual_bf16": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_int64, ctypes.c_void_p]),
    "moe_stack_forward": (ctypes.c_int, [ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(ctypes.c_void_p),
                                         ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32]),
    "moe_layer_stats": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(_Stats)]),
    "moe_layer_get_state": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_void_p]),
    "moe_timing_enable": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32]),
    "moe_timing_read": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(_Timing)]),
    "moe_timing_floor": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(ctypes.c_double)]),
    "moe_slots_for_budget": (ctypes.c_int32, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                              ctypes.c_int32, ctypes.c_int64]),
    "moe_preflight": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_double,
                                     ctypes.c_int32, ctypes.c_double, ctypes.c_double, ctypes.c_double,
                                     ctypes.c_void_p]),
    "moe_step_device": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "moe_step_device_static": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                              ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "moe_step_token_waves": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "moe_stack_forward_device": (ctypes.c_int, [ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(ctypes.c_void_p),
                                                ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32,
                                                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32]),
    "moe_read_probe": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_size_t,
                                      ctypes.c_int32, ctypes.POINTER(ctypes.c_double)]),
    "moe_host_alloc": (ctypes.c_void_p, [ctypes.c_size_t]),
    "moe_host_free": (None, [ctypes.c_void_p]),
    "moe_last_error": (ctypes.c_char_p, []),
}

_lib = None


def lib():
    """The loaded library; raises if it has not been built (no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libmoepage.so is not built (run __graft_entry__.build() or "
                              "python -m expert_weight_paging_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(status):
    if status != 0:
        raise MoeError(status, lib().moe_last_error().decode(errors="replace"))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(s):
    if s is None:
        return None
    return ctypes.c_void_p(s.cuda_stream)


def record_bytes(fmt, hidden, intermediate):
    return int(lib().moe_record_bytes(fmt, hidden, intermediate))


def state_bytes(num_experts, num_slots):
    return int(lib().moe_state_bytes(num_experts, num_slots))


class HostStore:
    """Page-locked host buffer [E][record_bytes] (hipHostMalloc) with a numpy view."""

    def __init__(self, num_experts, rec_bytes):
        n = int(num_experts) * int(rec_bytes)
        p = lib().moe_host_alloc(n)
        if not p:
            raise MoeError(-4, lib().moe_last_error().decode())
        self.ptr, self.nbytes = p, n
        buf = (ctypes.c_uint8 * n).from_address(p)
        self.array = np.frombuffer(buf, dtype=np.uint8).reshape(num_experts, rec_bytes)

    def free(self):
        if self.ptr:
            self.array = None
            lib().moe_host_free(self.ptr)
            self.ptr = None

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


class Plan:
    def __init__(self, layer, max_tokens):
        h = ctypes.c_void_p()
        _check(lib().moe_plan_create(layer.handle, int(max_tokens), ctypes.byref(h)))
        self.handle, self.layer, self.max_tokens = h, layer, int(max_tokens)
        self.dev_tokens = None  # token count of the last device-resolved step, if that was the last routing

    def close(self):
        if self.handle:
            lib().moe_plan_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def info(self):
        i = _PlanInfo()
        _check(lib().moe_plan_get_info(self.handle, ctypes.byref(i)))
        return {f: getattr(i, f) for f, _ in _PlanInfo._fields_}

    def wave(self, w):
        wi = _WaveInfo()
        _check(lib().moe_plan_get_wave(self.handle, int(w), ctypes.byref(wi)))
        n, m = wi.num_experts, wi.num_misses
        ex = [wi.experts[i] for i in range(n)]
        sl = [wi.slots[i] for i in range(n)]
        misses = [(wi.miss_experts[i], wi.miss_slots[i]) for i in range(m)]
        return ex, sl, misses

    def read(self):
        # after a device-resolved step the host view is stale: use its token count
        T = self.dev_tokens if self.dev_tokens is not None else self.info()["num_tokens"]
        n = T * self.layer.top_k
        ids = np.zeros(n, np.int32)
        w = np.zeros(n, np.float32)
        sid = np.zeros(n, np.int32)
        wo = np.zeros(n, np.int32)
        _check(lib().moe_plan_read(self.handle, ids.ctypes.data_as(ctypes.c_void_p),
                                   w.ctypes.data_as(ctypes.c_void_p),
                                   sid.ctypes.data_as(ctypes.c_void_p),
                                   wo.ctypes.data_as(ctypes.c_void_p)))
        shp = (T, self.layer.top_k)
        return ids.reshape(shp), w.reshape(shp), sid.reshape(shp), wo.reshape(shp)


class Layer:
    """One paged MoE layer. slot_store and state are torch CUDA uint8 tensors."""

    def __init__(self, num_experts, top_k, hidden, intermediate, num_slots, fmt, host_store,
                 slot_store, state, compute_stream=None, copy_stream=None, route_stream=None,
                 initial_fill=False, self_check=False):
        rb = record_bytes(fmt, hidden, intermediate)
        d = _Desc(num_experts, top_k, hidden, intermediate, num_slots, fmt, rb,
                  ctypes.c_void_p(host_store.ptr if isinstance(host_store, HostStore) else host_store),
                  _ptr(slot_store), _ptr(state), int(bool(initial_fill)), int(bool(self_check)))
        h = ctypes.c_void_p()
        _check(lib().moe_layer_init(ctypes.byref(d), _stream(compute_stream), _stream(copy_stream),
                                    _stream(route_stream), ctypes.byref(h)))
        self.handle = h
        self.E, self.top_k, self.H, self.I, self.K, self.fmt = (num_experts, top_k, hidden,
                                                                intermediate, num_slots, fmt)
        self.record_bytes = rb
        self._keep = (host_store, slot_store, state)

    def close(self):
        if self.handle:
            lib().moe_layer_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def route(self, plan, logits, num_tokens=None):
        T = logits.shape[0] if num_tokens is None else num_tokens
        _check(lib().moe_route(self.handle, _ptr(logits), int(T), plan.handle))
        plan.dev_tokens = None
        return plan.info()

    def page_in(self, plan, wave):
        _check(lib().moe_page_in(self.handle, plan.handle, int(wave)))

    def forward(self, plan, wave, x, out):
        _check(lib().moe_forward(self.handle, plan.handle, int(wave), _ptr(x), _ptr(out)))

    def step(self, plan, logits, x, out):
        """route, then page_in + forward for every wave; returns the plan info."""
        info = self.route(plan, logits)
        for w in range(info["num_waves"]):
            self.page_in(plan, w)
            self.forward(plan, w, x, out)
        return info

    def step_device(self, plan, logits, x, out, x_res=None, num_tokens=None):
        """Device-resolved single-wave step (no host synchronisation; capturable
        in a HIP graph): route, page-in by a copy kernel and expert FFN on the
        compute stream. Requires num_tokens * top_k <= K."""
        T = logits.shape[0] if num_tokens is None else num_tokens
        _check(lib().moe_step_device(self.handle, plan.handle, _ptr(logits), int(T), _ptr(x), _ptr(out),
                                     _ptr(x_res)))
        plan.dev_tokens = int(T)

    def step_device_static(self, logits, x, out, x_res=None, num_tokens=None):
        """moe_step_device without a plan: the step's workspace is the
        library's fixed device array (allocates nothing; calls that overlap
        on one GPU race)."""
        T = logits.shape[0] if num_tokens is None else num_tokens
        _check(lib().moe_step_device_static(self.handle, _ptr(logits), int(T), _ptr(x), _ptr(out),
                                            _ptr(x_res)))

    def group_tokens(self, plan):
        """Tokens per group of step_token_waves: min(K // top_k, max_tokens, 64)."""
        return min(self.K // self.top_k, plan.max_tokens, 64)

    def step_token_waves(self, plan, logits, x, out, x_res=None, num_tokens=None):
        """Token-partitioned waves: groups of group_tokens(plan) consecutive
        tokens, each one device-resolved single-wave step, no host sync."""
        T = logits.shape[0] if num_tokens is None else num_tokens
        _check(lib().moe_step_token_waves(self.handle, plan.handle, _ptr(logits), int(T), _ptr(x), _ptr(out),
                                          _ptr(x_res)))
        G = self.group_tokens(plan)
        plan.dev_tokens = int(T) - (int(T) - 1) // G * G  # the last group's size

    def reset(self):
        _check(lib().moe_layer_reset(self.handle))

    def stats(self):
        s = _Stats()
        _check(lib().moe_layer_stats(self.handle, ctypes.byref(s)))
        return {f: getattr(s, f) for f, _ in _Stats._fields_}

    def get_state(self):
        se = np.zeros(self.K, np.int32)
        es = np.zeros(self.E, np.int32)
        st = np.zeros(self.K, np.int64)
        clk = np.zeros(1, np.int64)
        _check(lib().moe_layer_get_state(self.handle, se.ctypes.data_as(ctypes.c_void_p),
                                         es.ctypes.data_as(ctypes.c_void_p),
                                         st.ctypes.data_as(ctypes.c_void_p),
                                         clk.ctypes.data_as(ctypes.c_void_p)))
        return se, es, st, int(clk[0])

    def timing_enable(self, on=True):
        _check(lib().moe_timing_enable(self.handle, int(bool(on))))

    def timing_read(self):
        t = _Timing()
        _check(lib().moe_timing_read(self.handle, ctypes.byref(t)))
        return {name: {"count": t.count[i], "ms": t.ms[i], "bytes": t.bytes[i], "flops": t.flops[i]}
                for i, name in enumerate(TIMERS)}


class _Preflight(ctypes.Structure):
    _fields_ = [("slot_mb", ctypes.c_double), ("kv_tokens_per_slot", ctypes.c_double),
                ("batch_cap", ctypes.c_int32), ("all_miss_gb_per_token", ctypes.c_double),
                ("max_miss", ctypes.c_double), ("random_miss", ctypes.c_double),
                ("reuse_implied", ctypes.c_int32)]


def slots_for_budget(fmt, hidden, intermediate, num_experts, layers, budget_bytes):
    """Slots per layer that a device-memory budget holds (same K in every layer)."""
    k = lib().moe_slots_for_budget(int(fmt), int(hidden), int(intermediate), int(num_experts), int(layers),
                                   int(budget_bytes))
    if k < 0:
        _check(k)
    return k


def preflight(layers, experts, top_k, expert_mb, num_slots, link_gbps, tok_s, kv_bytes_per_token):
    """The preflight numbers of the scheme: slot cost, KV tokens per slot, batch
    cap, all-miss bytes per token, highest allowed and no-reuse miss rates."""
    r = _Preflight()
    _check(lib().moe_preflight(int(layers), int(experts), int(top_k), float(expert_mb), int(num_slots),
                               float(link_gbps), float(tok_s), float(kv_bytes_per_token),
                               ctypes.byref(r)))
    d = {f: getattr(r, f) for f, _ in _Preflight._fields_}
    d["reuse_implied"] = bool(d["reuse_implied"])
    return d


def timing_floor(stream=None, reps=100):
    """Microseconds the layer timers report for an empty kernel on `stream`:
    the per-launch floor included in every timing_read figure."""
    us = ctypes.c_double()
    _check(lib().moe_timing_floor(_stream(stream), int(reps), ctypes.byref(us)))
    return us.value


def read_probe(buf, nbytes, stream=None, reps=40):
    """Median microseconds of one launch that plainly streams `nbytes` bytes of
    the device buffer `buf` (a torch uint8 tensor), each launch reading a part
    the previous ones did not: the reference for the FFN launches' times."""
    us = ctypes.c_double()
    _check(lib().moe_read_probe(_stream(stream), _ptr(buf), buf.numel(), int(nbytes), int(reps),
                                ctypes.byref(us)))
    return us.value


def rmsnorm_bf16(x, a, stream=None):
    """a = bf16_rne(x / sqrt(mean(x^2) + 1e-6)) per row (x, a bf16 [T][H], may alias): the
    input of every layer of a stack."""
    T, H = x.shape
    _check(lib().moe_rmsnorm_bf16(_ptr(x), _ptr(a), int(T), int(H), _stream(stream)))


def residual_bf16(x_in, out, x_out, stream=None):
    """x_out = bf16_rne(x_in + out) on the device (x bf16, out float32)."""
    _check(lib().moe_residual_bf16(_ptr(x_in), _ptr(out), _ptr(x_out), int(out.numel()),
                                   _stream(stream)))


def stack_forward(layers, plans, logits, x, out, lookahead=False):
    """One batch through a stack of layers: out = MoE_l(x); x = bf16_rne(x + out).

    logits: device float32 [L][T][E]; x: device bf16 (int16 view) [T][H], in
    place; out: device float32 [T][H] scratch."""
    n = len(layers)
    la = (ctypes.c_void_p * n)(*[l.handle.value for l in layers])
    pa = (ctypes.c_void_p * n)(*[p.handle.value for p in plans])
    _check(lib().moe_stack_forward(la, pa, n, _ptr(logits), int(logits.shape[1]), _ptr(x), _ptr(out),
                                   int(bool(lookahead))))
    for p in plans:
        p.dev_tokens = None


def stack_forward_device(layers, plans, logits, x, out, lookahead=False):
    """stack_forward through device-resolved steps: every layer's route,
    page-in and FFN enqueued with no host wait (lookahead: routes and copies
    on the shared copy stream, FFNs on the compute stream)."""
    n = len(layers)
    la = (ctypes.c_void_p * n)(*[l.handle.value for l in layers])
    pa = (ctypes.c_void_p * n)(*[p.handle.value for p in plans])
    _check(lib().moe_stack_forward_device(la, pa, n, _ptr(logits), int(logits.shape[1]), _ptr(x),
                                          _ptr(out), int(bool(lookahead))))
    for p in plans:
        p.dev_tokens = int(logits.shape[1])


def alloc_layer_buffers(num_experts, num_slots, rec_bytes, device="cuda"):
    """Slot store [K][rec] and state buffer as torch uint8 device tensors."""
    import torch
    slots = torch.empty(num_slots * rec_bytes, dtype=torch.uint8, device=device)
    state = torch.empty(state_bytes(num_experts, num_slots), dtype=torch.uint8, device=device)
    return slots, state
