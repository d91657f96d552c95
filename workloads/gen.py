"""Seeded generators (see the package docstring for the workloads)."""
from dataclasses import dataclass, field

import numpy as np

F32, BF16, FP8, INT4, MXFP4 = 0, 1, 2, 3, 4
ROUTE_SHIFT = np.float32(16.0)


@dataclass(frozen=True)
class Config:
    cid: int
    name: str
    fmt: int
    E: int
    top_k: int
    H: int
    I: int
    K: int
    layers: int
    steps: int
    batches: tuple
    routing: str            # "normal" | "correlated" | "uniform"
    p_keep: float
    sigma: float
    initial_fill: bool
    tokens: int = 1         # prefill chunk length (config 5)
    extra: dict = field(default_factory=dict)

    @property
    def seed(self):
        return 1000 + self.cid


CONFIGS = {
    1: Config(1, "tiny-f32", F32, 8, 2, 64, 32, 4, 1, 16, (1,), "normal", 0.0, 0.05, False),
    2: Config(2, "layer-bf16", BF16, 128, 8, 2048, 768, 40, 1, 256, (1,), "correlated", 0.75, 0.02, False),
    3: Config(3, "layer-fp8", FP8, 128, 8, 2048, 768, 40, 1, 256, (1, 2, 4, 5, 6, 8), "correlated", 0.75, 0.02, False),
    4: Config(4, "stack48-int4", INT4, 128, 8, 2048, 768, 92, 48, 256, (1,), "correlated", 0.75, 0.02, False),
    5: Config(5, "prefill48-bf16", BF16, 128, 8, 2048, 768, 92, 48, 1, (2048,), "uniform", 0.0, 0.02, True, tokens=2048),
    # the next format row: the bf16 layer's shape and routing with MXFP4 experts
    6: Config(6, "layer-mxfp4", MXFP4, 128, 8, 2048, 768, 40, 1, 256, (1,), "correlated", 0.75, 0.02, False),
}


def streams(cid, *salt):
    """Independent generators for one workload: logits/routing, weights, hidden, layers."""
    base = [1000 + int(cid)] + [int(s) for s in salt]
    names = ("routing", "weights", "hidden", "layers")
    return {n: np.random.Generator(np.random.PCG64(np.random.SeedSequence(base + [i])))
            for i, n in enumerate(names)}


# ------------------------------------------------------------ normal draws

_TABLES = {}


def normal_table_f32(sigma):
    """65536 quantiles of N(0, sigma^2) at the midpoints (i + 0.5) / 65536."""
    key = ("f32", float(sigma))
    if key not in _TABLES:
        from scipy.special import ndtri
        u = (np.arange(65536, dtype=np.float64) + 0.5) / 65536.0
        _TABLES[key] = (sigma * ndtri(u)).astype(np.float32)
    return _TABLES[key]


def f32_to_bf16_bits(x):
    """float32 -> bfloat16 bit patterns, round to nearest even (finite inputs)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(u):
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_table_bf16(sigma):
    key = ("bf16", float(sigma))
    if key not in _TABLES:
        _TABLES[key] = f32_to_bf16_bits(normal_table_f32(sigma))
    return _TABLES[key]


def draw_normal_f32(rng, n, sigma):
    idx = rng.integers(0, 65536, size=n, dtype=np.uint16)
    return normal_table_f32(sigma)[idx]


def draw_normal_bf16(rng, n, sigma):
    idx = rng.integers(0, 65536, size=n, dtype=np.uint16)
    return _normal_table_bf16(sigma)[idx]


# ------------------------------------------------------------ record encoding

def _payload(fmt, H, I):
    if fmt == F32:
        return 3 * H * I * 4
    if fmt == BF16:
        return 3 * H * I * 2
    if fmt == FP8:
        return 3 * H * I + 4 * ((2 * I // 128) * (H // 128) + (H // 128) * (I // 128))
    if fmt == INT4:
        return 3 * H * I // 2 + 2 * 2 * (2 * I * (H // 128) + H * (I // 128))
    if fmt == MXFP4:
        return 3 * H * I // 2 + (2 * I * (H // 32) + H * (I // 32))
    raise ValueError(fmt)


def record_stride(fmt, H, I):
    return (_payload(fmt, H, I) + 255) // 256 * 256


def _fp8_tiles(w):
    """w float32 [R][C] -> (codes uint8 [R][C], scales float32 [R/128][C/128])."""
    import torch
    R, C = w.shape
    t = w.reshape(R // 128, 128, C // 128, 128)
    amax = np.abs(t).max(axis=(1, 3)).astype(np.float32)
    s = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    q = (t / s[:, None, :, None]).astype(np.float32)
    q = np.clip(q, -448.0, 448.0).reshape(R, C)
    codes = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, s


def _int4_groups(w):
    """w float32 [R][C] -> (words uint32 [R][C/8], scales f16 [R][C/128], zeros f16 [R][C/128])."""
    R, C = w.shape
    g = w.reshape(R, C // 128, 128)
    lo, hi = g.min(axis=2), g.max(axis=2)
    s = np.where(hi > lo, (hi - lo) / np.float32(15.0), np.float32(1.0)).astype(np.float16)
    s32 = s.astype(np.float32)
    z = (-lo / s32).astype(np.float16)
    q = np.rint(g / s32[:, :, None] + z.astype(np.float32)[:, :, None])
    q = np.clip(q, 0, 15).astype(np.uint32).reshape(R, C // 8, 8)
    words = np.zeros((R, C // 8), dtype=np.uint32)
    for n in range(8):
        words |= q[:, :, n] << np.uint32(4 * n)
    return words, s, z


# magnitudes of the E2M1 codes 0..7 and the midpoints between neighbours
_E2M1_MID = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float32)


def _mxfp4_blocks(w):
    """w float32 [R][C] -> (code bytes uint8 [R][C/2], scale bytes uint8 [R][C/32]).

    Per block of 32 along a row: shared exponent floor(log2(amax)) - 2 (the
    largest E2M1 magnitude is 6 = 1.5 * 2^2), scale byte exponent + 127;
    each weight is rounded to the nearest E2M1 magnitude (saturating at 6)."""
    R, C = w.shape
    g = w.reshape(R, C // 32, 32).astype(np.float32)
    amax = np.abs(g).max(axis=2)
    e = np.where(amax > 0, np.floor(np.log2(np.maximum(amax, np.float32(1e-38)))) - 2, -127)
    e = np.clip(e, -127, 127).astype(np.int32)
    scaled = g / np.exp2(e.astype(np.float32))[:, :, None]
    idx = np.searchsorted(_E2M1_MID, np.abs(scaled)).astype(np.uint8)   # 0..7
    code = (idx | ((scaled < 0) & (idx > 0)).astype(np.uint8) << 3).reshape(R, C)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    return packed, (e + 127).astype(np.uint8)


def encode_record(fmt, w13, wd):
    """Pack one expert: w13 [2I][H] (gate rows then up rows), wd [H][I] -> uint8 [stride].

    For F32 the arrays are float32 values; for BF16 they may be float32 (rounded
    here) or uint16 bit patterns; FP8 and INT4 quantise float32 values.
    """
    R13, H = w13.shape
    I = R13 // 2
    parts = []
    if fmt == F32:
        parts = [np.asarray(w13, np.float32), np.asarray(wd, np.float32)]
    elif fmt == BF16:
        conv = (lambda a: a if a.dtype == np.uint16 else f32_to_bf16_bits(a))
        parts = [conv(np.asarray(w13)), conv(np.asarray(wd))]
    elif fmt == FP8:
        q13, s13 = _fp8_tiles(np.asarray(w13, np.float32))
        qd, sd = _fp8_tiles(np.asarray(wd, np.float32))
        parts = [q13, qd, s13, sd]
    elif fmt == INT4:
        p13, s13, z13 = _int4_groups(np.asarray(w13, np.float32))
        pd, sd, zd = _int4_groups(np.asarray(wd, np.float32))
        parts = [p13, pd, s13, sd, z13, zd]
    elif fmt == MXFP4:
        p13, s13 = _mxfp4_blocks(np.asarray(w13, np.float32))
        pd, sd = _mxfp4_blocks(np.asarray(wd, np.float32))
        parts = [p13, pd, s13, sd]
    else:
        raise ValueError(fmt)
    raw = np.concatenate([np.ascontiguousarray(p).view(np.uint8).ravel() for p in parts])
    rec = np.zeros(record_stride(fmt, H, I), dtype=np.uint8)
    rec[:raw.size] = raw
    return rec


def _expert_rng(cfg, e):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg.seed, 77, int(e)])))


def expert_record(cfg, e):
    """Record of pool expert e of a workload (uint8 [stride])."""
    rng = _expert_rng(cfg, e)
    H, I = cfg.H, cfg.I
    if cfg.fmt == BF16:
        w13 = draw_normal_bf16(rng, 2 * I * H, cfg.sigma).reshape(2 * I, H)
        wd = draw_normal_bf16(rng, H * I, cfg.sigma).reshape(H, I)
    elif cfg.fmt == F32:
        w13 = (rng.standard_normal((2 * I, H)) * cfg.sigma).astype(np.float32)
        wd = (rng.standard_normal((H, I)) * cfg.sigma).astype(np.float32)
    else:
        w13 = draw_normal_f32(rng, 2 * I * H, cfg.sigma).reshape(2 * I, H)
        wd = draw_normal_f32(rng, H * I, cfg.sigma).reshape(H, I)
    return encode_record(cfg.fmt, w13, wd)


def expert_store(cfg, out=None, layer=None):
    """Fill (or return) a host store [E][stride] for one layer.

    layer=None or 0 with a one-layer workload: records in pool order. For a
    stack, layer l uses pool record perm_l[e] for expert e.
    """
    stride = record_stride(cfg.fmt, cfg.H, cfg.I)
    if out is None:
        out = np.zeros((cfg.E, stride), dtype=np.uint8)
    perm = np.arange(cfg.E) if (layer is None or cfg.layers == 1) else layer_permutation(cfg, layer)
    for e in range(cfg.E):
        out[e] = expert_record(cfg, perm[e])
    return out


def layer_permutation(cfg, layer):
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg.seed, 88, int(layer)])))
    return rng.permutation(cfg.E)


def pool_records(cfg):
    """All E pool records of a workload, uint8 [E][stride]."""
    return expert_store(cfg)


def fill_layer_store(cfg, layer, out, pool):
    """Layer `layer` of a stack: out[e] = pool[perm_layer[e]] (pool from pool_records)."""
    perm = layer_permutation(cfg, layer)
    for e in range(cfg.E):
        out[e] = pool[perm[e]]
    return out


# ------------------------------------------------------------ routing

def correlated_sets(rng, steps, E, k, p):
    """[steps][k] sorted expert sets of one chain (see the package docstring)."""
    sets = np.zeros((steps, k), dtype=np.int32)
    cur = np.sort(rng.choice(E, size=k, replace=False))
    for t in range(steps):
        if t > 0:
            keep = cur[rng.random(k) < p]
            pool = np.setdiff1d(np.arange(E), keep)
            new = rng.choice(pool, size=k - keep.size, replace=False)
            cur = np.sort(np.concatenate([keep, new]))
        sets[t] = cur
    return sets


def uniform_sets(rng, steps, E, k):
    """[steps][k] sorted uniform k-subsets of E (first k of a random permutation)."""
    perm = np.argsort(rng.random((steps, E)), axis=1)[:, :k]
    return np.sort(perm, axis=1).astype(np.int32)


def logits_from_sets(rng, sets, E):
    """sets int [..., k] -> float32 logits [..., E] whose top-k is the set."""
    sets = np.asarray(sets)
    shape = sets.shape[:-1]
    z = rng.standard_normal(shape + (E,)).astype(np.float32)
    flat = z.reshape(-1, E)
    fs = sets.reshape(-1, sets.shape[-1])
    member = np.zeros(flat.shape, dtype=bool)
    np.put_along_axis(member, fs, True, axis=1)
    flat[member] += ROUTE_SHIFT
    lo_in = np.where(member, flat, np.inf).min(axis=1)
    hi_out = np.where(member, -np.inf, flat).max(axis=1)
    assert np.all(lo_in > hi_out)
    return flat.reshape(shape + (E,))


def normal_logits(rng, shape, E):
    return rng.standard_normal(tuple(shape) + (E,)).astype(np.float32)


def hidden_states(rng, shape, fmt):
    """N(0,1) hidden states: float32 for the f32 workload, else bf16 bit patterns."""
    x = rng.standard_normal(shape).astype(np.float32)
    return x if fmt == F32 else f32_to_bf16_bits(x)


# ------------------------------------------------------------ per-workload bundles

def decode_inputs(cfg, batch, steps=None):
    """Single-layer decode inputs: logits float32 [steps][B][E], x [steps][B][H]."""
    steps = cfg.steps if steps is None else steps
    st = streams(cfg.cid, batch)
    if cfg.routing == "normal":
        logits = normal_logits(st["routing"], (steps, batch), cfg.E)
    else:
        chains = []
        for b in range(batch):
            if cfg.routing == "correlated":
                chains.append(correlated_sets(st["routing"], steps, cfg.E, cfg.top_k, cfg.p_keep))
            else:
                chains.append(uniform_sets(st["routing"], steps, cfg.E, cfg.top_k))
        sets = np.stack(chains, axis=1)                        # [steps][B][k]
        logits = logits_from_sets(st["routing"], sets, cfg.E)
    x = hidden_states(st["hidden"], (steps, batch, cfg.H), cfg.fmt)
    return logits, x


def stack_inputs(cfg, steps=None, routing=None):
    """Stack inputs: logits float32 [steps][layers][B][E], x0 [steps][B][H]."""
    steps = cfg.steps if steps is None else steps
    routing = cfg.routing if routing is None else routing
    B = cfg.tokens
    st = streams(cfg.cid, 0 if routing == cfg.routing else 1)
    sets = np.zeros((steps, cfg.layers, B, cfg.top_k), dtype=np.int32)
    for l in range(cfg.layers):
        for b in range(B):
            if routing == "correlated":
                sets[:, l, b] = correlated_sets(st["routing"], steps, cfg.E, cfg.top_k, cfg.p_keep)
            else:
                sets[:, l, b] = uniform_sets(st["routing"], steps, cfg.E, cfg.top_k)
    logits = logits_from_sets(st["routing"], sets, cfg.E)
    x0 = hidden_states(st["hidden"], (steps, B, cfg.H), cfg.fmt)
    return logits, x0


def prefill_inputs(cfg, layers=None, tokens=None, salt=0):
    """Prefill inputs: logits float32 [layers][T][E] (fresh uniform k of E per
    token and layer), x0 [T][H] hidden states."""
    layers = cfg.layers if layers is None else layers
    T = cfg.tokens if tokens is None else tokens
    st = streams(cfg.cid, 100 + salt)
    sets = uniform_sets(st["routing"], layers * T, cfg.E, cfg.top_k).reshape(layers, T, cfg.top_k)
    logits = logits_from_sets(st["routing"], sets, cfg.E)
    x0 = hidden_states(st["hidden"], (T, cfg.H), cfg.fmt)
    return logits, x0


def cold_cycle_inputs(cfg, n_layers, batch, steps):
    """Decode inputs for n_layers independent layers of a one-layer workload's
    shape, taken in turn at every step (so a layer's experts leave the chip's
    caches before that layer runs again): logits float32
    [steps][n_layers][B][E], one routing chain of the workload's kind per layer
    and sequence, and x [steps][B][H]."""
    st = streams(cfg.cid, 300 + batch)
    sets = np.zeros((steps, n_layers, batch, cfg.top_k), dtype=np.int32)
    for l in range(n_layers):
        for b in range(batch):
            if cfg.routing == "correlated":
                sets[:, l, b] = correlated_sets(st["routing"], steps, cfg.E, cfg.top_k, cfg.p_keep)
            else:
                sets[:, l, b] = uniform_sets(st["routing"], steps, cfg.E, cfg.top_k)
    logits = logits_from_sets(st["routing"], sets, cfg.E)
    x = hidden_states(st["hidden"], (steps, batch, cfg.H), cfg.fmt)
    return logits, x
