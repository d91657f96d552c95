"""Oracle slot-table pins.

* an independent move-to-front model (a recency list of slots, no stamps) on
  every routing sequence over tiny E, every K, must give the same slots, miss
  lists and waves;
* the LRU property: nothing is evicted while a less recently used,
  unprotected resident stays;
* K = E gives zero misses once every expert has been seen;
* misses per step <= B * top_k and <= distinct; one wave iff distinct <= K
  ([PE] "What happens with more than one request?");
* uniform routing misses at 1 - K/E ([PE] "Why is it fast ...", no-reuse column);
* the correlated process misses at its closed form.
"""
import itertools
import math

import numpy as np
import pytest

from oracle.lru import SlotTable
from workloads import gen


class MoveToFront:
    """Recency list of slot indices, least recent first; a wave moves its slots
    to the back in ascending slot order. Empty slots start at the front."""

    def __init__(self, E, K, fill=False):
        self.E, self.K = E, K
        self.slot = [s if fill else None for s in range(K)]
        self.recency = list(range(K))

    def step(self, ids):
        distinct = sorted(set(int(e) for e in np.ravel(ids)))
        resident = set(e for e in self.slot if e is not None)
        order = [e for e in distinct if e in resident] + [e for e in distinct if e not in resident]
        waves = []
        where = {}
        for w0 in range(0, len(order), self.K):
            need = order[w0:w0 + self.K]
            resident = set(e for e in self.slot if e is not None)
            miss = [e for e in need if e not in resident]
            victims = [s for s in self.recency if self.slot[s] not in need][:len(miss)]
            pairs = list(zip(miss, victims))
            for e, s in pairs:
                self.slot[s] = e
            used = sorted(self.slot.index(e) for e in need)
            self.recency = [s for s in self.recency if s not in used] + used
            for e in need:
                where[e] = (len(waves), self.slot.index(e))
            waves.append((list(need), pairs))
        return waves, where


def _compare(E, K, k, B, seq, fill=False):
    t = SlotTable(E, K, fill)
    m = MoveToFront(E, K, fill)
    for ids in seq:
        ids = np.asarray(ids).reshape(B, k)
        p = t.plan(ids)
        waves, where = m.step(ids)
        assert [w.experts for w in p.waves] == [w[0] for w in waves]
        assert [w.misses for w in p.waves] == [w[1] for w in waves]
        for b in range(B):
            for j in range(k):
                assert (p.wave_of[b, j], p.slot_ids[b, j]) == where[int(ids[b, j])]
        assert [e if e is not None else -1 for e in m.slot] == t.slot_expert.tolist()


def test_move_to_front_all_sequences_b1():
    for E in range(1, 6):
        for k in range(1, min(E, 2) + 1):
            sets = list(itertools.combinations(range(E), k))
            for K in range(1, E + 1):
                for seq in itertools.product(sets, repeat=3):
                    _compare(E, K, k, 1, seq)
                    _compare(E, K, k, 1, seq, fill=True)


def test_move_to_front_all_sequences_b2():
    E, k, B = 4, 1, 2
    toks = list(itertools.product(range(E), repeat=B))
    for K in range(1, E + 1):
        for seq in itertools.product(toks, repeat=3):
            _compare(E, K, k, B, seq)


def test_move_to_front_random_long():
    rng = np.random.default_rng(3)
    for _ in range(40):
        E = int(rng.integers(4, 24))
        k = int(rng.integers(1, min(E, 4) + 1))
        K = int(rng.integers(1, E + 1))
        B = int(rng.integers(1, 4))
        seq = [np.stack([rng.choice(E, k, replace=False) for _ in range(B)]) for _ in range(30)]
        _compare(E, K, k, B, seq, fill=bool(rng.integers(2)))


def test_lru_property_and_bounds():
    rng = np.random.default_rng(4)
    for _ in range(30):
        E = int(rng.integers(6, 40))
        k = int(rng.integers(1, 5))
        K = int(rng.integers(1, E + 1))
        B = int(rng.integers(1, 4))
        t = SlotTable(E, K)
        last_use = {}
        tick = 0
        for _step in range(40):
            ids = np.stack([rng.choice(E, k, replace=False) for _ in range(B)])
            slots = [int(e) if e >= 0 else None for e in t.slot_expert]
            before = set(e for e in slots if e is not None)
            p = t.plan(ids)
            D = len(set(ids.ravel().tolist()))
            assert p.n_waves == math.ceil(D / K)
            assert (p.n_waves == 1) == (D <= K)
            assert p.n_misses <= B * k and p.n_misses <= D
            assert p.n_misses == len([e for e in set(ids.ravel().tolist()) if e not in before])
            # replay the miss lists on our own copy of the table
            for w in p.waves:
                tick += 1
                need = set(w.experts)
                for e, s in w.misses:
                    old = slots[s]
                    if old is None:
                        pass
                    else:
                        assert old not in need
                        # no empty slot may be left while a resident is evicted
                        assert None not in slots
                        # the evicted expert is (one of) the least recently used evictable
                        others = [r for r in slots if r is not None and r not in need]
                        assert last_use[old] == min(last_use[r] for r in others)
                    slots[s] = e
                for e in need:
                    last_use[e] = tick
                assert need <= set(slots)
            assert slots == [int(e) if e >= 0 else None for e in t.slot_expert]


def test_k_equals_e_no_misses_after_warmup():
    rng = np.random.default_rng(5)
    E, k = 32, 4
    t = SlotTable(E, E)
    seen = set()
    for step in range(300):
        ids = rng.choice(E, k, replace=False)[None]
        p = t.plan(ids)
        if seen >= set(range(E)):
            assert p.n_misses == 0 and p.n_waves == 1
        seen |= set(ids.ravel().tolist())
    assert seen == set(range(E))


def _rate(E, K, k, steps, sets):
    t = SlotTable(E, K)
    miss = acts = 0
    for s in range(steps):
        p = t.plan(sets[s][None])
        if s >= 200:
            miss += p.n_misses
            acts += k
    return miss, acts


def test_uniform_routing_miss_rate():
    E, K, k, steps = 128, 40, 8, 6200
    rng = np.random.default_rng(6)
    sets = gen.uniform_sets(rng, steps, E, k)
    miss, acts = _rate(E, K, k, steps, sets)
    p = 1 - K / E
    # per-step draws are independent: binomial-ish error over activations
    se = math.sqrt(p * (1 - p) / acts) * math.sqrt(k)
    assert abs(miss / acts - p) < 4 * se, (miss / acts, p)


def _correlated_closed_form(E, K, k, p):
    """E[misses per step] after warm-up: keep m ~ Bin(k, p); each of the k - m
    new draws is uniform over the E - m experts not kept, of which E - K are
    not resident (the K residents include the whole previous set)."""
    return sum(math.comb(k, m) * p ** m * (1 - p) ** (k - m) * (k - m) * (E - K) / (E - m)
               for m in range(k + 1))


@pytest.mark.parametrize("K,expect", [(40, 1.4339), (92, 0.5866)])
def test_correlated_routing_closed_form(K, expect):
    E, k, p, steps = 128, 8, 0.75, 8200
    assert abs(_correlated_closed_form(E, K, k, p) - expect) < 1e-4
    rng = np.random.default_rng(7 + K)
    sets = gen.correlated_sets(rng, steps, E, k, p)
    miss, _ = _rate(E, K, k, steps, sets)
    mean = miss / (steps - 200)
    # misses per step are bounded by k and only weakly correlated across steps
    se = math.sqrt(k * k / 4 / (steps - 200)) * 2
    assert abs(mean - expect) < 4 * se, (mean, expect)
    assert abs(mean - expect) < 0.08


def _p_one_wave(E, k, B, K):
    """Exact P(|union of B independent uniform k-sets of E| <= K)."""
    dist = {k: 1.0}
    tot = math.comb(E, k)
    for _ in range(B - 1):
        nd = {}
        for u, pu in dist.items():
            for j in range(0, k + 1):
                if j > E - u or k - j > u:
                    continue
                pj = math.comb(E - u, j) * math.comb(u, k - j) / tot
                nd[u + j] = nd.get(u + j, 0.0) + pu * pj
        dist = nd
    return sum(p for u, p in dist.items() if u <= K)


def test_wave_split_statistics_batch6():
    E, k, K, B, n = 128, 8, 40, 6, 3000
    exact = _p_one_wave(E, k, B, K)
    assert abs(exact - 0.377) < 0.001
    assert _p_one_wave(E, k, 5, K) == pytest.approx(1.0)
    rng = np.random.default_rng(8)
    t = SlotTable(E, K)
    one = 0
    for _ in range(n):
        ids = np.stack([rng.choice(E, k, replace=False) for _ in range(B)])
        one += t.plan(ids).n_waves == 1
    se = math.sqrt(exact * (1 - exact) / n)
    assert abs(one / n - exact) < 4 * se


def test_batch_cap_always_one_wave():
    # B <= K // top_k always fits one wave ([PE] "What happens with more than one request?")
    rng = np.random.default_rng(9)
    for K in (8, 16, 40, 92):
        t = SlotTable(128, K)
        B = K // 8
        for _ in range(200):
            ids = np.stack([rng.choice(128, 8, replace=False) for _ in range(B)])
            assert t.plan(ids).n_waves == 1


def test_initial_fill_state():
    t = SlotTable(10, 4, initial_fill=True)
    se, es, st, clk = t.state()
    assert se.tolist() == [0, 1, 2, 3] and st.tolist() == [0, 0, 0, 0] and clk == 0
    assert es.tolist() == [0, 1, 2, 3, -1, -1, -1, -1, -1, -1]
    p = t.plan(np.array([[5, 1]]))
    # hit 1 (slot 1); miss 5 takes the lowest-index slot among the equal-stamp others
    assert p.waves[0].misses == [(5, 0)]
    assert p.slot_ids.tolist() == [[0, 1]]
