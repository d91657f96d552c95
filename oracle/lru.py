"""Per-layer K-slot expert table with least-recently-used replacement and waves.

[PE] "TL;DR" / "What does Paged Experts actually do?": every MoE layer keeps K
of its E experts in a slot table on the GPU; each step copies in only the
routed experts that are not resident, the least recently used slot going out.
[LRU] "The fix": a hit computes from the cached copy and moves no bytes; a miss
copies that one expert in and evicts the least recently used one.
[PE] "What happens with more than one request?": a step fits one wave only when
what it routes fits the table; otherwise it runs several waves, each with its
own page-in.

State per layer: slot_expert[K] (-1 = empty), expert_slot[E] (-1 = absent),
stamp[K] (-1 = empty slot), clock (starts at 0).

Readings where the pages leave a step open:
  * distinct set D = sorted distinct routed ids; hits H = resident members of D,
    misses M = the rest, both ascending; the wave order is H followed by M and
    waves are consecutive chunks of K of it, so n_waves = ceil(|D| / K) and a
    step is one wave exactly when |D| <= K;
  * the clock ticks once per wave; every expert of a wave gets that wave's
    stamp (hits and misses alike);
  * experts of the current wave are never victims; victims are the other slots
    ordered by (stamp, slot index), so empty slots go first, then the oldest,
    equal stamps to the lower slot index; the i-th miss (ascending id) goes to
    the i-th victim;
  * with initial fill, experts 0..K-1 sit in slots 0..K-1 with stamp 0.
"""
import numpy as np


class WavePlan:
    """One wave: its experts (wave order), the slot each sits in, and the miss list."""

    def __init__(self, experts, slots, misses):
        self.experts = experts      # list[int], wave order (hits first, then misses)
        self.slots = slots          # list[int], slot of each expert during this wave
        self.misses = misses        # list[(expert, slot)], ascending expert id


class StepPlan:
    def __init__(self):
        self.distinct = []          # sorted distinct ids
        self.hits = []              # ascending
        self.missed = []            # ascending (all waves)
        self.waves = []             # list[WavePlan]
        self.slot_ids = None        # int32 [B, k]: slot of each (token, j) during its wave
        self.wave_of = None         # int32 [B, k]

    @property
    def n_waves(self):
        return len(self.waves)

    @property
    def n_misses(self):
        return sum(len(w.misses) for w in self.waves)


class SlotTable:
    def __init__(self, num_experts, num_slots, initial_fill=False):
        if not (1 <= num_slots <= num_experts):
            raise ValueError("need 1 <= K <= E")
        self.E = int(num_experts)
        self.K = int(num_slots)
        self.initial_fill = bool(initial_fill)
        self.reset()

    def reset(self):
        E, K = self.E, self.K
        self.slot_expert = np.full(K, -1, dtype=np.int32)
        self.expert_slot = np.full(E, -1, dtype=np.int32)
        self.stamp = np.full(K, -1, dtype=np.int64)
        self.clock = 0
        if self.initial_fill:
            for s in range(K):
                self.slot_expert[s] = s
                self.expert_slot[s] = s
                self.stamp[s] = 0

    def state(self):
        return (self.slot_expert.copy(), self.expert_slot.copy(),
                self.stamp.copy(), int(self.clock))

    def plan(self, ids, on_page_in=None):
        """Plan one step for routed ids int [B, k]; mutates the table.

        on_page_in(expert, slot) is called for each miss, in wave order, at
        the moment the expert enters its slot (the caller copies the record).
        """
        ids = np.asarray(ids, dtype=np.int64)
        B, k = ids.shape
        K = self.K
        plan = StepPlan()
        distinct = sorted(set(int(e) for e in ids.ravel()))
        hits = [e for e in distinct if self.expert_slot[e] >= 0]
        missed = [e for e in distinct if self.expert_slot[e] < 0]
        order = hits + missed
        plan.distinct, plan.hits, plan.missed = distinct, hits, missed
        n_waves = (len(order) + K - 1) // K
        wave_index = {}
        slot_at_wave = {}
        for w in range(n_waves):
            need = order[w * K:(w + 1) * K]
            need_set = set(need)
            self.clock += 1
            miss_w = [e for e in need if self.expert_slot[e] < 0]   # ascending (M is)
            candidates = [s for s in range(K)
                          if not (self.slot_expert[s] >= 0 and int(self.slot_expert[s]) in need_set)]
            candidates.sort(key=lambda s: (int(self.stamp[s]), s))
            victims = candidates[:len(miss_w)]
            misses = []
            for e, s in zip(miss_w, victims):
                old = int(self.slot_expert[s])
                if old >= 0:
                    self.expert_slot[old] = -1
                self.slot_expert[s] = e
                self.expert_slot[e] = s
                misses.append((e, s))
                if on_page_in is not None:
                    on_page_in(e, s)
            slots = []
            for e in need:
                s = int(self.expert_slot[e])
                self.stamp[s] = self.clock
                slots.append(s)
                wave_index[e] = w
                slot_at_wave[e] = s
            plan.waves.append(WavePlan(list(need), slots, misses))
        plan.slot_ids = np.array([[slot_at_wave[int(e)] for e in row] for row in ids],
                                 dtype=np.int32).reshape(B, k)
        plan.wave_of = np.array([[wave_index[int(e)] for e in row] for row in ids],
                                dtype=np.int32).reshape(B, k)
        return plan
