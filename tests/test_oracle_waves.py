"""Pins of the token-partitioned wave policy (batches larger than one wave).

[PE] "What happens with more than one request?": up to K // top_k tokens
always fit one wave; a larger batch needs several waves, each with its own
page-in. Two ways to cut it: by experts (the distinct set in chunks of K, each
expert paged at most once per step) and by tokens (groups of at most
K // top_k tokens, each group a single-wave step). The pins below come from
the mathematics, not from the oracle: a lower bound every policy obeys, a
worked case where token groups page an expert twice, the group count, and the
equality of outputs with the plain (unpaged) MoE layer."""
import numpy as np
import pytest

from oracle.layer import PagedLayer
from oracle.lru import SlotTable
from workloads import gen


def _store(E, H, I, seed):
    rng = np.random.default_rng(seed)
    return np.stack([gen.encode_record(gen.F32, (rng.standard_normal((2 * I, H)) * 0.2).astype(np.float32),
                                       (rng.standard_normal((H, I)) * 0.2).astype(np.float32))
                     for _ in range(E)])


def _logits_for(sets, E, rng):
    """Logits whose top-k is exactly each row's set (set members lifted by 16)."""
    lg = rng.standard_normal((len(sets), E)).astype(np.float32)
    for b, s in enumerate(sets):
        lg[b, list(s)] += 16.0
    return lg


def test_worked_case_token_groups_page_an_expert_twice():
    """k = K = 2, groups of one token: tokens 0 and 2 route to {0, 1}, token 1
    to {2, 3}. Token groups page {0,1}, then {2,3} (evicting both), then {0,1}
    again: 6 page-ins. Expert waves page each of the 4 distinct experts once."""
    E, k, K, H, I = 6, 2, 2, 8, 4
    store = _store(E, H, I, 1)
    lg = _logits_for([{0, 1}, {2, 3}, {0, 1}], E, np.random.default_rng(2))
    x = np.random.default_rng(3).standard_normal((3, H))
    tok = PagedLayer(store, gen.F32, E, k, H, I, K)
    out_t, _, _, plans = tok.step_token_waves(lg, x, group=1)
    assert [p.n_waves for p in plans] == [1, 1, 1]
    assert sum(p.n_misses for p in plans) == 6
    exp = PagedLayer(store, gen.F32, E, k, H, I, K)
    out_e, _, _, plan = exp.step(lg, x)
    assert plan.n_misses == 4 and plan.n_waves == 2
    assert np.allclose(out_t, out_e, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("K,k,B", [(4, 2, 5), (6, 3, 7), (8, 2, 9), (5, 2, 3)])
def test_token_waves_bounds_and_outputs(K, k, B):
    """From the same table state, every group is one wave, the number of
    groups is ceil(B / G), the page-ins are at least the batch's missing
    distinct experts (each must be paged once; the expert-partitioned step
    reaches that bound), and the outputs equal the unpaged layer's."""
    E, H, I = 10, 8, 4
    store = _store(E, H, I, K * 10 + B)
    rng = np.random.default_rng(K + 100 * B)
    G = K // k
    tok = PagedLayer(store, gen.F32, E, k, H, I, K)
    exp = PagedLayer(store, gen.F32, E, k, H, I, K)
    for step in range(12):
        lg = rng.standard_normal((B, E)).astype(np.float32)
        x = rng.standard_normal((B, H))
        # same start state for both policies
        exp.table.slot_expert[:], exp.table.expert_slot[:] = tok.table.slot_expert, tok.table.expert_slot
        exp.table.stamp[:], exp.table.clock = tok.table.stamp, tok.table.clock
        exp.slots[:] = tok.slots
        exp._cache = {}
        resident = set(int(e) for e in tok.table.slot_expert if e >= 0)
        ref_unpaged = exp.unpaged_forward(lg, x)
        out_e, ids_e, _, plan_e = exp.step(lg, x)
        clock0 = tok.table.clock
        out_t, ids_t, _, plans = tok.step_token_waves(lg, x, group=G)
        assert len(plans) == -(-B // G) and tok.table.clock == clock0 + len(plans)
        assert all(p.n_waves == 1 for p in plans)
        assert np.array_equal(ids_t, ids_e)
        need = set(int(e) for e in ids_e.ravel()) - resident
        assert plan_e.n_misses == len(need)
        assert sum(p.n_misses for p in plans) >= len(need)
        assert np.allclose(out_t, ref_unpaged, rtol=1e-12, atol=1e-14)
        assert np.allclose(out_e, ref_unpaged, rtol=1e-12, atol=1e-14)


def test_one_group_is_the_plain_step():
    """B <= K // top_k: one group, the same plan and bytes as a plain step."""
    E, k, K, H, I, B = 12, 2, 6, 8, 4, 3
    store = _store(E, H, I, 5)
    rng = np.random.default_rng(6)
    a = PagedLayer(store, gen.F32, E, k, H, I, K)
    b = PagedLayer(store, gen.F32, E, k, H, I, K)
    for _ in range(10):
        lg = rng.standard_normal((B, E)).astype(np.float32)
        x = rng.standard_normal((B, H))
        oa, _, _, pa = a.step(lg, x)
        ob, _, _, pb = b.step_token_waves(lg, x, group=K // k)
        assert len(pb) == 1 and np.array_equal(oa, ob)
        assert np.array_equal(pa.slot_ids, pb[0].slot_ids) and pa.missed == pb[0].missed
    with pytest.raises(ValueError):
        b.step_token_waves(lg, x, group=K // k + 1)
