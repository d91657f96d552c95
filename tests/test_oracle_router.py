"""Oracle router pins: brute-force tie rule, torch.topk, softmax identities."""
import itertools

import numpy as np
import pytest
import torch

from oracle.router import route, topk_ids


def _brute_ok(z, sel):
    """Definition check: every selected id beats every unselected id (tie -> smaller id),
    and the listing is by descending logit then ascending id."""
    sel = list(sel)
    others = [j for j in range(len(z)) if j not in sel]
    for i in sel:
        for j in others:
            if not (z[i] > z[j] or (z[i] == z[j] and i < j)):
                return False
    for a, b in zip(sel, sel[1:]):
        if not (z[a] > z[b] or (z[a] == z[b] and a < b)):
            return False
    return True


def test_topk_brute_force_with_ties():
    rng = np.random.default_rng(0)
    for E in (2, 3, 5, 8):
        for _ in range(200):
            z = rng.integers(-2, 3, size=E).astype(np.float32)      # many ties
            if rng.random() < 0.3:
                z[rng.integers(E)] = -0.0
            for k in range(1, E + 1):
                sel = topk_ids(z, k)
                assert _brute_ok(z, sel)
                # exhaustive: the selected set is the unique k-subset passing the rule
                n_ok = sum(_brute_ok(z, sorted(c, key=lambda i: (-z[i], i)))
                           for c in itertools.combinations(range(E), k))
                assert n_ok == 1


def test_topk_matches_torch_on_tie_free_inputs():
    rng = np.random.default_rng(1)
    for _ in range(50):
        z = rng.standard_normal(128).astype(np.float32)
        assert len(np.unique(z)) == 128
        v, i = torch.topk(torch.from_numpy(z), 8)
        assert topk_ids(z, 8).tolist() == i.tolist()


def test_signed_zero_is_a_tie():
    z = np.array([-0.0, 0.0, -1.0], dtype=np.float32)
    assert topk_ids(z, 1).tolist() == [0]
    z = np.array([0.0, -0.0, -1.0], dtype=np.float32)
    assert topk_ids(z, 1).tolist() == [0]


def test_weights_renormalised_softmax():
    rng = np.random.default_rng(2)
    logits = rng.standard_normal((16, 128)).astype(np.float32) * 3
    ids, w = route(logits, 8)
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-15)
    for b in range(16):
        # softmax over all E then renormalised == softmax over the k selected logits
        sel = torch.from_numpy(logits[b, ids[b]].astype(np.float64))
        ref = torch.softmax(sel, dim=0).numpy()
        assert np.allclose(w[b], ref, rtol=1e-13, atol=0)
        # weights follow the logit order
        assert np.all(np.diff(w[b]) <= 0)


def test_route_rejects_nonfinite():
    z = np.zeros((1, 4), dtype=np.float32)
    z[0, 2] = np.nan
    with pytest.raises(ValueError):
        route(z, 2)
