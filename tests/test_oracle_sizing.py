"""Oracle sizing arithmetic pinned to the numbers the [PE] page prints."""
import json
import os

import numpy as np
import pytest

from oracle import sizing

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _pct(v):
    # the page prints with a whole-percent format, which rounds half to even
    return int(format(v, ".0%").rstrip("%"))


@pytest.mark.parametrize("i", [0, 1, 2])
def test_preflight_worked_example(i):
    g = _load("preflight.json")
    s = g["setups"][i]
    kv = sizing.kv_bytes_per_token(**g["kv"])
    r = sizing.preflight(s["layers"], s["experts"], s["top_k"], s["expert_mb"], s["K"],
                         s["link_gbps"], s["tok_s"], kv)
    p = s["printed"]
    assert int(format(r["slot_mb"], ".0f")) == p["slot_mb"]
    assert int(format(r["kv_tokens_per_slot"], ".0f")) == p["kv_tokens"]
    assert r["batch_cap"] == p["batch_cap"]
    assert _pct(r["random_miss"]) == p["random_miss_pct"]
    assert _pct(r["max_miss"]) == p["max_miss_pct"]
    assert r["verdict"] == p["verdict"]


def test_closed_forms():
    g = {e["what"]: e for e in _load("closed_forms.json")["entries"]}
    kv = sizing.kv_bytes_per_token()
    i4 = sizing.preflight(48, 128, 8, 2.43, 92, 50.0, 205.6, kv)
    f8 = sizing.preflight(48, 128, 8, 4.72, 40, 50.0, 87.7, kv)
    lap = sizing.preflight(48, 128, 8, 2.43, 26, 15.75, 32.6, kv)
    got = {
        "bf16 KV bytes per token (2 x 48 layers x 4 heads x 128 dim x 2 B)": kv,
        "GB per token if every activation missed, int4 2.43 MB experts": i4["all_miss_gb_per_token"],
        "GB per token if every activation missed, FP8 4.72 MB experts": f8["all_miss_gb_per_token"],
        "GB/s needed at 87.7 tok/s if every FP8 activation missed":
            sizing.link_needed_gbps(f8["all_miss_gb_per_token"], 87.7),
        "int4 16 GB bound at a 63 GB/s link, percent":
            100 * sizing.preflight(48, 128, 8, 2.43, 92, 63.0, 205.6, kv)["max_miss"],
        "FP8 K=40 decode cap under uniform routing at 50 GB/s, tok/s":
            50.0 / (sizing.uniform_miss_rate(128, 40) * f8["all_miss_gb_per_token"]),
        "laptop int4 K=26 decode cap under uniform routing at 15.75 GB/s, tok/s":
            15.75 / (sizing.uniform_miss_rate(128, 26) * lap["all_miss_gb_per_token"]),
        "prefill page-in int4 K=92, GB": sizing.prefill_page_in_gb(128, 92, i4["slot_mb"]),
        "prefill page-in FP8 K=40, GB": sizing.prefill_page_in_gb(128, 40, f8["slot_mb"]),
        "prefill page-in laptop int4 K=26, GB": sizing.prefill_page_in_gb(128, 26, lap["slot_mb"]),
        "laptop prefill page-in time at 15.75 GB/s, at least this many ms":
            1e3 * sizing.prefill_page_in_gb(128, 26, lap["slot_mb"]) / 15.75,
        "host RAM to pin, int4, GB": sizing.host_store_gb(128, 48, 2.43),
        "host RAM to pin, FP8, GB": sizing.host_store_gb(128, 48, 4.72),
        "int4 slot in KV tokens with an FP8 KV cache, about":
            i4["slot_mb"] * 1e6 / sizing.kv_bytes_per_token(elem_bytes=1),
        "KV tokens bought by dropping K by 10 on int4, roughly": 10 * i4["kv_tokens_per_slot"],
        "the 10,240-token KV cache, GB": 10240 * kv / 1e9,
    }
    assert set(got) == set(g)
    for k, v in got.items():
        assert abs(v - g[k]["value"]) <= g[k]["tol"], (k, v, g[k]["value"])
    # the laptop figure is a lower bound ("at least")
    assert got["laptop prefill page-in time at 15.75 GB/s, at least this many ms"] >= 750


def test_uniform_rate_table():
    # [PE] 'Why is it fast ...', the no-reuse column: 69%, 80%, 28%
    assert round(100 * sizing.uniform_miss_rate(128, 40)) == 69
    assert round(100 * sizing.uniform_miss_rate(128, 26)) == 80
    assert round(100 * sizing.uniform_miss_rate(128, 92)) == 28


def _largest_fit(rec, E, layers, budget):
    # brute force: walk K up while one more slot per layer still fits
    K = 0
    while K < E and (K + 1) * layers * rec <= budget:
        K += 1
    return K


def test_slots_for_budget_against_brute_force():
    rng = np.random.default_rng(3)
    for _ in range(300):
        rec = int(rng.integers(1, 10_000_000))
        E = int(rng.integers(1, 300))
        layers = int(rng.integers(1, 64))
        budget = int(rng.integers(0, 2 * E * layers * rec + 1))
        assert sizing.slots_for_budget(rec, E, layers, budget) == _largest_fit(rec, E, layers, budget)


def test_slots_for_budget_boundaries():
    rec, layers = 2_506_752, 48          # int4 asym g128 record of the stack workload
    exact = 92 * layers * rec
    assert sizing.slots_for_budget(rec, 128, layers, exact) == 92
    assert sizing.slots_for_budget(rec, 128, layers, exact - 1) == 91
    assert sizing.slots_for_budget(rec, 128, layers, 10 ** 15) == 128   # never more than E
    assert sizing.slots_for_budget(rec, 128, layers, 0) == 0
