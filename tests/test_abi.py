"""The C-ABI library loads and exports every function include/*.h declares
(no compute calls: this runs without a GPU)."""
import ctypes
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "expert_weight_paging_amd", "libmoepage.so")

DECL = re.compile(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s+\**\s*(moe_[a-z0-9_]+)\s*\(", re.M)


def declared():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        txt = open(h).read()
        txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
        names |= set(DECL.findall(txt))
    return sorted(names)


def test_header_declares_the_boundary():
    names = declared()
    for n in ("moe_layer_init", "moe_route", "moe_page_in", "moe_forward", "moe_plan_create",
              "moe_layer_stats", "moe_layer_get_state", "moe_layer_reset", "moe_layer_destroy",
              "moe_last_error", "moe_record_bytes", "moe_state_bytes"):
        assert n in names


@pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")
def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(LIB)
    missing = [n for n in declared() if not hasattr(lib, n)]
    assert not missing, missing


@pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")
def test_binding_covers_every_declared_symbol():
    import expert_weight_paging_amd as ewp
    assert set(declared()) == set(ewp.EXPORTS)


@pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")
def test_host_only_queries():
    """Pure host functions of the ABI (no GPU needed)."""
    import expert_weight_paging_amd as ewp
    from workloads import gen
    for fmt in (0, 1, 2, 3, 4):
        for H, I in ((2048, 768), (256, 384)):
            assert ewp.record_bytes(fmt, H, I) == gen.record_stride(fmt, H, I)
    assert ewp.record_bytes(1, 2048, 768) == 9437184
    assert ewp.record_bytes(2, 2048, 768) == 4719872          # 4,719,744 payload, 256-aligned
    assert ewp.record_bytes(3, 2048, 768) == 2506752
    assert ewp.record_bytes(2, 2000, 768) == 0                 # FP8 needs multiples of 128
    assert ewp.record_bytes(4, 2048, 768) == 2506752           # MXFP4: 4.25 bits a weight
    assert ewp.record_bytes(4, 2016, 768) == 2016 * 768 * 3 // 2 + 2016 * 768 * 3 // 32
    assert ewp.record_bytes(4, 2000, 768) == 0                 # MXFP4 needs multiples of 32
    assert ewp.record_bytes(9, 2048, 768) == 0
    assert ewp.state_bytes(128, 40) == 40 * 4 + 128 * 4 + 40 * 8 + 8
    assert ewp.lib().moe_last_error() is not None


@pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")
def test_slots_for_budget_matches_oracle():
    """Host-only sizing call against the oracle's definition."""
    import numpy as np
    import expert_weight_paging_amd as ewp
    from oracle import sizing
    rng = np.random.default_rng(7)
    for _ in range(200):
        fmt = int(rng.integers(1, 5))
        E, layers = int(rng.integers(1, 257)), int(rng.integers(1, 97))
        rec = ewp.record_bytes(fmt, 2048, 768)
        budget = int(rng.integers(0, 2 * E * layers * rec + 1))
        assert ewp.slots_for_budget(fmt, 2048, 768, E, layers, budget) == \
            sizing.slots_for_budget(rec, E, layers, budget)
    with pytest.raises(ewp.MoeError):
        ewp.slots_for_budget(1, 2048, 768, 128, 48, -1)
    with pytest.raises(ewp.MoeError):
        ewp.slots_for_budget(2, 2000, 768, 128, 48, 1 << 30)   # unsupported FP8 shape


@pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")
def test_preflight_matches_oracle():
    """Host-only preflight call against the oracle (pinned to the printed
    worked example in tests/golden/preflight.json) and on random inputs."""
    import json
    import numpy as np
    import expert_weight_paging_amd as ewp
    from oracle import sizing
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "preflight.json")))
    kv = sizing.kv_bytes_per_token(**g["kv"])
    rng = np.random.default_rng(8)
    cases = [(s["layers"], s["experts"], s["top_k"], s["expert_mb"], s["K"], s["link_gbps"], s["tok_s"])
             for s in g["setups"]]
    for _ in range(100):
        E = int(rng.integers(2, 300))
        cases.append((int(rng.integers(1, 96)), E, int(rng.integers(1, min(E, 32) + 1)),
                      float(rng.uniform(0.1, 20)), int(rng.integers(1, E + 1)),
                      float(rng.uniform(1, 100)), float(rng.uniform(1, 500))))
    for c in cases:
        got = ewp.preflight(*c, kv)
        ref = sizing.preflight(*c, kv)
        for key in ("slot_mb", "kv_tokens_per_slot", "all_miss_gb_per_token", "max_miss", "random_miss"):
            assert got[key] == pytest.approx(ref[key], rel=1e-12), (c, key)
        assert got["batch_cap"] == ref["batch_cap"]
        assert got["reuse_implied"] == (ref["verdict"] == "reuse implied")
    with pytest.raises(ewp.MoeError):
        ewp.preflight(48, 128, 8, 2.43, 129, 50.0, 205.6, kv)   # K > E


@pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")
def test_null_handles_are_refused_without_a_gpu():
    """Every entry point that takes a layer or plan handle returns
    MOE_ERR_INVALID_ARG (-1) for a null one, before any HIP call (the header
    promises that nothing aborts across the ABI)."""
    import expert_weight_paging_amd as ewp
    L = ewp.lib()
    assert L.moe_route(None, None, 1, None) == -1
    assert L.moe_route(None, None, 0, None) == -1
    assert L.moe_page_in(None, None, 0) == -1
    assert L.moe_forward(None, None, 0, None, None) == -1
    assert L.moe_layer_reset(None) == -1
    assert L.moe_layer_stats(None, None) == -1
    assert L.moe_layer_get_state(None, None, None, None, None) == -1
    assert L.moe_plan_get_info(None, None) == -1
    assert L.moe_plan_get_wave(None, 0, None) == -1
    assert L.moe_plan_read(None, None, None, None, None) == -1
    assert L.moe_plan_create(None, 1, None) == -1
    assert L.moe_step_device(None, None, None, 1, None, None, None) == -1
    assert L.moe_step_token_waves(None, None, None, 1, None, None, None) == -1
    assert L.moe_stack_forward(None, None, 0, None, 1, None, None, 0) == -1
    assert L.moe_stack_forward_device(None, None, 0, None, 1, None, None, 0) == -1
    assert L.moe_timing_enable(None, 1) == -1
    assert L.moe_timing_read(None, None) == -1
    assert L.moe_layer_init(None, None, None, None, None) == -1

    L.moe_layer_destroy(None)
    L.moe_plan_destroy(None)
    assert b"null" in L.moe_last_error()
    assert L.moe_rmsnorm_bf16(None, None, 1, 2048, None) == -1        # null rows
    assert L.moe_rmsnorm_bf16(None, None, 0, 2044, None) == -1        # H not a multiple of 8


@pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")
def test_read_probe_refuses_bad_arguments():
    """The measurement helper validates before any launch (no GPU needed)."""
    lib = ctypes.CDLL(LIB)
    lib.moe_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_size_t,
                                   ctypes.c_int32, ctypes.POINTER(ctypes.c_double)]
    us = ctypes.c_double()
    assert lib.moe_read_probe(None, None, 1 << 20, 4096, 10, ctypes.byref(us)) == -1
    assert lib.moe_read_probe(None, ctypes.c_void_p(256), 1 << 20, 100, 10, ctypes.byref(us)) == -1  # not 16-aligned size
    assert lib.moe_read_probe(None, ctypes.c_void_p(256), 4096, 4096, 10, ctypes.byref(us)) == -1     # over half the buffer
    assert lib.moe_read_probe(None, ctypes.c_void_p(256), 1 << 20, 4096, 0, ctypes.byref(us)) == -1   # reps
