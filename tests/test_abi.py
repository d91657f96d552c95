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
    for fmt in (0, 1, 2, 3):
        for H, I in ((2048, 768), (256, 384)):
            assert ewp.record_bytes(fmt, H, I) == gen.record_stride(fmt, H, I)
    assert ewp.record_bytes(1, 2048, 768) == 9437184
    assert ewp.record_bytes(2, 2048, 768) == 4719872          # 4,719,744 payload, 256-aligned
    assert ewp.record_bytes(3, 2048, 768) == 2506752
    assert ewp.record_bytes(2, 2000, 768) == 0                 # FP8 needs multiples of 128
    assert ewp.record_bytes(9, 2048, 768) == 0
    assert ewp.state_bytes(128, 40) == 40 * 4 + 128 * 4 + 40 * 8 + 8
    assert ewp.lib().moe_last_error() is not None
