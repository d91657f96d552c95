"""bench.py's command-line contract on the CPU (no GPU run): refusals that
must happen before any device work, and the default execution mode."""
import argparse
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*argv):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv],
                          capture_output=True, text=True, cwd=ROOT, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""


def test_conflicting_modes_are_refused():
    assert _run("--host", "--device").returncode == 2
    assert _run("--workload", "prefill-bf16", "--device").returncode == 2
    assert _run("--workload", "decode-bf16", "--graph").returncode == 2
    assert _run("--workload", "stack-int4", "--slots", "24").returncode == 2


def test_default_mode_follows_the_one_wave_condition():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)

    def mode(workload, batch=1, slots=None, host=False, lookahead=False):
        a = argparse.Namespace(host=host, device=False, graph=False, waves="expert", workload=workload,
                               batch=batch, slots=slots, lookahead=lookahead)
        b.resolve_default_mode(a)
        return a.device, a.graph
    assert mode("decode-bf16") == (True, False)              # 1 x 8 <= 40
    assert mode("decode-fp8", batch=5) == (True, False)      # 5 x 8 <= 40
    assert mode("decode-fp8", batch=6) == (True, False)      # 48 > 40: two device-resolved waves
    assert mode("decode-fp8", batch=4, slots=24) == (True, False)
    assert mode("decode-fp8", batch=8, slots=3) == (False, False)  # 22 possible waves of 3: host-driven
    assert mode("decode-bf16", host=True) == (False, False)
    assert mode("stack-int4") == (False, True)
    assert mode("stack-int4", lookahead=True) == (False, False)
    assert mode("prefill-bf16") == (False, False)


def _bench_module():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    return b


def _timing(entries):
    names = ("route", "page_in", "ffn_up", "ffn_down", "gemm_up", "gemm_down", "combine")
    t = {k: {"count": 0, "ms": 0.0, "bytes": 0.0, "flops": 0.0} for k in names}
    for k, v in entries.items():
        t[k].update(v)
    return t


def test_decode_roofline_is_the_ffn_pair_over_hbm():
    """Achieved = the weight bytes of both FFN launches over their summed
    event time; each kernel's own figure beside it."""
    b = _bench_module()
    tm = _timing({"ffn_up": {"count": 4, "ms": 4 * 10e-3, "bytes": 4 * 50331648.0},
                  "ffn_down": {"count": 4, "ms": 4 * 7e-3, "bytes": 4 * 25165824.0}})
    r = b.hbm_roofline(tm, 3.9, "no such variant")
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert abs(r["achieved"] - 75497472.0 / 17e-6 / 1e9) < 0.1
    assert abs(r["frac"] - r["achieved"] / 8000.0) < 1e-4
    assert abs(r["kernels"]["ffn_up_kernel"]["achieved"] - 50331648.0 / 10e-6 / 1e9) < 0.1
    assert r["traffic"] is None  # no counters stored for this variant


def test_prefill_roofline_takes_the_binding_roof():
    """A grouped GEMM below the bf16 MFMA ridge (312.5 flop per weight byte) is
    reported against HBM, one above it against the matrix cores; the other
    roof's figure is kept beside it."""
    b = _bench_module()
    W = 268435456.0  # weight bytes per launch
    res = {"floor_us": 3.9}
    for ai, bound in ((128.0, "hbm"), (400.0, "mfma")):
        res["timing"] = _timing({"gemm_up": {"count": 3, "ms": 3 * 0.08, "bytes": 3 * W, "flops": 3 * W * ai},
                                 "gemm_down": {"count": 3, "ms": 3 * 0.07, "bytes": 3 * W / 2,
                                               "flops": 3 * W / 2 * ai}})
        r = b.roofline(res, "prefill-bf16", "no such variant")
        assert r["bound"] == bound and r["kernel"] == "grouped_gemm_kernel<true,1>"
        assert abs(r["flop_per_weight_byte"] - ai) < 0.1
        gbps, tflops = W / 80e-6 / 1e9, W * ai / 80e-6 / 1e12
        if bound == "hbm":
            assert abs(r["achieved"] - gbps) < 0.2 and abs(r["mfma_TFLOPs"] - tflops) < 0.2
        else:
            assert abs(r["achieved"] - tflops) < 0.2 and r["unit"] == "TFLOP/s"


def test_expert_ffn_bytes_match_the_record_layouts():
    """The per-expert bytes the decode roofline counts are the record's
    sections: W13 plus its tables for the up launch, W_d plus its tables for
    the down launch; together they are the record's payload."""
    b = _bench_module()
    import expert_weight_paging_amd as ewp
    H, I = 2048, 768
    for fmt in range(5):
        up, dn = b.expert_ffn_bytes(fmt, H, I)
        rec = ewp.record_bytes(fmt, H, I)
        assert up + dn <= rec < up + dn + 256, fmt  # the stride pads the payload to 256 bytes
    assert b.expert_ffn_bytes(1, H, I) == (6291456, 3145728)
    assert b.expert_ffn_bytes(3, H, I) == (1671168, 835584)
