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
    assert mode("decode-fp8", batch=6) == (False, False)     # 48 > 40: host-driven waves
    assert mode("decode-fp8", batch=4, slots=24) == (False, False)
    assert mode("decode-bf16", host=True) == (False, False)
    assert mode("stack-int4") == (False, True)
    assert mode("stack-int4", lookahead=True) == (False, False)
    assert mode("prefill-bf16") == (False, False)
