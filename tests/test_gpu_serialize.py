"""Race check ([PE] "Can paging change the model's outputs?": paging mistakes
are silent): the same sequence of steps on streams that could race (copies
on a copy stream, routing on a route stream, lookahead across layers) run
once normally and once with the HIP runtime serialising every kernel and
every copy (AMD_SERIALIZE_KERNEL=3, AMD_SERIALIZE_COPY=3) must give the same
plans, table states and outputs, bit for bit. Each run is a child process
(the variables are read when the runtime starts)."""
import os
import subprocess
import sys

import numpy as np
import pytest

from gpu_harness import say

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


def _run(path, serialise):
    env = dict(os.environ)
    if serialise:
        env["AMD_SERIALIZE_KERNEL"] = "3"
        env["AMD_SERIALIZE_COPY"] = "3"
    else:
        env.pop("AMD_SERIALIZE_KERNEL", None)
        env.pop("AMD_SERIALIZE_COPY", None)
    r = subprocess.run([sys.executable, "-u", os.path.join(HERE, "serialize_run.py"), path], env=env,
                       capture_output=True, text=True, timeout=280)
    say(r.stdout.strip()[-300:])
    assert r.returncode == 0, r.stderr[-2000:]


@pytest.mark.timeout(600)
def test_serialised_run_equals_async_run(tmp_path):
    say("case: decode on 3 streams, host and device stacks with lookahead; async vs serialised")
    a, b = str(tmp_path / "async.npz"), str(tmp_path / "serial.npz")
    _run(a, False)
    _run(b, True)
    A, B = np.load(a), np.load(b)
    assert sorted(A.files) == sorted(B.files) and len(A.files) > 100
    diff = [k for k in A.files if not np.array_equal(A[k], B[k])]
    assert not diff, diff[:10]
