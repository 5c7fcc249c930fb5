"""bench.py's one-line JSON report, for every path it measures: the fields and types the
report promises (metric, value, unit, the step counts, the roofline entry, the workload),
on short runs (2 timed steps, 1 warm-up, no CPU baseline) of small configurations where
one exists.  Each run is a child process, one after the other."""
import json
import os
import subprocess
import sys

import pytest

from tests._gpu import say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CASES = [
    ["--config", "C3"],
    ["--config", "C1"],
    ["--config", "X1"],
    ["--op", "bwd", "--config", "C1"],
    ["--op", "merge"],
    ["--op", "qkv", "--config", "C1"],
    ["--op", "sparse", "--config", "C1"],
    ["--op", "fp8pv", "--config", "C1"],
    ["--op", "fps", "--config", "C1"],
]


@pytest.mark.parametrize("extra", CASES, ids=lambda c: " ".join(c))
def test_bench_line_fields(extra):
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "2", "--warmup", "1",
           "--no-cpu-baseline"] + extra
    say("[gpu] bench " + " ".join(extra))
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert res.returncode == 0, res.stdout[-2000:] + res.stderr[-2000:]
    lines = [ln for ln in res.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1, res.stdout[-2000:]
    rec = json.loads(lines[0])
    for key, typ in (("metric", str), ("value", (int, float)), ("unit", str), ("n_gpus", int),
                     ("steps", int), ("warmup", int), ("ms_per_step", (int, float)),
                     ("higher_is_better", bool), ("scaling", str), ("dtype", str), ("data", str),
                     ("config", dict), ("roofline", dict)):
        assert isinstance(rec.get(key), typ), (key, rec.get(key))
    assert "vs_baseline" in rec
    assert rec["n_gpus"] == 1 and rec["steps"] == 2 and rec["warmup"] == 1
    assert rec["value"] > 0 and rec["ms_per_step"] > 0
    assert isinstance(rec["config"].get("workload"), str) and rec["config"]["workload"]
    roof = rec["roofline"]
    assert roof["bound"] in ("hbm", "mfma", "alu")
    assert roof["unit"] in ("GB/s", "TFLOP/s")
    assert roof["achieved"] > 0 and roof["peak"] > 0
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 2e-3
    assert roof["traffic"] is None or roof["traffic"] > 0
    say(f"   value {rec['value']} {rec['unit']}, roofline {roof['achieved']} / {roof['peak']} {roof['unit']}")


def test_default_warmup_is_resolved_from_the_step_time():
    """Without --warmup the warm-up count is resolved to at least 0.15 s of GPU work (at
    least 50 launches), so the timed steps run at the settled clock; the line reports it."""
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "2", "--no-cpu-baseline",
           "--config", "C1"]
    say("[gpu] bench --config C1, default warm-up")
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert res.returncode == 0, res.stdout[-2000:] + res.stderr[-2000:]
    rec = json.loads([ln for ln in res.stdout.splitlines() if ln.startswith("{")][-1])
    kernel_ms = rec["roofline"]["kernel_ms"]
    assert rec["warmup"] >= 50
    # a C1 launch takes ~12 us, so 0.15 s of work is thousands of launches
    assert rec["warmup"] * kernel_ms >= 0.1 * 150.0, (rec["warmup"], kernel_ms)
    say(f"   warm-up {rec['warmup']} launches of {kernel_ms:.4f} ms")
