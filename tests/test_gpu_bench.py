"""bench.py on the tiny fp32 decode, as a child process: the JSON line keeps
its contract (the keys, one GPU, the roofline object), both with eager calls
and with the timed steps replayed from one captured HIP graph (--graph, which
also checks the replay's output against the same call made eagerly)."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KEYS = {"metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
        "scaling", "vs_baseline", "dtype", "data", "config", "roofline"}


@pytest.mark.parametrize("graph", [False, True], ids=["eager", "graph"])
def test_bench_line_tiny_decode(graph):
    cmd = [sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--workload", "tiny_decode",
           "--steps", "20", "--warmup", "5", "--no-cpu-baseline", "--no-extras"]
    if graph:
        cmd.append("--graph")
    print(f"[bench] {' '.join(cmd[2:])}", flush=True)
    r = subprocess.run(cmd, cwd=ROOT, capture_output=True, text=True, timeout=100)
    assert r.returncode == 0, r.stderr[-2000:]
    rec = json.loads(r.stdout.strip().splitlines()[-1])
    assert KEYS <= rec.keys(), KEYS - rec.keys()
    assert rec["n_gpus"] == 1 and rec["steps"] == 20 and rec["warmup"] == 5
    assert rec["value"] > 0 and rec["ms_per_step"] > 0 and rec["higher_is_better"] is True
    assert rec["config"]["workload"] == "tiny_decode"
    assert rec["config"]["launch"] == ("graph replay" if graph else "eager calls")
    roof = rec["roofline"]
    assert roof["bound"] == "hbm" and roof["peak"] == 8000.0 and roof["unit"] == "GB/s"
    assert roof["achieved"] > 0 and abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
