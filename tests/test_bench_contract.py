"""bench.py's output contract: exactly one JSON line on stdout with the keys and types the
benchmark record needs (the roofline and CPU-baseline objects included), consistent
figures, and --gpus above 1 refused with a message (this build measures one GPU).  The GPU
case runs the launch-bound tiny workload in a child process, so it takes seconds."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(args, timeout):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, cwd=ROOT,
                          capture_output=True, text=True, timeout=timeout)


def test_more_than_one_gpu_is_refused():
    r = _bench(["--gpus", "2"], 300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus 2" in r.stderr
    assert not [l for l in r.stdout.splitlines() if l.startswith("{")]


@pytest.mark.gpu
def test_one_json_line_with_the_record_keys():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    r = _bench(["--workload", "c1_tiny", "--steps", "50", "--warmup", "2", "--settle-ms", "10",
                "--cpu-seconds", "1", "--probe-mib", "0"], 600)
    assert r.returncode == 0, r.stderr[-3000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    kinds = {"metric": str, "value": float, "unit": str, "n_gpus": int, "steps": int,
             "warmup": int, "ms_per_step": float, "higher_is_better": bool, "scaling": str,
             "dtype": str, "data": str, "config": dict, "roofline": dict, "cpu_baseline": dict}
    for k, t in kinds.items():
        assert isinstance(d[k], t), (k, d[k])
    assert "vs_baseline" in d and d["vs_baseline"] is None
    assert d["n_gpus"] == 1 and d["steps"] == 50 and d["warmup"] == 2
    assert d["higher_is_better"] is True and d["scaling"] in ("weak", "strong")
    assert d["value"] > 0 and abs(d["value"] * d["ms_per_step"] / 1e3 - 1.0) < 1e-2
    assert d["unit"] == "steps/s" and d["data"] == "synthetic"
    assert d["config"]["workload"].startswith("c1_tiny")
    assert d["config"]["status"] == 0
    rl = d["roofline"]
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in rl, k
    assert rl["bound"] == "hbm" and rl["unit"] == "GB/s" and rl["peak"] == 8000.0
    assert rl["launches_timed"] >= 50 and rl["avg_launch_us"] > 0
    assert rl["read_ceiling"] is None            # the tiny shape reads a few bytes
    cb = d["cpu_baseline"]
    for k in ("value", "unit", "cores", "kind", "sample"):
        assert k in cb, k
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1
