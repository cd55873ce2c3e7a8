"""bench.py's output contract: one JSON line with the required fields (GPU),
and the refusal of more than one GPU (CPU, before anything touches a GPU)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
REQUIRED = {"metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
            "vs_baseline", "dtype", "data", "config", "roofline"}
ROOFLINE = {"bound", "achieved", "peak", "unit", "frac", "traffic"}


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120, cwd=ROOT)
    assert r.returncode != 0
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


@pytest.mark.gpu
def test_bench_prints_one_json_line_with_the_contract_fields():
    print("[case] bench.py --steps 1 --warmup 0 --no-cpu-baseline", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "1", "--warmup", "0",
                        "--no-cpu-baseline"], capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.strip().splitlines() if l.strip()]
    assert len(lines) == 1, lines
    d = json.loads(lines[0])
    assert REQUIRED <= set(d), REQUIRED - set(d)
    assert ROOFLINE <= set(d["roofline"]), ROOFLINE - set(d["roofline"])
    assert d["n_gpus"] == 1 and d["steps"] == 1 and d["warmup"] == 0
    assert d["value"] > 0 and d["ms_per_step"] > 0
    assert 0 < d["roofline"]["frac"] < 1
    assert d["config"]["workload"].startswith("sdxl_3840")
    # one patch's GN -> conv -> splice -> attention, by events from one attention's end to the next's: patches
    # 1 .. 7 of the step
    pl = d["patch_layer_step_ms"]
    assert pl["samples"] == 7 and 0 < pl["p10"] <= pl["median"] <= pl["p90"] < d["ms_per_step"]
