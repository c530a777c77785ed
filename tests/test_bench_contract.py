"""bench.py keeps its output contract: one JSON line with the fields the measurement reads.

The one-GPU check runs on the CPU; the short run needs the GPU and the built library."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


@pytest.mark.gpu
def test_short_run_prints_one_json_line_with_the_contract_fields():
    r = subprocess.run([sys.executable, BENCH, "--steps", "3", "--warmup", "1", "--parts", "4",
                        "--cpu-seconds", "0.5", "--preroll-ms", "50"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, lines
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0
    assert d["config"]["workload"] == "modernbert_global_long"
    assert d["config"]["preroll"]["steps"] >= 1
    roof = d["roofline"]
    assert roof["bound"] == "mfma" and roof["peak"] == 157.3 and roof["unit"] == "TFLOP/s"
    assert 0 < roof["frac"] < 1
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    # the headline's value and its kernel's time agree: the tile kernel is most of the step
    assert roof["mean_launch_ms"] < d["ms_per_step"]
    base = d["cpu_baseline"]
    assert base["kind"] == "oracle" and base["value"] > 0 and base["cores"] >= 1
    ctx = d["pages_cpu_context"]
    assert ctx["masked_fill_ms_per_layer"]["value"] == 114.13
    assert ctx["kv_cat_ms_per_decode_token"]["value"] == 14.0
    dec = d["parts"]["decode_b64"]
    assert dec["decode_ms"] > 0 and dec["back_to_back_ms"] > 0 and dec["flushed_loop_ms"] > 0
    assert 0 < dec["frac_hbm"] < 1 and 0 < dec["back_to_back_frac_hbm"] < 1
    # each part is timed after a pre-roll of its own calls
    assert dec["preroll"]["calls"] >= 1 and dec["preroll"]["ms"] >= 100.0
