"""bench.py's output contract, on the GPU (a short run in a child process).

The benchmark prints one JSON line: the headline metric and its roofline
object, the decode and 128K-history sub-objects, and (when not skipped) the
measured ceilings with each roofline's fraction of them.
"""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
pytestmark = pytest.mark.gpu


def test_bench_json_contract():
    print("[case] bench.py --steps 2 --warmup 1 --no-reports --no-cpu", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "2", "--warmup", "1",
                        "--no-reports", "--no-cpu"], capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
              "scaling", "vs_baseline", "dtype", "data", "config", "roofline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 2 and d["warmup"] == 1 and d["unit"] == "TFLOP/s"
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["vs_baseline"] is None
    rl = d["roofline"]
    assert rl["bound"] == "mfma" and rl["peak"] == 2500.0 and rl["unit"] == "TFLOP/s"
    assert abs(rl["frac"] - rl["achieved"] / rl["peak"]) < 1e-3
    assert 0 < rl["frac"] < 1
    assert d["decode"]["roofline"]["bound"] == "hbm" and 0 < d["decode"]["roofline"]["frac"] < 1
    mp = d["measured_peaks"]
    assert 1000 < mp["mfma_bf16_TFLOP/s"] < 2600 and 3000 < mp["hbm_read_GB/s"] < 8000
    assert abs(rl["frac_of_measured"] - rl["achieved"] / mp["mfma_bf16_TFLOP/s"]) < 1e-3

