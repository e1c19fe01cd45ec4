"""Host-side checks of the benchmark's contract (no GPU): a run asked for more
than one GPU exits with a JSON line that says so, and the CPU-oracle baseline
returns the fields the benchmark line carries."""

import json
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_cpu_baseline_fields():
    sys.path.insert(0, ROOT)
    import bench
    from workloads import bf16_bits_from_f32
    rng = np.random.default_rng(0)
    xb = bf16_bits_from_f32(rng.standard_normal((128, 256)).astype(np.float32))
    w = (rng.standard_normal((2048, 256)) * 0.02).astype(np.float32)
    out = bench.cpu_baseline(xb, w, 0.02, lambda *a: None)
    assert out["kind"] == "oracle" and out["unit"] == "TFLOP/s"
    assert out["value"] > 0
    assert out["cores"] == len(os.sched_getaffinity(0))
    assert "64 of the 128 rows" in out["sample"] and "1024 of the 2048 output channels" in out["sample"]
