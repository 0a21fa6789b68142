"""Host-side checks of bench.py: the one-GPU guard, and the oracle baseline
leg on a tiny workload (inputs drawn on the CPU)."""
import os
import subprocess
import sys

import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_cpu_baseline_record():
    sys.path.insert(0, ROOT)
    import bench
    from ssm_inputs import configs, generate

    cfg = configs.TINY_FP32
    rec = bench.cpu_baseline(torch, generate, cfg, target_s=0.05, dev="cpu")
    assert rec["kind"] == "oracle" and rec["unit"] == "elems/s"
    assert rec["value"] > 0 and rec["cores"] >= 1
    assert rec["sample"].startswith(cfg.name)
    assert rec["one_thread"]["value"] > 0
