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


def test_scan_record_fields():
    """The headline roofline carries the VALU-issue figure and the HBM
    fractions of the dominant kernel and of the whole step (algorithmic bytes
    over time against 8 TB/s)."""
    sys.path.insert(0, ROOT)
    import bench
    from ssm_inputs import configs, generate

    cfg = configs.MAMBA2P8B_LAYER
    kern = {"scan_output": {"avg_ms": 0.5}, "scan_aggregate": {"avg_ms": 0.4}}
    roof, hbm, cfgd, kms, proto = bench.scan_record(cfg, 1.0, kern, 64, 256, generate,
                                                    proto={"flushed_median_ms": 1.1})
    alg = generate.alg_bytes_scan(cfg)
    assert roof["bound"] == "alu" and roof["unit"] == "TFLOP/s"
    assert abs(roof["hbm_frac_kernel"] - alg / 0.5e-3 / 8e12) < 1e-4
    assert abs(roof["hbm_frac_step"] - alg / 1.0e-3 / 8e12) < 1e-4
    assert abs(roof["achieved"] - cfg.elems() * bench.SCAN_FLOPS_PER_ELEM / 0.5e-3 / 1e12) < 1e-2
    # the published fp32 vector peak of MI355X, not the single-issue rate
    assert abs(roof["peak"] - 157.29) < 0.01
    assert abs(roof["frac"] - roof["achieved"] / 157.286) < 1e-3
    # one wave-step = one step of one 64-channel tile: 4 x 80 x 16384 of them
    assert abs(roof["cycles_per_wave_step_per_simd"] - 0.5e-3 * 2.4e9 * 1024 / (4 * 80 * 16384)) < 0.1
    assert hbm["algorithmic_bytes"] == alg and cfgd["segments"] == 64
    assert proto["flushed_median_elems_per_s"] > 0


def test_rotation_and_backward_bytes():
    sys.path.insert(0, ROOT)
    import bench
    from ssm_inputs import configs

    assert bench.rotation_count(2_000_000_000) == 1
    assert bench.rotation_count(150_000_000) == 8       # >= 4 x the 256 MiB cache
    b = bench.alg_bytes_bwd(configs.MAMBA2P8B_LAYER)
    assert 3.3e9 < b < 3.5e9                            # x, delta, dy read; dx, ddelta written; dB, dC
    # packed: the same per-step arrays for one row of 65536 steps, plus three
    # [nseq][Dm][N] fp32 state rows (h_init, dh_final, dh_init) and the offsets
    pc = configs.PACKED_2P8B_LAYER
    bp = bench.alg_bytes_bwd_packed(pc, 40)
    assert bp == (5 * 65536 * 5120 * 2 + 2 * 65536 * 16 * 2 + 2 * 65536 * 16 * 4 + 2 * 5120 * 16 * 4 + 2 * 5120 * 4
                  + 3 * 40 * 5120 * 16 * 4 + 8 * 41)
