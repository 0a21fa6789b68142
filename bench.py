#!/usr/bin/env python3
"""Throughput benchmark of libssmscan on one MI355X.

A step is one selective-scan forward (B/C prep, segment aggregate, carry and
output kernels) over the Mamba-2.8B-shaped layer: Bsz=4, L=16384, D=5120,
N=16, bf16 storage, fp32 arithmetic, synthetic seeded inputs resident in HBM.
The JSON line reports elements/s (B*L*D*N per second), the achieved
algorithmic HBM bandwidth, the roofline of the dominant kernel, the fp64 CPU
oracle timed on a bounded sample of the same workload, and -- under
"secondary" -- the long-context scan, the scan options (fused delta
activation, Euler input term), a packed variable-length prefill, the scan
with complex A, the backward, the general-A path forced on the same layer,
the scalar-decay (state-space duality) layer and the decode step.  A measured device-copy rate is reported beside the
8 TB/s specification.

    python bench.py [--gpus 1] [--steps 50] [--warmup 5]
                    [--no-cpu-baseline] [--no-secondary]
    python bench.py --only decode      # one workload, for profiler runs
                                       # (scan, long, small, packed, options, backward,
                                       #  complex, general, ssd, decode)
    python bench.py --copy-calibration # plain copy of known size (for counters)
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "selective-scan elems/s (B·L·D·N) + achieved HBM GB/s vs MI355X peak"
HBM_PEAK_GBPS = 8000.0
# Non-packed fp32 FMA issue rate: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz x 2 flops.
VALU_FP32_PEAK_TFLOPS = 256 * 4 * 16 * 2.4e9 * 2 / 1e12
# Dense bf16 matrix-core peak of MI355X (no sparsity).
BF16_MFMA_PEAK_TFLOPS = 2500.0
# Algorithmic fp32 flops per state element of the scan: z = delta*A, exp(z)-1,
# divide by A, times B, times x, Abar*h + Bbar*x (FMA, 2), C*h + y (FMA, 2).
SCAN_FLOPS_PER_ELEM = 9
# Backward, per state element: the adjoint step mu = C dy + nu, (1 + E) mu and
# the six gradient terms (dx, dDelta, two for dA, dB, dC lane values: 20), the
# channel sums of dB and dC (2), and one forward recurrence for the states
# (exp-chain, input and update FMAs: 6).
BWD_FLOPS_PER_ELEM = 28
# Complex A, per state element of the output pass: delta*a, delta*w (2); exp,
# sin, cos (3, one each); Abar (2); Abar - 1 (3); (Abar - 1)/A (complex
# multiply, 6); B x and its product with it (3); Abar h + k u (8); C Re(h) + y (2).
CPLX_FLOPS_PER_ELEM = 29
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SRC = os.path.join(ROOT, "selective_state_space_18_amd", "csrc")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# Sources each measured kernel is built from: a counter figure is reported
# only while all of them are unchanged.
KERNEL_SOURCES = {
    "scan": ("scan_kernels.h", "ssm_device.h", "ssm_launch.h"),
    "step": ("step_kernel.hip", "ssm_device.h", "ssm_launch.h"),
    "bwd": ("bwd_kernels.h", "scan_kernels.h", "ssm_device.h", "ssm_launch.h"),
    "ssd": ("ssd_kernels.h", "ssm_device.h", "ssm_launch.h"),
}


def source_sha(kind):
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kind]:
        with open(os.path.join(KERNEL_SRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(kernel, kind):
    """HBM bytes per launch measured with counters, if the kernel is unchanged."""
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(kernel)
    if not rec or rec.get("source_sha") != source_sha(kind):
        return None
    return rec.get("hbm_bytes_per_launch")


def timed_loop(torch, fn, steps, warmup):
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(st)
    for i in range(steps):
        fn(warmup + i)
    b.record(st)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def bench_scan(torch, ss, generate, cfg, steps, warmup, **opts):
    """opts: scan options (delta_bias is taken from the inputs when the
    workload's delta is the raw projection output)."""
    dev = "cuda:0"
    log(f"[bench] generating {cfg.name}")
    inp = generate.scan_inputs(cfg, dev)
    if "delta_bias" in inp:
        opts = dict(opts, delta_bias=inp["delta_bias"], delta_softplus=True)
    y = torch.empty_like(inp["x"])
    hf = torch.empty(cfg.Bsz, cfg.Dm, cfg.N, device=dev, dtype=torch.float32)

    def fn(_i):
        ss.scan_fwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], y=y, h_final=hf, **opts)

    log(f"[bench] timing {cfg.name} {sorted(k for k, v in opts.items() if v is not None and v is not False)}: "
        f"{warmup} warmup + {steps} steps")
    ms, kern = profiled_loop(torch, ss, fn, steps, warmup)
    S, seg = ss.plan(cfg.Bsz, cfg.L, cfg.Dm, cfg.N)
    del inp, y, hf
    torch.cuda.empty_cache()
    return ms, kern, S, seg


def bench_unfused_softplus(torch, ss, generate, cfg, steps, warmup):
    """For comparison only: the activation as a separate torch pass
    (softplus(delta + bias) written back to HBM in the storage dtype), then the
    plain scan.  Returns ms per step."""
    dev = "cuda:0"
    inp = generate.scan_inputs(cfg, dev)
    y = torch.empty_like(inp["x"])
    hf = torch.empty(cfg.Bsz, cfg.Dm, cfg.N, device=dev, dtype=torch.float32)
    act = torch.empty_like(inp["delta"])
    bias = inp["delta_bias"].to(inp["delta"].dtype)

    def fn(_i):
        torch.nn.functional.softplus(torch.add(inp["delta"], bias, out=act), out=act)
        ss.scan_fwd(inp["x"], act, inp["A"], inp["B"], inp["C"], inp["D"], y=y, h_final=hf)

    log(f"[bench] timing {cfg.name} with a separate softplus pass: {warmup} warmup + {steps} steps")
    ms = timed_loop(torch, fn, steps, warmup)
    del inp, y, hf, act
    torch.cuda.empty_cache()
    return ms


def profiled_loop(torch, ss, fn, steps, warmup):
    """Wall time per step of `steps` calls, then each kernel kind's average
    launch duration over the same number of calls with the library's
    per-kernel HIP-event timers on.  The event records add gaps between
    launches, so the wall time is taken with the timers off."""
    ms = timed_loop(torch, fn, steps, warmup)
    ss.set_option(ss.SSM_OPT_PROFILE, 1)
    ss.profile_read()
    try:
        timed_loop(torch, fn, steps, 0)
        prof = ss.profile_read()
    finally:
        ss.set_option(ss.SSM_OPT_PROFILE, 0)
    kern = {k: {"avg_ms": v[0] / v[1], "launches_per_step": v[1] / steps}
            for k, v in prof.items() if v[1] > 0}
    return ms, kern


def bench_options(torch, ss, generate, configs, steps):
    """The Mamba-2.8B-shaped layer with the scan options: delta's activation
    fused (softplus(delta + bias) inside the kernels), and the Euler input
    term, against the separate-activation route."""
    out = {}
    fc = configs.FUSED_2P8B_LAYER
    ms, kern, S, seg = bench_scan(torch, ss, generate, fc, steps, 2)
    roof, hbm, cfgd, kms = scan_record(fc, ms, kern, S, seg, generate)
    out["fused_softplus"] = {"workload": fc.name, "ms_per_step": round(ms, 5), "value": fc.elems() / (ms * 1e-3),
                             "unit": "elems/s", "hbm": hbm, "roofline": roof, "kernels_avg_ms": kms,
                             "config": dict(cfgd, delta="softplus(raw + bias) in the kernels")}
    ums = bench_unfused_softplus(torch, ss, generate, fc, steps, 2)
    out["separate_softplus_pass"] = {"ms_per_step": round(ums, 5), "value": fc.elems() / (ums * 1e-3),
                                     "note": "torch softplus pass over delta, then the plain scan"}
    ec = configs.MAMBA2P8B_LAYER
    ms, kern, S, seg = bench_scan(torch, ss, generate, ec, steps, 2, euler_b=True)
    roof, hbm, cfgd, kms = scan_record(ec, ms, kern, S, seg, generate)
    out["euler_b"] = {"workload": ec.name, "ms_per_step": round(ms, 5), "value": ec.elems() / (ms * 1e-3),
                      "unit": "elems/s", "hbm": hbm, "roofline": roof, "kernels_avg_ms": kms,
                      "config": dict(cfgd, input_term="Euler: delta * B")}
    return out


def bench_general_path(torch, ss, generate, cfg, steps):
    """The same layer with the structured-A fast path switched off, so every
    state element takes its own exponential (the path a layer with arbitrary
    real A runs)."""
    ss.set_option(ss.SSM_OPT_FORCE_GENERAL, 1)
    try:
        ms, kern, S, seg = bench_scan(torch, ss, generate, cfg, steps, 2)
    finally:
        ss.set_option(ss.SSM_OPT_FORCE_GENERAL, 0)
    roof, hbm, cfgd, kms = scan_record(cfg, ms, kern, S, seg, generate)
    roof["kernel"] = "scan_segment_kernel (output pass, general A)"
    roof["traffic"] = None  # the counter figures are the structured kernel's
    return {"workload": cfg.name, "ms_per_step": round(ms, 5), "value": cfg.elems() / (ms * 1e-3),
            "unit": "elems/s", "hbm": hbm, "roofline": roof, "kernels_avg_ms": kms,
            "config": dict(cfgd, A="general path forced (one exp per state element)")}


def bench_ssd(torch, ss, generate, cfg, steps, warmup):
    """The scalar-decay layer (heads of 64 channels sharing A and delta, N =
    128) in its chunked matrix form.  Algorithmic flops of the output pass per
    (b, t, d): 2N for C H, 2N for the state update B^T (w x), Q + 1 for the
    causal intra-chunk product (Q = 64 steps; the lower triangle of a Q x Q
    matrix times x), plus (Q + 1) N / Dm for the shared G = C B^T."""
    dev = "cuda:0"
    log(f"[bench] generating {cfg.name}")
    inp = generate.ssd_inputs(cfg, dev)
    y = torch.empty_like(inp["x"])
    hf = torch.empty((cfg.Bsz, cfg.Dm, cfg.N), dtype=torch.float32, device=dev)

    def fn(_i):
        ss.scan_ssd_fwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], cfg.head_dim, y=y, h_final=hf)

    log(f"[bench] timing {cfg.name}: {warmup} warmup + {steps} steps")
    ms, kern = profiled_loop(torch, ss, fn, steps, warmup)
    del inp, y, hf
    torch.cuda.empty_cache()
    Q = 64
    BLD = cfg.Bsz * cfg.L * cfg.Dm
    flops_out = BLD * (4 * cfg.N + (Q + 1) + (Q + 1) * cfg.N / cfg.Dm)
    out_ms = kern["ssd_output"]["avg_ms"]
    alg = generate.alg_bytes_ssd(cfg)
    mfma = flops_out / (out_ms * 1e-3) / 1e12
    return {"workload": cfg.name, "ms_per_step": round(ms, 5), "value": cfg.elems() / (ms * 1e-3),
            "unit": "elems/s",
            "hbm": {"achieved": round(alg / (ms * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4), "algorithmic_bytes": alg},
            "roofline": {"kernel": "ssd_chunk_kernel (output pass)", "bound": "mfma",
                         "achieved": round(mfma, 2), "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(mfma / BF16_MFMA_PEAK_TFLOPS, 4), "avg_ms": round(out_ms, 5),
                         "traffic": traffic_for("ssd_output_" + cfg.name, "ssd"),
                         "algorithmic_flops_per_launch": flops_out,
                         "hbm_frac_at_algorithmic_bytes": round(alg / (out_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)},
            "kernels_avg_ms": {k: round(v["avg_ms"], 5) for k, v in kern.items()},
            "config": {"workload": cfg.name, "Bsz": cfg.Bsz, "L": cfg.L, "Dm": cfg.Dm, "N": cfg.N,
                       "head_dim": cfg.head_dim, "storage": cfg.dtype,
                       "A": "one real scalar per head, -exp(N(0, 0.5))", "delta": "per head, " + cfg.delta_kind,
                       "input_term": "ZOH"}}


def bench_backward(torch, ss, generate, cfg, steps, warmup):
    """Backward of the scan over the layer: every input gradient for a random
    dy (and dh_final), forward states recomputed inside the call."""
    dev = "cuda:0"
    log(f"[bench] generating {cfg.name} (backward)")
    inp = generate.scan_inputs(cfg, dev)
    g = torch.Generator(device=dev)
    g.manual_seed(cfg.seed + 1)
    dy = torch.randn(inp["x"].shape, generator=g, device=dev).to(inp["x"].dtype)
    dhf = torch.randn((cfg.Bsz, cfg.Dm, cfg.N), generator=g, device=dev)
    out = {}

    def fn(_i):
        nonlocal out
        out = ss.scan_bwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], dy, dh_final=dhf,
                          out=out or None)

    log(f"[bench] timing {cfg.name} backward: {warmup} warmup + {steps} steps")
    ms, kern = profiled_loop(torch, ss, fn, steps, warmup)
    del inp, dy, dhf, out
    torch.cuda.empty_cache()
    elems = cfg.elems()
    main_ms = kern["bwd_main"]["avg_ms"]
    achieved = elems * BWD_FLOPS_PER_ELEM / (main_ms * 1e-3) / 1e12
    return {"workload": cfg.name, "ms_per_step": round(ms, 5), "value": elems / (ms * 1e-3), "unit": "elems/s",
            "roofline": {"kernel": "bwd_main_kernel", "bound": "alu", "achieved": round(achieved, 3),
                         "peak": round(VALU_FP32_PEAK_TFLOPS, 2), "unit": "TFLOP/s",
                         "frac": round(achieved / VALU_FP32_PEAK_TFLOPS, 4), "traffic": None,
                         "avg_ms": round(main_ms, 5), "algorithmic_flops_per_launch": elems * BWD_FLOPS_PER_ELEM},
            "kernels_avg_ms": {k: round(v["avg_ms"], 5) for k, v in kern.items()},
            "main_kernel_elems_per_s": elems / (main_ms * 1e-3)}


def bench_complex(torch, ss, generate, cfg, steps, warmup):
    """The layer with complex diagonal A (decaying oscillators): one exp and
    one sin/cos pair per state element; no structured fast path."""
    dev = "cuda:0"
    log(f"[bench] generating {cfg.name} (complex A)")
    inp = generate.scan_inputs(cfg, dev)
    A = generate.complex_A(cfg.Dm, cfg.N, cfg.seed + 100, dev)
    y = torch.empty_like(inp["x"])
    hf = torch.empty((cfg.Bsz, cfg.Dm, cfg.N), dtype=torch.complex64, device=dev)

    def fn(_i):
        ss.scan_complex_fwd(inp["x"], inp["delta"], A, inp["B"], inp["C"], inp["D"], y=y, h_final=hf)

    log(f"[bench] timing {cfg.name} complex: {warmup} warmup + {steps} steps")
    ms, kern = profiled_loop(torch, ss, fn, steps, warmup)
    del inp, A, y, hf
    torch.cuda.empty_cache()
    out_ms = kern["scan_output"]["avg_ms"]
    achieved = cfg.elems() * CPLX_FLOPS_PER_ELEM / (out_ms * 1e-3) / 1e12
    return {"workload": cfg.name + "_complex_A", "ms_per_step": round(ms, 5), "value": cfg.elems() / (ms * 1e-3),
            "unit": "elems/s",
            "roofline": {"kernel": "cplx_segment_kernel (output pass)", "bound": "alu", "achieved": round(achieved, 3),
                         "peak": round(VALU_FP32_PEAK_TFLOPS, 2), "unit": "TFLOP/s",
                         "frac": round(achieved / VALU_FP32_PEAK_TFLOPS, 4), "traffic": None,
                         "avg_ms": round(out_ms, 5), "algorithmic_flops_per_launch": cfg.elems() * CPLX_FLOPS_PER_ELEM,
                         "note": "exp, sin and cos count one flop each and issue at a quarter of the VALU rate"},
            "kernels_avg_ms": {k: round(v["avg_ms"], 5) for k, v in kern.items()}}


def bench_packed(torch, ss, generate, cfg, steps, warmup):
    """Packed variable-length prefill: one row of cfg.L steps holding a few
    dozen sequences, each restarting from its own initial state."""
    dev = "cuda:0"
    log(f"[bench] generating {cfg.name}")
    inp = generate.packed_inputs(cfg, dev)
    nseq = inp["cu"].numel() - 1
    y = torch.empty_like(inp["x"])
    hf = torch.empty(nseq, cfg.Dm, cfg.N, device=dev, dtype=torch.float32)

    def fn(_i):
        ss.scan_varlen_fwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["cu"],
                           h_init=inp["h_init"], y=y, h_final=hf)

    log(f"[bench] timing {cfg.name}: {warmup} warmup + {steps} steps")
    ms, kern = profiled_loop(torch, ss, fn, steps, warmup)
    S, seg = ss.plan(1, cfg.L, cfg.Dm, cfg.N)
    lens = (inp["cu"][1:] - inp["cu"][:-1]).tolist()
    del inp, y, hf
    torch.cuda.empty_cache()
    elems = cfg.elems()
    alg = generate.alg_bytes_varlen(cfg.L, cfg.Dm, cfg.N, nseq, cfg.dtype, cfg.h0_std > 0)
    out_ms = kern["scan_output"]["avg_ms"]
    achieved = elems * SCAN_FLOPS_PER_ELEM / (out_ms * 1e-3) / 1e12
    return {
        "workload": cfg.name, "ms_per_step": round(ms, 5), "value": elems / (ms * 1e-3), "unit": "elems/s",
        "config": {"workload": cfg.name, "L": cfg.L, "Dm": cfg.Dm, "N": cfg.N, "storage": cfg.dtype,
                   "A": cfg.a_kind, "sequences": nseq, "empty_sequences": lens.count(0),
                   "longest": max(lens), "segments": S, "segment_len": seg, "h_init": cfg.h0_std > 0},
        "hbm": {"achieved": round(alg / (ms * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4), "algorithmic_bytes": alg},
        "roofline": {"kernel": "scan_segment_kernel (output pass, packed)", "bound": "alu",
                     "achieved": round(achieved, 3), "peak": round(VALU_FP32_PEAK_TFLOPS, 2), "unit": "TFLOP/s",
                     "frac": round(achieved / VALU_FP32_PEAK_TFLOPS, 4),
                     "traffic": traffic_for("scan_output_" + cfg.name, "scan"),
                     "avg_ms": round(out_ms, 5)},
        "kernels_avg_ms": {k: round(v["avg_ms"], 5) for k, v in kern.items()},
    }


def scan_record(cfg, ms, kern, S, seg, generate):
    elems = cfg.elems()
    alg = generate.alg_bytes_scan(cfg)
    out_ms = kern["scan_output"]["avg_ms"]
    achieved = elems * SCAN_FLOPS_PER_ELEM / (out_ms * 1e-3) / 1e12
    roof = {
        "kernel": "scan_segment_kernel (output pass)",
        "bound": "alu",
        "achieved": round(achieved, 3),
        "peak": round(VALU_FP32_PEAK_TFLOPS, 2),
        "unit": "TFLOP/s",
        "frac": round(achieved / VALU_FP32_PEAK_TFLOPS, 4),
        "traffic": traffic_for("scan_output_" + cfg.name, "scan"),
        "avg_ms": round(out_ms, 5),
        "algorithmic_flops_per_launch": elems * SCAN_FLOPS_PER_ELEM,
        "hbm_frac_at_algorithmic_bytes": round(alg / (out_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
    }
    hbm = {"achieved": round(alg / (ms * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
           "frac": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4), "algorithmic_bytes": alg}
    cfgd = {"workload": cfg.name, "Bsz": cfg.Bsz, "L": cfg.L, "Dm": cfg.Dm, "N": cfg.N,
            "storage": cfg.dtype, "A": cfg.a_kind, "delta": cfg.delta_kind,
            "segments": S, "segment_len": seg}
    return roof, hbm, cfgd, {k: round(v["avg_ms"], 5) for k, v in kern.items()}


def bench_decode(torch, ss, generate, cfg, n_tokens, layers=4):
    """n_tokens consecutive steps; the resident state cycles over `layers`
    independent layer states so the working set (layers x 134 MB) exceeds the
    256 MB last-level cache, as in a multi-layer model."""
    dev = "cuda:0"
    log(f"[bench] generating {cfg.name} ({layers} layer states)")
    states = [generate.step_state(cfg, dev, seed=cfg.seed + 17 * k) for k in range(layers)]
    toks = generate.step_tokens(cfg, states[0], 16)
    y = torch.empty(cfg.Bsz, cfg.Dm, dtype=toks[0]["x"].dtype, device=dev)

    def fn(i):
        st = states[i % layers]
        t = toks[i % 16]
        ss.step(t["x"], t["delta"], st["A"], t["B"], t["C"], st["D"], st["h"], y=y)

    log(f"[bench] timing {cfg.name}: {n_tokens} steps")
    ms, kern = profiled_loop(torch, ss, fn, n_tokens, 16)
    k_ms = kern["step"]["avg_ms"]
    alg = generate.alg_bytes_step(cfg)
    # The same steps replayed from a captured HIP graph (a decode loop of a
    # serving engine): removes the host launch gap between steps.
    graph_ms = None
    try:
        per_graph = 16 * layers // 4
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            fn(0)
        s.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for i in range(per_graph):
                fn(i)
        reps = max(1, n_tokens // per_graph)
        g.replay()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        graph_ms = a.elapsed_time(b) / (reps * per_graph)
        del g
    except Exception as e:  # graph capture is an extra figure, never the value
        log(f"[bench] decode graph timing skipped: {e}")
    del states, toks, y
    torch.cuda.empty_cache()
    return {
        "workload": cfg.name, "steps": n_tokens, "ms_per_step": round(ms, 5),
        "value": cfg.elems_per_step() / (ms * 1e-3), "unit": "elems/s",
        "hbm": {"achieved": round(alg / (ms * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4), "algorithmic_bytes": alg},
        "roofline": {"kernel": "step_kernel", "bound": "hbm",
                     "achieved": round(alg / (k_ms * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(alg / (k_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                     "traffic": traffic_for("step_" + cfg.name, "step"),
                     "avg_ms": round(k_ms, 5)},
        "state_layers_cycled": layers,
        "graph_ms_per_step": None if graph_ms is None else round(graph_ms, 5),
        "graph_value": None if graph_ms is None else cfg.elems_per_step() / (graph_ms * 1e-3),
    }


def bench_complex_decode(torch, ss, generate, cfg, n_tokens, layers=4):
    """The decode workload with complex A and a complex state (2 x 134 MB per
    layer), cycling over `layers` layer states as bench_decode does."""
    dev = "cuda:0"
    log(f"[bench] generating {cfg.name} with complex A ({layers} layer states)")
    states = [generate.step_state_complex(cfg, dev, seed=cfg.seed + 17 * k) for k in range(layers)]
    toks = generate.step_tokens(cfg, states[0], 16)
    y = torch.empty(cfg.Bsz, cfg.Dm, dtype=toks[0]["x"].dtype, device=dev)

    def fn(i):
        st = states[i % layers]
        t = toks[i % 16]
        ss.step_complex(t["x"], t["delta"], st["A"], t["B"], t["C"], st["D"], st["h"], y=y)

    log(f"[bench] timing {cfg.name} (complex A): {n_tokens} steps")
    ms, kern = profiled_loop(torch, ss, fn, n_tokens, 16)
    k_ms = kern["step"]["avg_ms"]
    alg = generate.alg_bytes_step_complex(cfg)
    del states, toks, y
    torch.cuda.empty_cache()
    return {
        "workload": cfg.name + "_complex_A", "steps": n_tokens, "ms_per_step": round(ms, 5),
        "value": cfg.elems_per_step() / (ms * 1e-3), "unit": "elems/s",
        "hbm": {"achieved": round(alg / (ms * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4), "algorithmic_bytes": alg},
        "roofline": {"kernel": "cplx_step_kernel", "bound": "hbm",
                     "achieved": round(alg / (k_ms * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(alg / (k_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4), "traffic": None,
                     "avg_ms": round(k_ms, 5)},
        "state_layers_cycled": layers,
    }


def cpu_baseline(torch, generate, cfg, target_s=10.0, dev="cuda:0"):
    """The fp64 oracle on a channel subset of the same workload (channels are
    independent, so a subset is the same work per element).  The inputs are
    drawn on `dev` as for the GPU run and copied to the host."""
    import numpy as np
    import oracle

    threads = len(os.sched_getaffinity(0))
    inp = generate.scan_inputs(cfg, dev)

    def run(nch, nthreads=threads):
        stride = max(1, cfg.Dm // nch)
        idx = torch.arange(0, cfg.Dm, stride, device=dev)[:nch]
        f = lambda t: t.detach().to("cpu").to(torch.float64).numpy()
        args = (f(inp["x"].index_select(2, idx)), f(inp["delta"].index_select(2, idx)),
                f(inp["A"].index_select(0, idx)), f(inp["B"]), f(inp["C"]), f(inp["D"].index_select(0, idx)))
        t0 = time.perf_counter()
        oracle.scan(*args, threads=nthreads)
        return time.perf_counter() - t0, len(idx)

    probe_ch = min(cfg.Dm, 2 * threads)
    dt, n = run(probe_ch)
    rate = cfg.Bsz * cfg.L * n * cfg.N / dt
    nch = int(min(cfg.Dm, max(probe_ch, target_s * rate / (cfg.Bsz * cfg.L * cfg.N))))
    dt, n = run(nch)
    elems = cfg.Bsz * cfg.L * n * cfg.N
    # one thread on 64 channels (about a second), for the per-core rate
    dt1, n1 = run(min(cfg.Dm, 64), nthreads=1)
    del inp
    torch.cuda.empty_cache()
    _ = np
    return {"value": elems / dt, "unit": "elems/s", "cores": threads, "kind": "oracle",
            "sample": f"{cfg.name}: all {cfg.Bsz} rows x {cfg.L} steps, {n} of {cfg.Dm} channels "
                      f"(every {max(1, cfg.Dm // nch)}th), fp64, {dt:.1f} s wall",
            "one_thread": {"value": cfg.Bsz * cfg.L * n1 * cfg.N / dt1, "unit": "elems/s",
                           "sample": f"{n1} channels, all rows and steps, {dt1:.1f} s wall"}}


def copy_peak(torch, nbytes=1 << 30, reps=10):
    """Device-to-device copy rate (bytes read + bytes written per second) of
    a plain torch copy: the practical HBM ceiling on this GPU, reported beside
    the 8 TB/s specification."""
    x = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    y = torch.empty_like(x)
    ms = timed_loop(torch, lambda _i: y.copy_(x), reps, 2)
    del x, y
    torch.cuda.empty_cache()
    return {"achieved": round(2 * nbytes / (ms * 1e-3) / 1e9, 1), "unit": "GB/s",
            "what": f"torch copy of {nbytes >> 20} MiB, read + write bytes"}


def copy_calibration(torch, nbytes=1 << 30):
    """A plain device copy of known size, for scaling HBM byte counters."""
    x = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    log(f"[bench] copied {nbytes} bytes 3 times")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--only", choices=["scan", "long", "decode", "small", "packed", "options", "backward",
                                       "complex", "cdecode", "general", "ssd"],
                    default=None)
    ap.add_argument("--copy-calibration", action="store_true")
    a = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the scan shards over (batch, channel) with no "
              f"exchange, so there is no multi-GPU path to time (asked for --gpus {a.gpus}, "
              f"WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)

    import torch
    from selective_state_space_18_amd import ssmscan as ss
    from ssm_inputs import configs, generate

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    ss.lib()
    torch.cuda.set_device(0)

    if a.copy_calibration:
        copy_calibration(torch)
        return

    if a.only == "decode":
        rec = bench_decode(torch, ss, generate, configs.DECODE_256x8192, a.steps)
        print(json.dumps(rec), flush=True)
        return
    if a.only == "cdecode":
        rec = bench_complex_decode(torch, ss, generate, configs.DECODE_256x8192, a.steps)
        print(json.dumps(rec), flush=True)
        return
    if a.only == "complex":
        rec = bench_complex(torch, ss, generate, configs.MAMBA2P8B_LAYER, a.steps, a.warmup)
        print(json.dumps(rec), flush=True)
        return
    if a.only == "ssd":
        rec = bench_ssd(torch, ss, generate, configs.SSD_LAYER, a.steps, a.warmup)
        print(json.dumps(rec), flush=True)
        return
    if a.only == "general":
        rec = bench_general_path(torch, ss, generate, configs.MAMBA2P8B_LAYER, a.steps)
        print(json.dumps(rec), flush=True)
        return
    if a.only == "backward":
        rec = bench_backward(torch, ss, generate, configs.MAMBA2P8B_LAYER, a.steps, a.warmup)
        print(json.dumps(rec), flush=True)
        return
    if a.only == "options":
        print(json.dumps(bench_options(torch, ss, generate, configs, a.steps)), flush=True)
        return
    if a.only == "packed":
        rec = bench_packed(torch, ss, generate, configs.PACKED_2P8B_LAYER, a.steps, a.warmup)
        print(json.dumps(rec), flush=True)
        return
    if a.only == "long":
        cfg = configs.LONG_CONTEXT_1M
        ms, kern, S, seg = bench_scan(torch, ss, generate, cfg, a.steps, a.warmup)
        roof, hbm, cfgd, kms = scan_record(cfg, ms, kern, S, seg, generate)
        print(json.dumps({"workload": cfg.name, "ms_per_step": ms, "value": cfg.elems() / (ms * 1e-3),
                          "hbm": hbm, "roofline": roof, "kernels_avg_ms": kms}), flush=True)
        return
    if a.only == "small":
        cfg = configs.MAMBA130M_LAYER
        ms, kern, S, seg = bench_scan(torch, ss, generate, cfg, a.steps, a.warmup)
        roof, hbm, cfgd, kms = scan_record(cfg, ms, kern, S, seg, generate)
        print(json.dumps({"workload": cfg.name, "ms_per_step": ms, "value": cfg.elems() / (ms * 1e-3),
                          "hbm": hbm, "roofline": roof, "kernels_avg_ms": kms}), flush=True)
        return

    cfg = configs.MAMBA2P8B_LAYER
    ms, kern, S, seg = bench_scan(torch, ss, generate, cfg, a.steps, a.warmup)
    roof, hbm, cfgd, kms = scan_record(cfg, ms, kern, S, seg, generate)
    out = {
        "metric": METRIC,
        "value": cfg.elems() / (ms * 1e-3),
        "unit": "elems/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": cfgd,
        "hbm": hbm,
        "roofline": roof,
        "kernels_avg_ms": kms,
    }
    if a.only is None and not a.no_secondary:
        sec = {}
        lc = configs.LONG_CONTEXT_1M
        lms, lk, lS, lseg = bench_scan(torch, ss, generate, lc, max(3, a.steps // 5), 2)
        lroof, lhbm, lcfg, lkms = scan_record(lc, lms, lk, lS, lseg, generate)
        sec["long_context"] = {"workload": lc.name, "ms_per_step": round(lms, 5),
                               "value": lc.elems() / (lms * 1e-3), "unit": "elems/s", "hbm": lhbm,
                               "roofline": lroof, "config": lcfg, "kernels_avg_ms": lkms}
        sm = configs.MAMBA130M_LAYER
        sms, sk, sS, sseg = bench_scan(torch, ss, generate, sm, a.steps, a.warmup)
        sroof, shbm, scfg, skms = scan_record(sm, sms, sk, sS, sseg, generate)
        sec["mamba130m_layer"] = {
            "workload": sm.name, "ms_per_step": round(sms, 5), "value": sm.elems() / (sms * 1e-3),
            "unit": "elems/s", "hbm": shbm, "roofline": sroof, "config": scfg, "kernels_avg_ms": skms,
            "note": "random A: every state element takes its own exp (general path); the 153 MB working "
                    "set stays in the 256 MB last-level cache between calls"}
        sec["fused_softplus"] = bench_options(torch, ss, generate, configs, max(5, a.steps // 5))
        sec["packed_prefill"] = bench_packed(torch, ss, generate, configs.PACKED_2P8B_LAYER,
                                             max(5, a.steps // 5), 2)
        sec["complex_A"] = bench_complex(torch, ss, generate, cfg, max(3, a.steps // 10), 1)
        sec["backward"] = bench_backward(torch, ss, generate, cfg, max(3, a.steps // 10), 1)
        sec["general_A_path"] = bench_general_path(torch, ss, generate, cfg, max(5, a.steps // 5))
        sec["ssd_layer"] = bench_ssd(torch, ss, generate, configs.SSD_LAYER, max(5, a.steps // 5), 2)
        sec["decode"] = bench_decode(torch, ss, generate, configs.DECODE_256x8192,
                                     configs.DECODE_256x8192.n_tokens)
        sec["complex_decode"] = bench_complex_decode(torch, ss, generate, configs.DECODE_256x8192,
                                                     configs.DECODE_256x8192.n_tokens)
        cp = copy_peak(torch)
        out["copy_peak"] = cp
        out["hbm"]["frac_of_copy_peak"] = round(out["hbm"]["achieved"] / cp["achieved"], 4)
        dec = sec["decode"]
        dec["roofline"]["frac_of_copy_peak"] = round(dec["roofline"]["achieved"] / cp["achieved"], 4)
        out["secondary"] = sec
    if a.only is None and not a.no_cpu_baseline:
        log("[bench] timing the fp64 oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(torch, generate, cfg)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
