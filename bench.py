#!/usr/bin/env python3
"""Throughput benchmark of libssmscan on one MI355X.

A step is one selective-scan forward (B/C prep, segment aggregate, carry and
output kernels) over the Mamba-2.8B-shaped layer: Bsz=4, L=16384, D=5120,
N=16, bf16 storage, fp32 arithmetic, synthetic seeded inputs resident in HBM.
`value` is elements/s (B*L*D*N per second) over exactly --steps back-to-back
steps, taken after --warmup untimed steps; before those, every timed workload
runs itself untimed for SETTLE_MS (60 ms), which the clocks need to reach
their loaded state after the input generation.  The JSON line also reports the achieved algorithmic HBM bandwidth;
the roofline of the dominant kernel (VALU-issue bound, with the HBM fractions
of the kernel and of the step, and counter-measured HBM traffic of the kernel
and of the whole call); the timing protocol (the median of individually
timed calls after a 512 MiB last-level-cache flush, and of cache-warm
calls); calibration probes (VALU and transcendental issue rates, streaming
read / read-modify-write / write HBM rates, empty-launch overhead, a torch
copy); the fp64 CPU oracle timed on a bounded sample of the same workload;
and -- under "secondary" -- the long-context scan, the Mamba-130M-shaped
layer, the scan options (fused delta activation, Euler input term), a packed
variable-length prefill, the scan with complex A, the backward (structured
and general A, and of the packed prefill), the general-A path forced on the
2.8B-shaped layer, the
scalar-decay (state-space duality) layer, and the decode step.

    python bench.py [--gpus 1] [--steps 50] [--warmup 20]
                    [--no-cpu-baseline] [--no-secondary]
    python bench.py --only scan        # one workload, for profiler runs
                                       # (scan, long, small, packed, options, backward,
                                       #  backward_general, packed_backward, complex,
                                       #  cdecode, general,
                                       #  ssd, decode, probe, hbmprobe)
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
# Published fp32 vector peak of MI355X: 256 CUs x 128 fp32 FMA lanes per cycle x
# 2 flops x 2.4 GHz = 157.3 TFLOP/s.  The probe kernels measure how much of it
# each instruction form reaches without packed FP32 (VGPR-only forms issue at
# up to twice the rate of a form with a scalar operand).
VALU_FP32_PEAK_TFLOPS = 256 * 128 * 2.4e9 * 2 / 1e12
# Wave64 VALU instructions per second at one instruction per 4 cycles per SIMD
# (the rate of an FMA with a scalar operand): 256 x 4 x 16 lanes x 2.4 GHz.
SINGLE_RATE_LANE_INSTR_PER_S = 256 * 4 * 16 * 2.4e9
SIMDS = 256 * 4
CLOCK_HZ = 2.4e9
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
# Complex-A backward, per state element: the forward recurrence once (27: the
# forward's count without the output term) and the adjoint with the gradient
# terms (71): lambda = C dy + nu (2); G_Abar = lambda conj(h_{t-1}) (6); G_k =
# lambda u (2); dL/du = Re(lambda conj(k)) (3) into dx (2), dB (1); dC (1);
# d(delta): A Abar (6) and two real parts (4 + 4); dA: delta Abar (2), its
# product (6) and sum (2), dk/dA = (z Abar - (Abar - 1)) / A^2 with 1/A^2
# per channel (14), its product (6) and sum (2); lambda conj(Abar) (6); the
# channel sums of dB and dC (2).
CBWD_FLOPS_PER_ELEM = 98
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
    "cplx": ("cplx_kernels.h", "scan_kernels.h", "ssm_device.h", "ssm_launch.h"),
    "cbwd": ("cbwd_kernels.h", "bwd_kernels.h", "cplx_kernels.h", "scan_kernels.h", "ssm_device.h",
             "ssm_launch.h"),
}


def source_sha(kind):
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kind]:
        with open(os.path.join(KERNEL_SRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(workload, kind):
    """HBM bytes measured with counters for one call of `workload`, if the
    kernel sources are unchanged since: (dominant kernel's bytes per launch,
    bytes of the whole call), else (None, None)."""
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None, None
    with open(path) as f:
        rec = json.load(f).get(workload)
    if not rec or rec.get("source_sha") != source_sha(kind):
        return None, None
    ks = rec["kernels"]
    return ks[rec["dominant"]]["hbm_bytes_per_launch"], sum(k["hbm_bytes_per_launch"] for k in ks.values())


def traffic_fields(workload, kind, alg):
    dom, call = traffic_for(workload, kind)
    return {"traffic": dom, "traffic_call": call,
            "traffic_call_over_algorithmic": None if call is None else round(call / alg, 3)}


# Sustained load the clocks need before a timed loop.  After input generation
# or any idle gap the GPU takes tens of milliseconds of load to settle: on the
# 2.8B-shaped scan a call after a 2 s pause ran 1.09 ms, the next ones 1.47,
# easing to 1.07 ms over about 30 calls.  Every timed workload first runs
# itself untimed for this long, then its W warmup steps, then the timed steps.
SETTLE_MS = 60.0


def settle(torch, fn, ms=SETTLE_MS):
    """Untimed calls of `fn` until about `ms` of wall time has passed
    (synchronising every 4 calls).  Returns the number of calls."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while True:
        for _ in range(4):
            fn(n)
            n += 1
        torch.cuda.synchronize()
        if (time.perf_counter() - t0) * 1e3 >= ms:
            return n


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


# Last-level cache (MALL) of MI355X: 256 MB.  Before each individually timed
# call a 512 MiB buffer is written so that nothing of the previous call stays
# cached; inputs are rotated over enough copies that back-to-back steps never
# find the previous step's inputs in that cache either.
MALL_BYTES = 256 << 20
FLUSH_BYTES = 512 << 20


class Flusher:
    def __init__(self, torch):
        self.buf = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda:0")

    def __call__(self, k):
        self.buf.fill_(float(k & 7))


def rotation_count(working_set_bytes):
    """Input copies so that the rotated working set is at least 4x the MALL."""
    return max(1, -(-4 * MALL_BYTES // max(1, working_set_bytes)))


def event_timed_calls(torch, fn, n, flush=None, start=0):
    """Median and all times (ms) of n calls, each bracketed by its own HIP
    events on the current stream (the stream the library launches on);
    flush(k) runs before call k, outside its events."""
    st = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for k in range(n):
        if flush is not None:
            flush(k)
        evs[k][0].record(st)
        fn(start + k)
        evs[k][1].record(st)
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in evs)
    return t[n // 2], t


def protocol_record(torch, fn, fn_fixed, steps, flusher, rotation):
    """The per-call figures beside the back-to-back rate: the median of
    individually timed calls after a MALL flush, and the median of calls
    repeated on one input set without a flush (cache-warm)."""
    n = max(5, min(steps, 20))
    fm, _ = event_timed_calls(torch, fn, n, flush=flusher)
    um, _ = event_timed_calls(torch, fn_fixed, n)
    return {"input_copies_rotated": rotation, "calls": n, "mall_flush_bytes": FLUSH_BYTES,
            "untimed_settle_ms_before_warmup": SETTLE_MS,
            "flushed_median_ms": round(fm, 5), "unflushed_same_input_median_ms": round(um, 5)}


def bench_scan(torch, ss, generate, cfg, steps, warmup, flusher=None, **opts):
    """opts: scan options (delta_bias is taken from the inputs when the
    workload's delta is the raw projection output).  Returns (ms per
    back-to-back step over rotated inputs, kernel times, S, segment length,
    protocol record)."""
    dev = "cuda:0"
    log(f"[bench] generating {cfg.name}")
    inp = generate.scan_inputs(cfg, dev)
    if "delta_bias" in inp:
        opts = dict(opts, delta_bias=inp["delta_bias"], delta_softplus=True)
    R = rotation_count(generate.alg_bytes_scan(cfg))
    sets = [inp] + [{k: (v.clone() if k in ("x", "delta", "B", "C") else v) for k, v in inp.items()}
                    for _ in range(R - 1)]
    y = torch.empty_like(inp["x"])
    hf = torch.empty(cfg.Bsz, cfg.Dm, cfg.N, device=dev, dtype=torch.float32)

    def call(z):
        ss.scan_fwd(z["x"], z["delta"], z["A"], z["B"], z["C"], z["D"], y=y, h_final=hf, **opts)

    def fn(i):
        call(sets[i % R])

    log(f"[bench] timing {cfg.name} {sorted(k for k, v in opts.items() if v is not None and v is not False)}: "
        f"{warmup} warmup + {steps} steps over {R} input copies")
    ms, kern = profiled_loop(torch, ss, fn, steps, warmup)
    proto = protocol_record(torch, fn, lambda _i: call(inp), steps, flusher, R) if flusher else None
    S, seg = ss.plan(cfg.Bsz, cfg.L, cfg.Dm, cfg.N)
    del inp, sets, y, hf
    torch.cuda.empty_cache()
    return ms, kern, S, seg, proto


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
    settle(torch, fn)
    ms = timed_loop(torch, fn, steps, warmup)
    del inp, y, hf, act
    torch.cuda.empty_cache()
    return ms


def profiled_loop(torch, ss, fn, steps, warmup):
    """Wall time per step of `steps` calls, then each kernel kind's average
    launch duration over the same number of calls with the library's
    per-kernel HIP-event timers on.  The event records add gaps between
    launches, so the wall time is taken with the timers off."""
    settle(torch, fn)
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


def scan_line(cfg, res, generate, **cfg_extra):
    ms, kern, S, seg, proto = res
    roof, hbm, cfgd, kms, proto = scan_record(cfg, ms, kern, S, seg, generate, proto=proto)
    rec = {"workload": cfg.name, "ms_per_step": round(ms, 5), "value": cfg.elems() / (ms * 1e-3),
           "unit": "elems/s", "hbm": hbm, "roofline": roof, "kernels_avg_ms": kms, "config": dict(cfgd, **cfg_extra)}
    if proto is not None:
        rec["protocol"] = proto
    return rec


def bench_options(torch, ss, generate, configs, steps, flusher=None, warmup=20):
    """The Mamba-2.8B-shaped layer with the scan options: delta's activation
    fused (softplus(delta + bias) inside the kernels), and the Euler input
    term, against the separate-activation route."""
    out = {}
    fc = configs.FUSED_2P8B_LAYER
    out["fused_softplus"] = scan_line(fc, bench_scan(torch, ss, generate, fc, steps, warmup, flusher),
                                      generate, delta="softplus(raw + bias) in the kernels")
    ums = bench_unfused_softplus(torch, ss, generate, fc, steps, warmup)
    out["separate_softplus_pass"] = {"ms_per_step": round(ums, 5), "value": fc.elems() / (ums * 1e-3),
                                     "note": "torch softplus pass over delta, then the plain scan"}
    ec = configs.MAMBA2P8B_LAYER
    out["euler_b"] = scan_line(ec, bench_scan(torch, ss, generate, ec, steps, warmup, flusher, euler_b=True),
                               generate, input_term="Euler: delta * B")
    return out


def bench_general_path(torch, ss, generate, cfg, steps, flusher=None, warmup=20):
    """The same layer with the structured-A fast path switched off, so every
    state element takes its own exponential (the path a layer with arbitrary
    real A runs)."""
    ss.set_option(ss.SSM_OPT_FORCE_GENERAL, 1)
    try:
        res = bench_scan(torch, ss, generate, cfg, steps, warmup, flusher)
    finally:
        ss.set_option(ss.SSM_OPT_FORCE_GENERAL, 0)
    rec = scan_line(cfg, res, generate, A="general path forced (one exp per state element)")
    rec["roofline"]["kernel"] = "scan_segment_kernel (output pass, general A)"
    # the counter figures are the structured kernels'
    rec["roofline"].update(traffic=None, traffic_call=None, traffic_call_over_algorithmic=None)
    return rec


def bench_ssd(torch, ss, generate, cfg, steps, warmup, flusher=None):
    """The scalar-decay layer (heads of 64 channels sharing A and delta, N =
    128) in its chunked matrix form.  Its binding roof is HBM: the layer's
    algorithmic bytes take longer at 8 TB/s than its algorithmic flops at the
    bf16 matrix-core peak.  Algorithmic flops of the output pass per (b, t, d):
    2N for C H, 2N for the state update B^T (w x), Q + 1 for the causal
    intra-chunk product (Q = 64 steps; the lower triangle of a Q x Q matrix
    times x), plus (Q + 1) N / Dm for the shared G = C B^T."""
    dev = "cuda:0"
    log(f"[bench] generating {cfg.name}")
    inp = generate.ssd_inputs(cfg, dev)
    y = torch.empty_like(inp["x"])
    hf = torch.empty((cfg.Bsz, cfg.Dm, cfg.N), dtype=torch.float32, device=dev)

    def fn(_i):
        ss.scan_ssd_fwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], cfg.head_dim, y=y, h_final=hf)

    log(f"[bench] timing {cfg.name}: {warmup} warmup + {steps} steps")
    ms, kern = profiled_loop(torch, ss, fn, steps, warmup)
    proto = protocol_record(torch, fn, fn, steps, flusher, 1) if flusher else None
    del inp, y, hf
    torch.cuda.empty_cache()
    Q = 64
    BLD = cfg.Bsz * cfg.L * cfg.Dm
    flops_out = BLD * (4 * cfg.N + (Q + 1) + (Q + 1) * cfg.N / cfg.Dm)
    out_ms = kern["ssd_output"]["avg_ms"]
    alg = generate.alg_bytes_ssd(cfg)
    mfma = flops_out / (out_ms * 1e-3) / 1e12
    gbs = alg / (out_ms * 1e-3) / 1e9
    roof = {"kernel": "ssd_chunk_kernel (output pass)", "bound": "hbm",
            "achieved": round(gbs, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBPS, 4), "avg_ms": round(out_ms, 5),
            "algorithmic_bytes_per_call": alg,
            "hbm_frac_step": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "floor_ms_hbm": round(alg / HBM_PEAK_GBPS / 1e9 * 1e3, 4),
            "floor_ms_mfma": round(flops_out / BF16_MFMA_PEAK_TFLOPS / 1e12 * 1e3, 4),
            "mfma_tflops": round(mfma, 2), "mfma_frac": round(mfma / BF16_MFMA_PEAK_TFLOPS, 4),
            "algorithmic_flops_per_launch": flops_out}
    roof.update(traffic_fields(cfg.name, "ssd", alg))
    rec = {"workload": cfg.name, "ms_per_step": round(ms, 5), "value": cfg.elems() / (ms * 1e-3),
           "unit": "elems/s",
           "hbm": {"achieved": round(alg / (ms * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                   "frac": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4), "algorithmic_bytes": alg},
           "roofline": roof,
           "kernels_avg_ms": {k: round(v["avg_ms"], 5) for k, v in kern.items()},
           "config": {"workload": cfg.name, "Bsz": cfg.Bsz, "L": cfg.L, "Dm": cfg.Dm, "N": cfg.N,
                      "head_dim": cfg.head_dim, "storage": cfg.dtype,
                      "A": "one real scalar per head, -exp(N(0, 0.5))", "delta": "per head, " + cfg.delta_kind,
                      "input_term": "ZOH"}}
    if proto is not None:
        rec["protocol"] = proto
    return rec


def alg_bytes_bwd(cfg):
    """Backward, inputs read once and outputs written once: x, delta, dy, B,
    C, A, D, dh_final read; dx, ddelta (storage type), dB, dC (fp32), dA, dD,
    dh_init written."""
    s = 2 if cfg.dtype == "bf16" else 4
    BLD, BLN, DN, BDN = cfg.Bsz * cfg.L * cfg.Dm, cfg.Bsz * cfg.L * cfg.N, cfg.Dm * cfg.N, cfg.Bsz * cfg.Dm * cfg.N
    return 5 * BLD * s + 2 * BLN * s + 2 * BLN * 4 + 2 * DN * 4 + 2 * cfg.Dm * 4 + 2 * BDN * 4


def bench_backward(torch, ss, generate, cfg, steps, warmup, flusher=None):
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
    proto = protocol_record(torch, fn, fn, steps, flusher, 1) if flusher else None
    plan = ss.bwd_plan(cfg.Bsz, cfg.L, cfg.Dm, cfg.N)
    del inp, dy, dhf, out
    torch.cuda.empty_cache()
    elems = cfg.elems()
    main_ms = kern["bwd_main"]["avg_ms"]
    alg = alg_bytes_bwd(cfg)
    achieved = elems * BWD_FLOPS_PER_ELEM / (main_ms * 1e-3) / 1e12
    roof = {"kernel": "bwd_main_kernel", "bound": "alu", "achieved": round(achieved, 3),
            "peak": round(VALU_FP32_PEAK_TFLOPS, 2), "unit": "TFLOP/s",
            "frac": round(achieved / VALU_FP32_PEAK_TFLOPS, 4),
            "avg_ms": round(main_ms, 5), "algorithmic_flops_per_launch": elems * BWD_FLOPS_PER_ELEM,
            "algorithmic_bytes_per_call": alg,
            "hbm_frac_kernel": round(alg / (main_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "hbm_frac_step": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
    roof.update(traffic_fields("backward_" + cfg.name, "bwd", alg))
    rec = {"workload": cfg.name, "ms_per_step": round(ms, 5), "value": elems / (ms * 1e-3), "unit": "elems/s",
           "roofline": roof, "kernels_avg_ms": {k: round(v["avg_ms"], 5) for k, v in kern.items()},
           "main_kernel_elems_per_s": elems / (main_ms * 1e-3),
           "config": {"workload": cfg.name, "A": cfg.a_kind, "segments": plan[0], "segment_len": plan[1],
                      "segments_per_group": plan[2], "groups": plan[3]}}
    if proto is not None:
        rec["protocol"] = proto
    return rec


def alg_bytes_bwd_packed(cfg, nseq):
    """Packed backward, inputs read once and outputs written once: as the
    dense backward for one row of cfg.L steps, with h_init, dh_final read and
    dh_init written per sequence and the sequence offsets read."""
    s = 2 if cfg.dtype == "bf16" else 4
    LD, LN, DN, SDN = cfg.L * cfg.Dm, cfg.L * cfg.N, cfg.Dm * cfg.N, nseq * cfg.Dm * cfg.N
    return 5 * LD * s + 2 * LN * s + 2 * LN * 4 + 2 * DN * 4 + 2 * cfg.Dm * 4 + 3 * SDN * 4 + 8 * (nseq + 1)


def bench_packed_backward(torch, ss, generate, cfg, steps, warmup, flusher=None):
    """Backward of the packed prefill: every input gradient of the packed scan
    for a random dy and dh_final, each sequence restarting from its own
    initial state; forward states recomputed inside the call."""
    dev = "cuda:0"
    log(f"[bench] generating {cfg.name} (packed backward)")
    inp = generate.packed_inputs(cfg, dev)
    nseq = inp["cu"].numel() - 1
    g = torch.Generator(device=dev)
    g.manual_seed(cfg.seed + 1)
    dy = torch.randn(inp["x"].shape, generator=g, device=dev).to(inp["x"].dtype)
    dhf = torch.randn((nseq, cfg.Dm, cfg.N), generator=g, device=dev)
    out = {}

    def fn(_i):
        nonlocal out
        out = ss.scan_varlen_bwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["cu"], dy,
                                 h_init=inp["h_init"], dh_final=dhf, out=out or None)

    log(f"[bench] timing {cfg.name} packed backward: {warmup} warmup + {steps} steps")
    ms, kern = profiled_loop(torch, ss, fn, steps, warmup)
    proto = protocol_record(torch, fn, fn, steps, flusher, 1) if flusher else None
    plan = ss.bwd_plan(1, cfg.L, cfg.Dm, cfg.N)
    lens = (inp["cu"][1:] - inp["cu"][:-1]).tolist()
    del inp, dy, dhf, out
    torch.cuda.empty_cache()
    elems = cfg.elems()
    main_ms = kern["bwd_main"]["avg_ms"]
    alg = alg_bytes_bwd_packed(cfg, nseq)
    achieved = elems * BWD_FLOPS_PER_ELEM / (main_ms * 1e-3) / 1e12
    roof = {"kernel": "bwd_main_kernel (packed)", "bound": "alu", "achieved": round(achieved, 3),
            "peak": round(VALU_FP32_PEAK_TFLOPS, 2), "unit": "TFLOP/s",
            "frac": round(achieved / VALU_FP32_PEAK_TFLOPS, 4),
            "avg_ms": round(main_ms, 5), "algorithmic_flops_per_launch": elems * BWD_FLOPS_PER_ELEM,
            "algorithmic_bytes_per_call": alg,
            "hbm_frac_kernel": round(alg / (main_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "hbm_frac_step": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
    roof.update(traffic_fields("packed_backward_" + cfg.name, "bwd", alg))
    rec = {"workload": cfg.name + "_backward", "ms_per_step": round(ms, 5), "value": elems / (ms * 1e-3),
           "unit": "elems/s", "roofline": roof,
           "kernels_avg_ms": {k: round(v["avg_ms"], 5) for k, v in kern.items()},
           "main_kernel_elems_per_s": elems / (main_ms * 1e-3),
           "config": {"workload": cfg.name, "A": cfg.a_kind, "sequences": nseq, "empty_sequences": lens.count(0),
                      "longest": max(lens), "segments": plan[0], "segment_len": plan[1],
                      "segments_per_group": plan[2], "groups": plan[3], "h_init": cfg.h0_std > 0}}
    if proto is not None:
        rec["protocol"] = proto
    return rec


def bench_complex(torch, ss, generate, cfg, steps, warmup, flusher=None):
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
    proto = protocol_record(torch, fn, fn, steps, flusher, 1) if flusher else None
    del inp, A, y, hf
    torch.cuda.empty_cache()
    out_ms = kern["scan_output"]["avg_ms"]
    achieved = cfg.elems() * CPLX_FLOPS_PER_ELEM / (out_ms * 1e-3) / 1e12
    alg = generate.alg_bytes_scan(cfg) + cfg.Dm * cfg.N * 4 + cfg.Bsz * cfg.Dm * cfg.N * 4  # complex A, h_final
    rec = {"workload": cfg.name + "_complex_A", "ms_per_step": round(ms, 5), "value": cfg.elems() / (ms * 1e-3),
           "unit": "elems/s",
           "roofline": {"kernel": "cplx_segment_kernel (output pass)", "bound": "alu",
                        "achieved": round(achieved, 3), "peak": round(VALU_FP32_PEAK_TFLOPS, 2), "unit": "TFLOP/s",
                        "frac": round(achieved / VALU_FP32_PEAK_TFLOPS, 4),
                        **traffic_fields("complex_A_" + cfg.name, "cplx", alg),
                        "avg_ms": round(out_ms, 5),
                        "algorithmic_flops_per_launch": cfg.elems() * CPLX_FLOPS_PER_ELEM,
                        "hbm_frac_kernel": round(alg / (out_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                        "hbm_frac_step": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                        "note": "exp, sin and cos count one flop each; each takes two VALU issue slots"},
           "kernels_avg_ms": {k: round(v["avg_ms"], 5) for k, v in kern.items()}}
    if proto is not None:
        rec["protocol"] = proto
    return rec


def alg_bytes_bwd_complex(cfg):
    """Complex-A backward, inputs read once and outputs written once: as the
    real backward, with A, dA and the state pairs (dh_final, dh_init) twice
    as large."""
    return alg_bytes_bwd(cfg) + 2 * cfg.Dm * cfg.N * 4 + 2 * cfg.Bsz * cfg.Dm * cfg.N * 4


def bench_complex_backward(torch, ss, generate, cfg, steps, warmup, flusher=None):
    """Backward of the complex-A layer: every input gradient for a random dy
    and dh_final, forward states recomputed inside the call."""
    dev = "cuda:0"
    log(f"[bench] generating {cfg.name} (complex A, backward)")
    inp = generate.scan_inputs(cfg, dev)
    A = generate.complex_A(cfg.Dm, cfg.N, cfg.seed + 100, dev)
    g = torch.Generator(device=dev)
    g.manual_seed(cfg.seed + 1)
    dy = torch.randn(inp["x"].shape, generator=g, device=dev).to(inp["x"].dtype)
    dhf = torch.complex(torch.randn((cfg.Bsz, cfg.Dm, cfg.N), generator=g, device=dev),
                        torch.randn((cfg.Bsz, cfg.Dm, cfg.N), generator=g, device=dev))
    out = {}

    def fn(_i):
        nonlocal out
        out = ss.scan_complex_bwd(inp["x"], inp["delta"], A, inp["B"], inp["C"], inp["D"], dy, dh_final=dhf,
                                  out=out or None)

    log(f"[bench] timing {cfg.name} complex backward: {warmup} warmup + {steps} steps")
    ms, kern = profiled_loop(torch, ss, fn, steps, warmup)
    proto = protocol_record(torch, fn, fn, steps, flusher, 1) if flusher else None
    del inp, A, dy, dhf, out
    torch.cuda.empty_cache()
    elems = cfg.elems()
    main_ms = kern["bwd_main"]["avg_ms"]
    alg = alg_bytes_bwd_complex(cfg)
    achieved = elems * CBWD_FLOPS_PER_ELEM / (main_ms * 1e-3) / 1e12
    roof = {"kernel": "cbwd_main_kernel", "bound": "alu", "achieved": round(achieved, 3),
            "peak": round(VALU_FP32_PEAK_TFLOPS, 2), "unit": "TFLOP/s",
            "frac": round(achieved / VALU_FP32_PEAK_TFLOPS, 4),
            "avg_ms": round(main_ms, 5), "algorithmic_flops_per_launch": elems * CBWD_FLOPS_PER_ELEM,
            "algorithmic_bytes_per_call": alg,
            "hbm_frac_kernel": round(alg / (main_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "hbm_frac_step": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "note": "exp, sin and cos count one flop each; each takes two VALU issue slots"}
    roof.update(traffic_fields("complex_backward_" + cfg.name, "cbwd", alg))
    rec = {"workload": cfg.name + "_complex_A_backward", "ms_per_step": round(ms, 5),
           "value": elems / (ms * 1e-3), "unit": "elems/s", "roofline": roof,
           "kernels_avg_ms": {k: round(v["avg_ms"], 5) for k, v in kern.items()},
           "main_kernel_elems_per_s": elems / (main_ms * 1e-3),
           "config": {"workload": cfg.name, "A": "complex: a = -exp(N(0, 0.5)), w = pi n (1 + 0.1 N(0, 1))",
                      "segment_len": 16}}
    if proto is not None:
        rec["protocol"] = proto
    return rec


def bench_packed(torch, ss, generate, cfg, steps, warmup, flusher=None):
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
    proto = protocol_record(torch, fn, fn, steps, flusher, 1) if flusher else None
    S, seg = ss.plan(1, cfg.L, cfg.Dm, cfg.N)
    lens = (inp["cu"][1:] - inp["cu"][:-1]).tolist()
    del inp, y, hf
    torch.cuda.empty_cache()
    elems = cfg.elems()
    alg = generate.alg_bytes_varlen(cfg.L, cfg.Dm, cfg.N, nseq, cfg.dtype, cfg.h0_std > 0)
    out_ms = kern["scan_output"]["avg_ms"]
    achieved = elems * SCAN_FLOPS_PER_ELEM / (out_ms * 1e-3) / 1e12
    roof = {"kernel": "scan_segment_kernel (output pass, packed)", "bound": "alu",
            "achieved": round(achieved, 3), "peak": round(VALU_FP32_PEAK_TFLOPS, 2), "unit": "TFLOP/s",
            "frac": round(achieved / VALU_FP32_PEAK_TFLOPS, 4), "avg_ms": round(out_ms, 5),
            "hbm_frac_kernel": round(alg / (out_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "hbm_frac_step": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
    roof.update(traffic_fields(cfg.name, "scan", alg))
    rec = {
        "workload": cfg.name, "ms_per_step": round(ms, 5), "value": elems / (ms * 1e-3), "unit": "elems/s",
        "config": {"workload": cfg.name, "L": cfg.L, "Dm": cfg.Dm, "N": cfg.N, "storage": cfg.dtype,
                   "A": cfg.a_kind, "sequences": nseq, "empty_sequences": lens.count(0),
                   "longest": max(lens), "segments": S, "segment_len": seg, "h_init": cfg.h0_std > 0},
        "hbm": {"achieved": round(alg / (ms * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4), "algorithmic_bytes": alg},
        "roofline": roof,
        "kernels_avg_ms": {k: round(v["avg_ms"], 5) for k, v in kern.items()},
    }
    if proto is not None:
        rec["protocol"] = proto
    return rec


def scan_record(cfg, ms, kern, S, seg, generate, kind="scan", proto=None):
    """Roofline of the dominant kernel (the output pass) and the step.  The
    binding roof is VALU issue: 'achieved' counts SCAN_FLOPS_PER_ELEM
    algorithmic flops per state element against the published fp32 vector
    peak; cycles_per_wave_step_per_simd is the pass's issue cost per time step
    of a 64-channel tile, to set beside the step-mix probe's.  The HBM
    fractions are the algorithmic bytes of the whole call over the output
    pass's time and over the whole step's time, against 8 TB/s."""
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
        "avg_ms": round(out_ms, 5),
        "algorithmic_flops_per_launch": elems * SCAN_FLOPS_PER_ELEM,
        "algorithmic_bytes_per_call": alg,
        "hbm_frac_kernel": round(alg / (out_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "hbm_frac_step": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
    }
    # one wave-step = one time step of one 64-channel tile; the output pass
    # runs Bsz * ceil(Dm/64) * L of them
    wave_steps = cfg.Bsz * ((cfg.Dm + 63) // 64) * cfg.L
    roof["cycles_per_wave_step_per_simd"] = round(out_ms * 1e-3 * CLOCK_HZ * SIMDS / wave_steps, 1)
    roof.update(traffic_fields(cfg.name, kind, alg))
    hbm = {"achieved": round(alg / (ms * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
           "frac": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4), "algorithmic_bytes": alg}
    cfgd = {"workload": cfg.name, "Bsz": cfg.Bsz, "L": cfg.L, "Dm": cfg.Dm, "N": cfg.N,
            "storage": cfg.dtype, "A": cfg.a_kind, "delta": cfg.delta_kind,
            "segments": S, "segment_len": seg}
    kms = {k: round(v["avg_ms"], 5) for k, v in kern.items()}
    if proto is not None:
        proto = dict(proto, flushed_median_elems_per_s=elems / (proto["flushed_median_ms"] * 1e-3))
    return roof, hbm, cfgd, kms, proto


def bench_decode(torch, ss, generate, cfg, n_tokens, layers=4, flusher=None, launch_us=None):
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
    ms, kern = profiled_loop(torch, ss, fn, n_tokens, 400)  # about 20 ms of warmup: the clocks come up
    k_ms = kern["step"]["avg_ms"]
    alg = generate.alg_bytes_step(cfg)
    proto = None
    if flusher is not None:
        fm, _ = event_timed_calls(torch, fn, 50, flush=flusher)
        um, _ = event_timed_calls(torch, lambda _i: fn(0), 50)
        proto = {"layer_states_cycled": layers, "calls": 50, "mall_flush_bytes": FLUSH_BYTES,
                 "flushed_median_ms": round(fm, 5), "unflushed_same_state_median_ms": round(um, 5),
                 "flushed_median_hbm_frac": round(alg / (fm * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
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
        "roofline": dict({"kernel": "step_kernel", "bound": "hbm",
                          "achieved": round(alg / (k_ms * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                          "frac": round(alg / (k_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                          "avg_ms": round(k_ms, 5), "algorithmic_bytes_per_launch": alg},
                         **traffic_fields(cfg.name, "step", alg)),
        "state_layers_cycled": layers,
        "graph_ms_per_step": None if graph_ms is None else round(graph_ms, 5),
        "graph_value": None if graph_ms is None else cfg.elems_per_step() / (graph_ms * 1e-3),
        "protocol": proto,
        "launch_overhead_us": launch_us,
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
    ms, kern = profiled_loop(torch, ss, fn, n_tokens, 400)  # about 20 ms of warmup: the clocks come up
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
                     "frac": round(alg / (k_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                     **traffic_fields("complex_" + cfg.name, "cplx", alg),
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


def bench_probe(torch, ss, iters=2048):
    """Measured issue rates of the VALU and the transcendental unit, from the
    library's probe kernels (known per-lane instruction mix, 16 independent
    chains per lane), each launch timed with HIP events on the stream it runs
    on.  Rates are lane-instructions per second, given as fractions of the
    single rate (one wave64 instruction per 4 cycles per SIMD, 3.93e13
    lane-instructions/s) and of the published peak (twice that: 157.3 TFLOP/s
    counting an FMA as two flops).  scan_step_mix is one structured output
    step of the scan (N = 16) without memory traffic; its cycles per
    wave-step are the issue ceiling of the scan's own instruction mix."""
    derived = SINGLE_RATE_LANE_INSTR_PER_S
    out = {"single_rate_lane_instr_per_s": derived, "published_peak_lane_instr_per_s": 2 * derived}
    st = torch.cuda.current_stream()
    for kind, blocks in (("fma_f32", 256), ("fma_f32", 1024), ("fma_f32", 4096), ("exp_f32", 4096),
                         ("fma_exp_f32", 4096), ("fma_f64", 4096), ("fmac_f32", 4096), ("mul_f32", 4096),
                         ("add_f32", 4096), ("fma_f32_vgpr", 4096), ("fmac_f32", 1024), ("fma_f32_vgpr", 1024),
                         ("scan_step_mix", 2048), ("scan_step_mix", 8192)):
        sink = torch.zeros(blocks * 256, dtype=torch.float32, device="cuda:0")
        ss.probe_issue(kind, blocks, 16, sink)  # warm-up
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        ms = []
        for _ in range(5):
            a.record(st)
            valu, trans = ss.probe_issue(kind, blocks, iters, sink)
            b.record(st)
            b.synchronize()
            ms.append(a.elapsed_time(b))
        ms.sort()
        t = ms[len(ms) // 2] * 1e-3
        lanes = blocks * 256 * iters
        rec = {"blocks": blocks, "waves_per_simd": blocks * 4 / 1024, "ms": round(t * 1e3, 4),
               "valu_per_iter": valu, "trans_per_iter": trans,
               "valu_lane_instr_per_s": lanes * valu / t,
               "frac_of_single_rate": round(lanes * valu / t / derived, 4),
               "frac_of_published_peak": round(lanes * valu / t / (2 * derived), 4),
               "cycles_per_wave_step_per_simd": round(t * CLOCK_HZ * SIMDS / (blocks * 4 * iters), 1)}
        if trans:
            rec["trans_lane_instr_per_s"] = lanes * trans / t
        out[f"{kind}_b{blocks}"] = rec
        log(f"[bench] probe {kind} blocks={blocks}: {rec['ms']} ms, {rec['frac_of_single_rate']} of the single rate")
        del sink
    return out


def hbm_probes(torch, ss, nbytes=2 << 30, reps=5):
    """Streaming read, in-place read-modify-write and write rates over a
    2 GiB buffer (8x the last-level cache), median of `reps` event-timed
    calls: the practical HBM ceiling beside the 8 TB/s specification."""
    buf = torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda:0")
    out = {}
    for kind in ("read", "rmw", "write"):
        moved = ss.probe_hbm(kind, buf)  # warm-up
        med, _ = event_timed_calls(torch, lambda _i: ss.probe_hbm(kind, buf), reps)
        out[kind] = {"GB/s": round(moved / (med * 1e-3) / 1e9, 1), "bytes": moved, "ms": round(med, 4)}
        log(f"[bench] hbm probe {kind}: {out[kind]['GB/s']} GB/s")
    del buf
    torch.cuda.empty_cache()
    out["practical_peak_gbps"] = max(v["GB/s"] for v in out.values() if isinstance(v, dict))
    return out


def launch_overhead_us(torch, ss, n=200):
    """Time per launch of an empty one-block kernel, back to back on one
    stream (what a step pays before any work)."""
    sink = torch.zeros(256, dtype=torch.float32, device="cuda:0")
    ss.probe_issue("empty", 1, 1, sink)
    ms = timed_loop(torch, lambda _i: ss.probe_issue("empty", 1, 1, sink), n, 10)
    return round(ms * 1e3, 3)


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
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--only", choices=["scan", "long", "decode", "small", "packed", "options", "backward",
                                       "backward_general", "packed_backward", "complex", "complex_backward", "cdecode",
                                       "general",
                                       "ssd", "probe", "hbmprobe"],
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

    if a.only == "probe":
        print(json.dumps(bench_probe(torch, ss)), flush=True)
        return
    if a.only == "hbmprobe":
        print(json.dumps(hbm_probes(torch, ss)), flush=True)
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
    if a.only == "complex_backward":
        rec = bench_complex_backward(torch, ss, generate, configs.MAMBA2P8B_LAYER, a.steps, a.warmup)
        print(json.dumps(rec), flush=True)
        return
    if a.only == "ssd":
        rec = bench_ssd(torch, ss, generate, configs.SSD_LAYER, a.steps, a.warmup)
        print(json.dumps(rec), flush=True)
        return
    if a.only == "general":
        rec = bench_general_path(torch, ss, generate, configs.MAMBA2P8B_LAYER, a.steps, warmup=a.warmup)
        print(json.dumps(rec), flush=True)
        return
    if a.only == "backward":
        rec = bench_backward(torch, ss, generate, configs.MAMBA2P8B_LAYER, a.steps, a.warmup)
        print(json.dumps(rec), flush=True)
        return
    if a.only == "backward_general":
        rec = bench_backward(torch, ss, generate, configs.MAMBA130M_LAYER, a.steps, a.warmup)
        print(json.dumps(rec), flush=True)
        return
    if a.only == "packed_backward":
        rec = bench_packed_backward(torch, ss, generate, configs.PACKED_2P8B_LAYER, a.steps, a.warmup)
        print(json.dumps(rec), flush=True)
        return
    if a.only == "options":
        print(json.dumps(bench_options(torch, ss, generate, configs, a.steps, warmup=a.warmup)), flush=True)
        return
    if a.only == "packed":
        rec = bench_packed(torch, ss, generate, configs.PACKED_2P8B_LAYER, a.steps, a.warmup)
        print(json.dumps(rec), flush=True)
        return
    if a.only in ("long", "small", "scan"):
        cfg = {"long": configs.LONG_CONTEXT_1M, "small": configs.MAMBA130M_LAYER,
               "scan": configs.MAMBA2P8B_LAYER}[a.only]
        print(json.dumps(scan_line(cfg, bench_scan(torch, ss, generate, cfg, a.steps, a.warmup), generate)),
              flush=True)
        return

    flusher = Flusher(torch)
    cfg = configs.MAMBA2P8B_LAYER
    ms, kern, S, seg, proto = bench_scan(torch, ss, generate, cfg, a.steps, a.warmup, flusher)
    roof, hbm, cfgd, kms, proto = scan_record(cfg, ms, kern, S, seg, generate, proto=proto)
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
        "protocol": proto,
    }
    if a.only is None and not a.no_secondary:
        cal = {"valu": bench_probe(torch, ss), "hbm": hbm_probes(torch, ss),
               "launch_overhead_us": launch_overhead_us(torch, ss), "copy": copy_peak(torch)}
        out["calibration"] = cal
        mix = cal["valu"]["scan_step_mix_b8192"]["cycles_per_wave_step_per_simd"]
        out["roofline"]["step_mix_cycles_per_wave_step_per_simd"] = mix
        out["roofline"]["frac_of_step_mix_rate"] = round(mix / out["roofline"]["cycles_per_wave_step_per_simd"], 4)
        practical = cal["hbm"]["practical_peak_gbps"]
        out["hbm"]["practical_peak_gbps"] = practical
        out["hbm"]["frac_of_practical_peak"] = round(out["hbm"]["achieved"] / practical, 4)
        steps5 = max(5, a.steps // 5)
        # every workload starts right after its input generation, when the
        # clocks are still coming up: the same warmup as the headline
        wu = a.warmup
        sec = {}
        lc = configs.LONG_CONTEXT_1M
        sec["long_context"] = scan_line(lc, bench_scan(torch, ss, generate, lc, max(3, a.steps // 5), wu, flusher),
                                        generate)
        sm = configs.MAMBA130M_LAYER
        sec["mamba130m_layer"] = scan_line(sm, bench_scan(torch, ss, generate, sm, a.steps, a.warmup, flusher),
                                           generate)
        sec["mamba130m_layer"]["note"] = (
            "random A: every state element takes its own exp (general path); ms_per_step rotates over input "
            "copies whose total exceeds the 256 MB last-level cache, protocol gives the flushed and the "
            "cache-warm (same input, no flush) per-call medians")
        sec["fused_softplus"] = bench_options(torch, ss, generate, configs, steps5, flusher, wu)
        sec["packed_prefill"] = bench_packed(torch, ss, generate, configs.PACKED_2P8B_LAYER, steps5, wu, flusher)
        sec["complex_A"] = bench_complex(torch, ss, generate, cfg, max(3, a.steps // 10), wu, flusher)
        sec["complex_A_backward"] = bench_complex_backward(torch, ss, generate, cfg, 3, wu, flusher)
        sec["backward"] = bench_backward(torch, ss, generate, cfg, max(3, a.steps // 10), wu, flusher)
        sec["backward_general_A"] = bench_backward(torch, ss, generate, configs.MAMBA130M_LAYER, steps5, wu,
                                                   flusher)
        sec["packed_backward"] = bench_packed_backward(torch, ss, generate, configs.PACKED_2P8B_LAYER,
                                                       max(3, a.steps // 10), wu, flusher)
        sec["general_A_path"] = bench_general_path(torch, ss, generate, cfg, steps5, flusher, wu)
        sec["ssd_layer"] = bench_ssd(torch, ss, generate, configs.SSD_LAYER, steps5, wu, flusher)
        sec["decode"] = bench_decode(torch, ss, generate, configs.DECODE_256x8192,
                                     configs.DECODE_256x8192.n_tokens, flusher=flusher,
                                     launch_us=cal["launch_overhead_us"])
        sec["complex_decode"] = bench_complex_decode(torch, ss, generate, configs.DECODE_256x8192,
                                                     configs.DECODE_256x8192.n_tokens)
        for rec in (sec["decode"], sec["complex_decode"], sec["ssd_layer"]):
            rec["roofline"]["frac_of_practical_peak"] = round(rec["roofline"]["achieved"] / practical, 4)
        out["secondary"] = sec
    if a.only is None and not a.no_cpu_baseline:
        log("[bench] timing the fp64 oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(torch, generate, cfg)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
