"""Seeded synthetic inputs, shared by the oracle side and the HIP side.

This module only draws random tensors with the distributions of the named
workloads; it contains none of the scan's arithmetic.  The transform applied to
delta (softplus of a shifted normal) is how the selection mechanism produces
delta upstream of the scan ("Mamba SSM Nedir?" page, section "Mamba'nin
Yeniligi: Selective SSM"); the scan itself consumes delta after it.

Draw order is fixed:  x, delta-noise (per-token recipe only), u_d, B, C, D,
then A (lognormal recipe only).  Decode draws u_d, D, h0 first, then per token
x, delta-noise, B, C.  Values are drawn in fp32 and then cast to the storage
dtype (round to nearest even for bf16).
"""
from typing import Dict, List

import numpy as np
import torch

from .configs import PackedConfig, ScanConfig, SsdConfig, StepConfig

_DT = {"fp32": torch.float32, "bf16": torch.bfloat16}

U_LO, U_HI = 1e-3, 1e-1


def storage_dtype(name: str) -> torch.dtype:
    return _DT[name]


def softplus(z: torch.Tensor) -> torch.Tensor:
    return torch.nn.functional.softplus(z)


def inv_softplus(u: torch.Tensor) -> torch.Tensor:
    # u + log(-expm1(-u)) = log(exp(u) - 1), computed without cancellation
    return u + torch.log(-torch.expm1(-u))


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _normal(shape, g, device, std=1.0):
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t


def s4d_real_A(Dm: int, N: int, device) -> torch.Tensor:
    """A[d, n] = -(n + 1) for every channel (fp32)."""
    a = -torch.arange(1, N + 1, device=device, dtype=torch.float32)
    return a.unsqueeze(0).expand(Dm, N).contiguous()


def scan_inputs(cfg: ScanConfig, device="cpu", seed=None) -> Dict[str, torch.Tensor]:
    """x, delta, A, B, C, D for one scan call on ``device``."""
    device = torch.device(device)
    g = _gen(device, cfg.seed if seed is None else seed)
    sd = _DT[cfg.dtype]
    Bsz, L, Dm, N = cfg.Bsz, cfg.L, cfg.Dm, cfg.N

    x = _normal((Bsz, L, Dm), g, device).to(sd)
    noise = _normal((Bsz, L, Dm), g, device, 0.5) if cfg.delta_kind in ("per_token", "raw_softplus") else None
    u = torch.rand((Dm,), generator=g, device=device, dtype=torch.float32) * (U_HI - U_LO) + U_LO
    delta_bias = None
    if cfg.delta_kind == "raw_softplus":
        # the projection output before the activation, and the projection's
        # bias: softplus(delta + delta_bias) has the per_token distribution
        delta = noise.to(sd)
        delta_bias = inv_softplus(u)
        del noise
    elif noise is not None:
        delta = softplus(noise.add_(inv_softplus(u))).to(sd)
        del noise
    elif cfg.delta_kind == "per_channel":
        delta = softplus(inv_softplus(u)).to(sd).view(1, 1, Dm).expand(Bsz, L, Dm).contiguous()
    else:
        raise ValueError(cfg.delta_kind)
    B = _normal((Bsz, L, N), g, device, cfg.bc_scale).to(sd)
    C = _normal((Bsz, L, N), g, device, cfg.bc_scale).to(sd)
    D = _normal((Dm,), g, device)
    if cfg.a_kind == "s4d_real":
        A = s4d_real_A(Dm, N, device)
    elif cfg.a_kind == "lognormal":
        A = -torch.exp(_normal((Dm, N), g, device, 0.5))
    else:
        raise ValueError(cfg.a_kind)
    out = {"x": x, "delta": delta, "A": A, "B": B, "C": C, "D": D}
    if delta_bias is not None:
        out["delta_bias"] = delta_bias
    return out


def step_state(cfg: StepConfig, device="cpu", seed=None) -> Dict[str, torch.Tensor]:
    """Per-layer constants and the resident state: u (for delta), A, D, h0."""
    device = torch.device(device)
    g = _gen(device, cfg.seed if seed is None else seed)
    Dm, N = cfg.Dm, cfg.N
    u = torch.rand((Dm,), generator=g, device=device, dtype=torch.float32) * (U_HI - U_LO) + U_LO
    D = _normal((Dm,), g, device)
    h = _normal((cfg.Bsz, Dm, N), g, device, cfg.h0_std)
    A = s4d_real_A(Dm, N, device)
    return {"A": A, "D": D, "h": h, "_u": u, "_gen": g}


def step_tokens(cfg: StepConfig, state: Dict[str, torch.Tensor], n_tokens: int) -> List[Dict[str, torch.Tensor]]:
    """``n_tokens`` consecutive decode inputs (x, delta [Bsz,Dm]; B, C [Bsz,N])."""
    g = state["_gen"]
    u = state["_u"]
    device = u.device
    sd = _DT[cfg.dtype]
    shift = inv_softplus(u)
    out = []
    for _ in range(n_tokens):
        x = _normal((cfg.Bsz, cfg.Dm), g, device).to(sd)
        delta = softplus(_normal((cfg.Bsz, cfg.Dm), g, device, 0.5).add_(shift)).to(sd)
        B = _normal((cfg.Bsz, cfg.N), g, device).to(sd)
        C = _normal((cfg.Bsz, cfg.N), g, device).to(sd)
        out.append({"x": x, "delta": delta, "B": B, "C": C})
    return out


def step_state_complex(cfg: StepConfig, device="cpu", seed=None) -> Dict[str, torch.Tensor]:
    """step_state with complex A (the complex_A recipe, seed + 100) and a
    complex resident state: the real part as step_state draws it, then the
    imaginary part ~ N(0, h0_std) from the same generator."""
    st = step_state(cfg, device, seed)
    im = _normal((cfg.Bsz, cfg.Dm, cfg.N), st["_gen"], torch.device(device), cfg.h0_std)
    st["h"] = torch.complex(st["h"], im)
    st["A"] = complex_A(cfg.Dm, cfg.N, (cfg.seed if seed is None else seed) + 100, device)
    return st


def complex_A(Dm: int, N: int, seed: int, device="cpu") -> torch.Tensor:
    """Complex diagonal A [Dm, N] (complex64): real part -exp(N(0, 0.5)),
    imaginary part pi * n * (1 + 0.1 N(0, 1)) -- decaying oscillators whose
    frequencies grow with the state index (draw order: real, then imaginary)."""
    g = _gen(torch.device(device), seed)
    re = -torch.exp(_normal((Dm, N), g, torch.device(device), 0.5))
    n = torch.arange(N, device=device, dtype=torch.float32).unsqueeze(0)
    im = torch.pi * n * (1.0 + 0.1 * _normal((Dm, N), g, torch.device(device)))
    return torch.complex(re, im)


def packed_lengths(nseq: int, mean_len: float, seed: int, p_empty: float = 0.0, sigma: float = 1.0,
                   max_len: int = 0) -> List[int]:
    """Lengths of ``nseq`` sequences for a packed (variable-length) call.

    A log-normal length mix around ``mean_len`` steps (long tail, as in packed
    prefill batches), each length at least 1, with a fraction ``p_empty`` of
    empty sequences; optionally capped at ``max_len``.
    """
    rng = np.random.default_rng(int(seed))
    mu = np.log(max(mean_len, 1.0)) - 0.5 * sigma * sigma
    lens = np.maximum(1, np.rint(rng.lognormal(mu, sigma, size=nseq))).astype(np.int64)
    if max_len > 0:
        lens = np.minimum(lens, max_len)
    if p_empty > 0:
        lens[rng.random(nseq) < p_empty] = 0
    return [int(v) for v in lens]


def cu_seqlens(lengths: List[int], device="cpu") -> torch.Tensor:
    """Start offsets [0, l0, l0+l1, ..., total] as int64."""
    out = [0]
    for v in lengths:
        out.append(out[-1] + int(v))
    return torch.tensor(out, dtype=torch.int64, device=device)


def packed_config_lengths(cfg: PackedConfig) -> List[int]:
    """Sequence lengths of a PackedConfig (they sum to cfg.L)."""
    draws = packed_lengths(max(1, 4 * cfg.L // max(cfg.mean_len, 1)), cfg.mean_len, cfg.seed,
                           p_empty=cfg.p_empty, max_len=cfg.max_len)
    out, total = [], 0
    for v in draws:
        if total + v > cfg.L:
            break
        out.append(v)
        total += v
    out.append(cfg.L - total)
    return out


def packed_inputs(cfg: PackedConfig, device="cpu") -> Dict[str, torch.Tensor]:
    """x, delta [L, Dm]; B, C [L, N]; A, D; cu_seqlens; h_init [nseq, Dm, N] or None."""
    inp = scan_inputs(cfg.as_scan(), device)
    out = {k: (v[0] if k in ("x", "delta", "B", "C") else v) for k, v in inp.items()}
    lengths = packed_config_lengths(cfg)
    out["cu"] = cu_seqlens(lengths, device)
    out["h_init"] = None
    if cfg.h0_std > 0:
        g = _gen(torch.device(device), cfg.seed + 1000)
        out["h_init"] = _normal((len(lengths), cfg.Dm, cfg.N), g, torch.device(device), cfg.h0_std)
    return out


def ssd_inputs(cfg: SsdConfig, device="cpu", seed=None) -> Dict[str, torch.Tensor]:
    """x, delta [Bsz,L,H], A [H], B, C, D [Dm] (and delta_bias [H], h_init)
    for a layer with a scalar decay per head.  Draw order: x, delta noise,
    u_h, B, C, D, A, h_init."""
    device = torch.device(device)
    g = _gen(device, cfg.seed if seed is None else seed)
    sd = _DT[cfg.dtype]
    Bsz, L, Dm, N, H = cfg.Bsz, cfg.L, cfg.Dm, cfg.N, cfg.heads()
    x = _normal((Bsz, L, Dm), g, device).to(sd)
    noise = _normal((Bsz, L, H), g, device, 0.5)
    u = torch.rand((H,), generator=g, device=device, dtype=torch.float32) * (U_HI - U_LO) + U_LO
    out = {}
    if cfg.delta_kind == "raw_softplus":
        delta = noise.to(sd)
        out["delta_bias"] = inv_softplus(u)
    elif cfg.delta_kind == "per_token":
        delta = softplus(noise.add_(inv_softplus(u))).to(sd)
    else:
        raise ValueError(cfg.delta_kind)
    del noise
    B = _normal((Bsz, L, N), g, device, cfg.bc_scale).to(sd)
    C = _normal((Bsz, L, N), g, device, cfg.bc_scale).to(sd)
    D = _normal((Dm,), g, device)
    A = -torch.exp(_normal((H,), g, device, 0.5))
    out.update({"x": x, "delta": delta, "A": A, "B": B, "C": C, "D": D})
    if cfg.h0_std > 0:
        out["h_init"] = _normal((Bsz, Dm, N), g, device, cfg.h0_std)
    return out


def alg_bytes_ssd(cfg: SsdConfig) -> int:
    """Minimum bytes of a scalar-decay layer call: x, delta, B, C, A, D (and
    h_init) read once, y and h_final written once."""
    s = 4 if cfg.dtype == "fp32" else 2
    BLD = cfg.Bsz * cfg.L * cfg.Dm
    return (2 * BLD * s + cfg.Bsz * cfg.L * cfg.heads() * s + 2 * cfg.Bsz * cfg.L * cfg.N * s
            + 4 * cfg.heads() + 4 * cfg.Dm + (2 if cfg.h0_std > 0 else 1) * 4 * cfg.Bsz * cfg.Dm * cfg.N)


def alg_bytes_scan(cfg: ScanConfig) -> int:
    """Bytes the scan must move at minimum: inputs once, outputs once."""
    s = 4 if cfg.dtype == "fp32" else 2
    BLD = cfg.Bsz * cfg.L * cfg.Dm
    BLN = cfg.Bsz * cfg.L * cfg.N
    return (2 * BLD * s + 2 * BLN * s + 4 * cfg.Dm * cfg.N + 4 * cfg.Dm
            + BLD * s + 4 * cfg.Bsz * cfg.Dm * cfg.N)


def alg_bytes_varlen(L: int, Dm: int, N: int, nseq: int, dtype: str, with_h_init: bool) -> int:
    """Minimum bytes of a packed call: x, delta, B, C, A, D, offsets, h_init
    (if given) read once; y and h_final written once."""
    s = 4 if dtype == "fp32" else 2
    return (3 * L * Dm * s + 2 * L * N * s + 4 * Dm * N + 4 * Dm + 8 * (nseq + 1)
            + (2 if with_h_init else 1) * 4 * nseq * Dm * N)


def alg_bytes_step(cfg: StepConfig) -> int:
    s = 4 if cfg.dtype == "fp32" else 2
    BD, BN = cfg.Bsz * cfg.Dm, cfg.Bsz * cfg.N
    return (8 * BD * cfg.N + 2 * s * BD + 2 * s * BN + s * BD
            + 4 * cfg.Dm * cfg.N + 4 * cfg.Dm)


def alg_bytes_step_complex(cfg: StepConfig) -> int:
    """As alg_bytes_step with a complex state and A (8 bytes per value)."""
    s = 4 if cfg.dtype == "fp32" else 2
    BD, BN = cfg.Bsz * cfg.Dm, cfg.Bsz * cfg.N
    return (16 * BD * cfg.N + 2 * s * BD + 2 * s * BN + s * BD
            + 8 * cfg.Dm * cfg.N + 4 * cfg.Dm)

