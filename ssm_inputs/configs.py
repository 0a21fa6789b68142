"""Named synthetic workloads for the selective scan and the decode step.

Shapes and distributions follow the five workload descriptions this project is
measured on; none of them needs trained weights or a dataset.  Notation:
N(mu, sigma) has standard deviation sigma; U[a, b] is uniform.

The sizes imitate the layer shapes of the Mamba checkpoints the pages name
(mamba-130m, mamba-2.8b; "Mamba SSM Nedir?" page, section "Nasil Denerim?"),
but every value is drawn at random.
"""
from dataclasses import dataclass, replace
from typing import Optional


@dataclass(frozen=True)
class ScanConfig:
    name: str
    Bsz: int
    L: int
    Dm: int
    N: int
    dtype: str              # storage dtype of x, delta, B, C, y: "fp32" | "bf16"
    a_kind: str             # "s4d_real": A[d,n] = -(n+1);  "lognormal": A = -exp(N(0, 0.5))
    delta_kind: str         # "per_token": softplus(0.5*N(0,1) + inv_softplus(u_d));
                            # "per_channel": softplus(inv_softplus(u_d)) = u_d for every t;
                            # "raw_softplus": delta stores 0.5*N(0,1) and delta_bias[d] =
                            #   inv_softplus(u_d); the scan applies softplus(delta + bias)
    bc_scale: float         # B, C ~ N(0,1) * bc_scale
    seed: int

    def elems(self) -> int:
        return self.Bsz * self.L * self.Dm * self.N

    def with_shape(self, **kw) -> "ScanConfig":
        return replace(self, **kw)


@dataclass(frozen=True)
class StepConfig:
    name: str
    Bsz: int
    Dm: int
    N: int
    dtype: str              # dtype of x, delta, B, C, y
    h0_std: float           # resident state h ~ N(0, h0_std), fp32
    n_tokens: int
    seed: int

    def elems_per_step(self) -> int:
        return self.Bsz * self.Dm * self.N

    def with_shape(self, **kw) -> "StepConfig":
        return replace(self, **kw)


# Tiny fp32 scan (the case the oracle runs in full in well under a second).
TINY_FP32 = ScanConfig("tiny_fp32_b1_l256_d64_n16", 1, 256, 64, 16, "fp32",
                       "s4d_real", "per_token", 1.0, seed=0)

# A Mamba-130M-shaped layer: random (non-structured) negative A.
MAMBA130M_LAYER = ScanConfig("mamba130m_layer_b8_l2048_d1536_n16", 8, 2048, 1536, 16,
                             "bf16", "lognormal", "per_token", 1.0, seed=1)

# A Mamba-2.8B-shaped layer: the headline throughput workload.
MAMBA2P8B_LAYER = ScanConfig("mamba2p8b_layer_b4_l16384_d5120_n16", 4, 16384, 5120, 16,
                             "bf16", "s4d_real", "per_token", 0.25, seed=2)

# The same layer with delta's activation fused into the scan: delta holds the
# projection output and delta_bias the projection bias; the draw order makes
# softplus(delta + delta_bias) the layer's delta before storage rounding.
FUSED_2P8B_LAYER = ScanConfig("fused_softplus_b4_l16384_d5120_n16", 4, 16384, 5120, 16,
                              "bf16", "s4d_real", "raw_softplus", 0.25, seed=2)

# Long context: one sequence of 2^20 tokens, slow-decay channels.
LONG_CONTEXT_1M = ScanConfig("long_context_b1_l1048576_d1024_n16", 1, 1 << 20, 1024, 16,
                             "bf16", "s4d_real", "per_channel", 1.0, seed=3)

# Recurrent decode step on a resident state.
DECODE_256x8192 = StepConfig("decode_b256_d8192_n16", 256, 8192, 16, "bf16",
                             h0_std=0.1, n_tokens=1000, seed=4)

@dataclass(frozen=True)
class PackedConfig:
    """Several sequences packed along time into one row (variable-length scan).

    Lengths: log-normal around ``mean_len`` (capped at ``max_len``), a share
    ``p_empty`` of empty sequences, drawn until the next one would overflow
    ``L``; the rest of ``L`` is one last sequence.  Each sequence starts from
    h_init ~ N(0, h0_std) when ``h0_std`` > 0.  x, delta, B, C follow the
    ScanConfig recipe for a [1, L, Dm] row.
    """
    name: str
    L: int
    Dm: int
    N: int
    dtype: str
    a_kind: str
    delta_kind: str
    bc_scale: float
    mean_len: int
    max_len: int
    p_empty: float
    h0_std: float
    seed: int

    def elems(self) -> int:
        return self.L * self.Dm * self.N

    def as_scan(self) -> ScanConfig:
        return ScanConfig(self.name, 1, self.L, self.Dm, self.N, self.dtype, self.a_kind,
                          self.delta_kind, self.bc_scale, self.seed)


# Packed prefill of a Mamba-2.8B-shaped layer: the same 4 x 16384 steps as
# MAMBA2P8B_LAYER, as a few dozen sequences of mixed length in one row.
PACKED_2P8B_LAYER = PackedConfig("packed_prefill_l65536_d5120_n16", 65536, 5120, 16, "bf16",
                                 "s4d_real", "per_token", 0.25, mean_len=2048, max_len=16384,
                                 p_empty=0.05, h0_std=0.5, seed=5)

@dataclass(frozen=True)
class SsdConfig:
    """A layer with a scalar decay per head (the state-space-duality form).

    Channels form heads of ``head_dim`` consecutive channels.  Head h has one
    real A[h] for all N states and its own delta per step; B_t and C_t are
    shared by every head of a batch row.  Recipe: x ~ N(0,1) [Bsz,L,Dm];
    delta per (b, t, h) from the per-token recipe with u_h ~ U[1e-3, 1e-1]
    per head (or the raw projection output and its bias, "raw_softplus");
    B, C ~ N(0,1) * bc_scale; D ~ N(0,1) per channel; A[h] = -exp(N(0, 0.5));
    h_init ~ N(0, h0_std) when h0_std > 0.
    """
    name: str
    Bsz: int
    L: int
    Dm: int
    N: int
    head_dim: int
    dtype: str
    delta_kind: str
    bc_scale: float
    h0_std: float
    seed: int

    def heads(self) -> int:
        return self.Dm // self.head_dim

    def elems(self) -> int:
        return self.Bsz * self.L * self.Dm * self.N

    def with_shape(self, **kw) -> "SsdConfig":
        return replace(self, **kw)


# The 2.8B-shaped layer width (80 heads of 64 channels) with the larger state
# a scalar-decay layer affords (N = 128); B, C ~ N(0,1)/sqrt(N).
SSD_LAYER = SsdConfig("ssd_layer_b4_l16384_d5120_n128_p64", 4, 16384, 5120, 128, 64, "bf16",
                      "per_token", 128 ** -0.5, h0_std=0.0, seed=6)

SCAN_CONFIGS = {c.name: c for c in (TINY_FP32, MAMBA130M_LAYER, MAMBA2P8B_LAYER,
                                    FUSED_2P8B_LAYER, LONG_CONTEXT_1M)}
STEP_CONFIGS = {DECODE_256x8192.name: DECODE_256x8192}


def get(name: str):
    if name in SCAN_CONFIGS:
        return SCAN_CONFIGS[name]
    if name in STEP_CONFIGS:
        return STEP_CONFIGS[name]
    raise KeyError(name)


def maybe(cfg: Optional[object], **kw):
    return cfg.with_shape(**kw) if kw else cfg
