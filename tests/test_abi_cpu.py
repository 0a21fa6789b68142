"""C ABI on the CPU: the library loads, exports every declared symbol, and
rejects bad arguments before touching the GPU (no compute call is made)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssmscan.h")


@pytest.fixture(scope="module")
def L():
    from selective_state_space_18_amd import ssmscan
    try:
        return ssmscan.lib()
    except ImportError as e:  # pragma: no cover - build() runs before the suite
        pytest.fail(str(e))


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ssm_[a-z_]+)\s*\(", src)))


def test_header_and_binding_agree():
    from selective_state_space_18_amd import ssmscan
    assert declared_functions() == sorted(ssmscan.EXPORTS)


def test_every_declared_symbol_is_exported(L):
    from selective_state_space_18_amd import ssmscan
    out = subprocess.run(["nm", "-D", "--defined-only", ssmscan.LIB_PATH], check=True,
                         capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (ssm_\w+)", out))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(L, name)


def test_version_and_strerror(L):
    assert L.ssm_version() == 10000
    for code in range(0, 11):
        assert L.ssm_strerror(code) != b"unknown status code"
    assert L.ssm_strerror(12345) == b"unknown status code"


# Fake, well-aligned device addresses: validation rejects the call before any
# HIP call, so they are never dereferenced.
P = [0x100000 * (i + 1) for i in range(10)]


def scan(L, *, x=P[0], dl=P[1], A=P[2], B=P[3], C=P[4], D=P[5], y=P[6], hf=P[7], hi=None,
         Bsz=2, Ls=8, Dm=64, N=16, dtype=1):
    v = ctypes.c_void_p
    return L.ssm_scan_fwd_ex(v(x), v(dl), v(A), v(B), v(C), v(D), v(hi), v(y), v(hf),
                             Bsz, Ls, Dm, N, dtype, None)


def step(L, *, x=P[0], dl=P[1], A=P[2], B=P[3], C=P[4], D=P[5], h=P[6], y=P[7],
         Bsz=2, Dm=64, N=16, dtype=1):
    v = ctypes.c_void_p
    return L.ssm_step_ex(v(x), v(dl), v(A), v(B), v(C), v(D), v(h), v(y), Bsz, Dm, N, dtype, None)


def test_scan_argument_errors(L):
    assert scan(L, dtype=7) == 3
    assert scan(L, N=3) == 4 and scan(L, N=32) == 4 and scan(L, N=0) == 4
    assert scan(L, Bsz=-1) == 2 and scan(L, Ls=-5) == 2 and scan(L, Dm=-1) == 2
    assert scan(L, Bsz=1 << 40, Ls=1 << 40) == 2
    assert scan(L, C=0) == 1 and scan(L, y=0) == 1 and scan(L, D=0) == 1
    assert scan(L, x=0) == 1
    assert b"x is NULL" in L.ssm_last_error()
    assert scan(L, x=P[0] + 1) == 5            # bf16 needs 2-byte alignment
    assert scan(L, dtype=0, B=P[3] + 2) == 5   # fp32 needs 4-byte alignment
    assert scan(L, A=P[2] + 2) == 5
    assert scan(L, y=P[0]) == 6                # y aliases x
    assert scan(L, y=P[0] + 64) == 6           # partial overlap with x
    assert scan(L, hf=P[6]) == 6               # h_final aliases y
    assert scan(L, hf=P[1]) == 6               # h_final aliases delta
    assert scan(L, hi=P[6]) == 6               # h_init overlaps the output y
    assert scan(L, hi=P[7] + 4) == 6           # h_init partially overlaps h_final
    assert b"overlaps" in L.ssm_last_error()


def test_scan_empty_is_valid_without_pointers(L):
    # Bsz * Dm == 0: nothing to do, NULL pointers allowed, no device call.
    assert scan(L, Bsz=0, x=0, dl=0, B=0, C=0, y=0, hf=0) == 0
    assert scan(L, Dm=0, x=0, dl=0, A=0, D=0, y=0, hf=0) == 0
    assert L.ssm_last_error() == b""


def varlen(L, *, x=P[0], dl=P[1], A=P[2], B=P[3], C=P[4], D=P[5], cu=P[8], nseq=3, hi=None, y=P[6],
           hf=P[7], Ls=8, Dm=64, N=16, dtype=1):
    v = ctypes.c_void_p
    return L.ssm_scan_varlen_fwd(v(x), v(dl), v(A), v(B), v(C), v(D), v(cu), nseq, v(hi), v(y), v(hf),
                                 Ls, Dm, N, dtype, None)


def test_varlen_argument_errors(L):
    assert varlen(L, cu=0) == 1
    assert b"cu_seqlens" in L.ssm_last_error()
    assert varlen(L, nseq=-1) == 2
    assert varlen(L, nseq=0) == 2              # L > 0 needs at least one sequence
    assert varlen(L, cu=P[8] + 4) == 5         # int64 offsets need 8-byte alignment
    assert varlen(L, dtype=5) == 3 and varlen(L, N=6) == 4
    assert varlen(L, y=P[8]) == 6              # y overlaps cu_seqlens
    assert varlen(L, hf=P[8] + 8) == 6         # h_final overlaps cu_seqlens
    assert varlen(L, hi=P[7]) == 6             # in place is not allowed for packed sequences
    assert b"packed" in L.ssm_last_error()
    assert varlen(L, hi=P[9], x=0) == 1
    assert varlen(L, nseq=1 << 60) == 2        # nseq * Dm * N overflows
    # nothing to do: no device call
    assert varlen(L, nseq=0, Ls=0, x=0, dl=0, B=0, C=0, y=0, hf=0) == 0
    assert varlen(L, Dm=0, x=0, dl=0, A=0, D=0, y=0, hf=0) == 0
    assert L.ssm_last_error() == b""


def fused(L, *, x=P[0], dl=P[1], bias=None, A=P[2], B=P[3], C=P[4], D=P[5], cu=None, nseq=0, hi=None, y=P[6],
          hf=P[7], Bsz=2, Ls=8, Dm=64, N=16, dtype=1, flags=1):
    v = ctypes.c_void_p
    return L.ssm_scan_fused_fwd(v(x), v(dl), v(bias), v(A), v(B), v(C), v(D), v(cu), nseq, v(hi), v(y), v(hf),
                                Bsz, Ls, Dm, N, dtype, flags, None)


def test_fused_argument_errors(L):
    assert fused(L, flags=4) == 9 and fused(L, flags=0x80000000) == 9
    assert b"flag" in L.ssm_last_error()
    assert fused(L, bias=P[8] + 2) == 5        # fp32 bias needs 4-byte alignment
    assert fused(L, y=P[8], bias=P[8]) == 6    # y overlaps delta_bias
    assert fused(L, hf=P[8] + 64, bias=P[8]) == 6
    assert fused(L, cu=P[9], nseq=3, Bsz=2) == 2   # packed sequences need Bsz = 1
    assert fused(L, cu=P[9], nseq=-1, Bsz=1) == 2
    assert fused(L, cu=P[9], nseq=3, Bsz=1, hi=P[7]) == 6  # packed: no in-place state
    assert fused(L, Bsz=0, x=0, dl=0, B=0, C=0, y=0, hf=0, flags=3) == 0
    v = ctypes.c_void_p
    step_f = lambda **k: L.ssm_step_fused(v(P[0]), v(P[1]), v(k.get("bias")), v(P[2]), v(P[3]), v(P[4]),
                                          v(P[5]), v(k.get("h", P[6])), v(P[7]), 2, 64, 16, 1,
                                          k.get("flags", 1), None)
    assert step_f(flags=8) == 9
    assert step_f(bias=P[8] + 1) == 5
    assert step_f(bias=P[6]) == 6              # h overlaps delta_bias


def test_bwd_argument_errors(L):
    v = ctypes.c_void_p
    Q = [0x10000000 * (i + 1) for i in range(20)]  # fake, aligned, far apart

    def bwd(**k):
        a = dict(x=Q[0], dl=Q[1], bias=None, A=Q[2], B=Q[3], C=Q[4], D=Q[5], hi=None, dy=Q[6], dhf=None,
                 dx=Q[7], ddl=Q[8], dbias=None, dA=Q[9], dB=Q[10], dC=Q[11], dD=Q[12], dhi=None,
                 Bsz=2, Ls=8, Dm=64, N=16, dtype=1, flags=0)
        a.update(k)
        return L.ssm_scan_bwd(v(a["x"]), v(a["dl"]), v(a["bias"]), v(a["A"]), v(a["B"]), v(a["C"]), v(a["D"]),
                              v(a["hi"]), v(a["dy"]), v(a["dhf"]), v(a["dx"]), v(a["ddl"]), v(a["dbias"]),
                              v(a["dA"]), v(a["dB"]), v(a["dC"]), v(a["dD"]), v(a["dhi"]), a["Bsz"], a["Ls"],
                              a["Dm"], a["N"], a["dtype"], a["flags"], None)
    assert bwd(dtype=3) == 3 and bwd(N=7) == 4 and bwd(flags=4) == 9 and bwd(Ls=-1) == 2
    assert bwd(dy=0) == 1 and bwd(dA=0) == 1 and bwd(dB=0) == 1 and bwd(dx=0) == 1
    assert b"dx is NULL" in L.ssm_last_error()
    assert bwd(dB=Q[10] + 2) == 5              # fp32 gradients need 4-byte alignment
    assert bwd(dx=Q[7] + 1) == 5
    assert bwd(dx=Q[0]) == 6                   # dx overlaps x
    assert bwd(dC=Q[10]) == 6                  # dC overlaps dB
    assert bwd(dhi=Q[13], dhf=Q[13]) == 6      # dh_init overlaps dh_final
    assert bwd(dD=Q[6]) == 6                   # dD overlaps dy
    assert b"overlaps" in L.ssm_last_error()
    assert bwd(Bsz=1 << 40, Ls=1 << 40) == 2


def test_varlen_bwd_argument_errors(L):
    v = ctypes.c_void_p
    Q = [0x10000000 * (i + 1) for i in range(20)]  # fake, aligned, far apart

    def bwd(**k):
        a = dict(x=Q[0], dl=Q[1], bias=None, A=Q[2], B=Q[3], C=Q[4], D=Q[5], cu=Q[14], nseq=3, hi=None, dy=Q[6],
                 dhf=None, dx=Q[7], ddl=Q[8], dbias=None, dA=Q[9], dB=Q[10], dC=Q[11], dD=Q[12], dhi=None,
                 Ls=8, Dm=64, N=16, dtype=1, flags=0)
        a.update(k)
        return L.ssm_scan_varlen_bwd(v(a["x"]), v(a["dl"]), v(a["bias"]), v(a["A"]), v(a["B"]), v(a["C"]),
                                     v(a["D"]), v(a["cu"]), a["nseq"], v(a["hi"]), v(a["dy"]), v(a["dhf"]),
                                     v(a["dx"]), v(a["ddl"]), v(a["dbias"]), v(a["dA"]), v(a["dB"]), v(a["dC"]),
                                     v(a["dD"]), v(a["dhi"]), a["Ls"], a["Dm"], a["N"], a["dtype"], a["flags"],
                                     None)
    assert bwd(cu=0) == 1
    assert b"cu_seqlens" in L.ssm_last_error()
    assert bwd(nseq=-1) == 2
    assert bwd(nseq=0) == 2                    # L > 0 needs at least one sequence
    assert bwd(cu=Q[14] + 4) == 5              # int64 offsets need 8-byte alignment
    assert bwd(dtype=3) == 3 and bwd(N=7) == 4 and bwd(flags=4) == 9 and bwd(Ls=-1) == 2
    assert bwd(dy=0) == 1 and bwd(dx=0) == 1
    assert bwd(dx=Q[14]) == 6                  # dx overlaps cu_seqlens
    assert bwd(dhi=Q[14] + 8) == 6             # dh_init overlaps cu_seqlens
    assert bwd(dhi=Q[13], dhf=Q[13] + 64) == 6  # dh_init overlaps dh_final ([nseq][Dm][N] rows)
    assert b"overlaps" in L.ssm_last_error()
    assert bwd(nseq=1 << 60) == 2              # nseq * Dm * N overflows


def test_complex_bwd_argument_errors(L):
    v = ctypes.c_void_p
    Q = [0x10000000 * (i + 1) for i in range(20)]  # fake, aligned, far apart

    def bwd(**k):
        a = dict(x=Q[0], dl=Q[1], bias=None, A=Q[2], B=Q[3], C=Q[4], D=Q[5], hi=None, dy=Q[6], dhf=None, dx=Q[7],
                 ddl=Q[8], dbias=None, dA=Q[9], dB=Q[10], dC=Q[11], dD=Q[12], dhi=None, Bsz=2, Ls=8, Dm=64, N=16,
                 dtype=1, flags=0)
        a.update(k)
        return L.ssm_scan_complex_bwd(v(a["x"]), v(a["dl"]), v(a["bias"]), v(a["A"]), v(a["B"]), v(a["C"]),
                                      v(a["D"]), v(a["hi"]), v(a["dy"]), v(a["dhf"]), v(a["dx"]), v(a["ddl"]),
                                      v(a["dbias"]), v(a["dA"]), v(a["dB"]), v(a["dC"]), v(a["dD"]), v(a["dhi"]),
                                      a["Bsz"], a["Ls"], a["Dm"], a["N"], a["dtype"], a["flags"], None)
    assert bwd(dtype=3) == 3 and bwd(N=7) == 4 and bwd(flags=4) == 9 and bwd(Ls=-1) == 2
    assert bwd(x=0) == 1 and bwd(dy=0) == 1 and bwd(dA=0) == 1 and bwd(dx=0) == 1
    assert bwd(A=Q[2] + 2) == 5                # fp32 pairs need 4-byte alignment
    # A and dA hold (re, im) pairs: 2 * Dm * N floats (8 KiB here)
    assert bwd(dA=Q[2] + 4096) == 6
    assert b"dA" in L.ssm_last_error()
    # dh_init and dh_final hold Bsz * Dm * N pairs (16 KiB here)
    assert bwd(dhi=Q[13], dhf=Q[13] + 8192) == 6
    assert bwd(dx=Q[0]) == 6 and bwd(dB=Q[10] + 0, dC=Q[10] + 64) == 6
    assert bwd(Dm=1 << 40) == 2                # sizes overflow
    assert bwd(Dm=(1 << 30) // 32) == 2        # a 16-step bf16 segment spans 1 GiB


def test_ssd_argument_errors(L):
    v = ctypes.c_void_p
    Q = [0x10000000 * (i + 1) for i in range(12)]  # fake, 16-byte aligned, far apart

    def ssd(**k):
        a = dict(x=Q[0], dl=Q[1], bias=None, A=Q[2], B=Q[3], C=Q[4], D=Q[5], hi=None, y=Q[6], hf=Q[7],
                 Bsz=2, Ls=100, Dm=128, N=64, P=64, dtype=1, flags=0)
        a.update(k)
        return L.ssm_scan_ssd_fwd(v(a["x"]), v(a["dl"]), v(a["bias"]), v(a["A"]), v(a["B"]), v(a["C"]),
                                  v(a["D"]), v(a["hi"]), v(a["y"]), v(a["hf"]), a["Bsz"], a["Ls"], a["Dm"],
                                  a["N"], a["P"], a["dtype"], a["flags"], None)
    assert ssd(dtype=2) == 3
    assert ssd(N=16) == 4 and ssd(N=256) == 4
    assert b"32, 64, 128" in L.ssm_last_error()
    assert ssd(P=32) == 2 and b"head_dim" in L.ssm_last_error()
    assert ssd(Dm=96) == 2 and b"multiple" in L.ssm_last_error()
    assert ssd(flags=4) == 9
    assert ssd(Ls=-1) == 2
    assert ssd(x=0) == 1 and ssd(A=0) == 1 and ssd(y=0) == 1
    assert ssd(x=Q[0] + 8) == 5 and b"16-byte" in L.ssm_last_error()   # bf16 x needs 16 bytes here
    assert ssd(B=Q[3] + 4) == 5 and ssd(hf=Q[7] + 4) == 5 and ssd(hi=Q[8] + 4) == 5
    assert ssd(bias=Q[8] + 2) == 5
    assert ssd(y=Q[0]) == 6 and ssd(hf=Q[3]) == 6 and ssd(hf=Q[6]) == 6
    assert ssd(hi=Q[7], hf=Q[7] + 16) == 6      # partial overlap of the states
    assert ssd(Bsz=1 << 40, Ls=1 << 40) == 2
    assert ssd(Dm=(1 << 23)) == 2
    assert ssd(Bsz=0, x=0, dl=0, B=0, C=0, y=0, hf=0) == 0


def test_step_argument_errors(L):
    assert step(L, dtype=2) == 3
    assert step(L, N=5) == 4
    assert step(L, Bsz=-2) == 2
    assert step(L, h=0) == 1
    assert step(L, h=P[6] + 2) == 5
    assert step(L, y=P[6]) == 6                # y aliases h
    assert step(L, h=P[0]) == 6                # h aliases x
    assert step(L, Bsz=0, x=0, dl=0, B=0, C=0, h=0, y=0) == 0
    assert step(L, Dm=1 << 21) == 2            # 2^25 states per batch row
    v = ctypes.c_void_p
    assert L.ssm_step(v(0), v(P[1]), v(P[2]), v(P[3]), v(P[4]), v(P[5]), v(P[6]), v(P[7]),
                      2, 64, 16, None) == 1


def test_complex_step_argument_errors(L):
    v = ctypes.c_void_p

    def cstep(Bsz=2, Dm=64, N=16, dtype=1, flags=0, h=P[6]):
        return L.ssm_step_complex(v(P[0]), v(P[1]), v(None), v(P[2]), v(P[3]), v(P[4]), v(P[5]), v(h), v(P[7]),
                                  Bsz, Dm, N, dtype, flags, None)

    assert cstep(dtype=2) == 3
    assert cstep(N=3) == 4
    assert cstep(flags=8) == 9
    assert cstep(Dm=1 << 20) == 2          # 2^24 complex states per batch row
    assert cstep(h=P[6] + 2) == 5


def test_options(L):
    from selective_state_space_18_amd import ssmscan
    assert L.ssm_get_option(1) == 0 and L.ssm_get_option(2) == 0 and L.ssm_get_option(4) == 4
    assert L.ssm_set_option(4, 3) == 9
    assert L.ssm_set_option(1, -1) == 9
    assert L.ssm_set_option(2, 3) == 9
    assert L.ssm_set_option(99, 0) == 9
    assert L.ssm_get_option(99) == -1
    ssmscan.set_option(1, 128)
    assert ssmscan.get_option(1) == 128
    ssmscan.set_option(1, 0)
    with pytest.raises(ssmscan.SSMError):
        ssmscan.set_option(2, 5)


@pytest.mark.parametrize("shape,expect", [
    # (Bsz, L, Dm) on 256 CUs -> (segments, segment length)
    ((4, 16384, 5120), (64, 256)),       # Mamba-2.8B-shaped layer: 20 blocks per CU
    ((1, 1 << 20, 1024), (1024, 1024)),  # long context: 16 blocks per CU
    ((8, 2048, 1536), (32, 64)),         # Mamba-130M-shaped layer: capped by the 64-step minimum
    ((1, 256, 64), (4, 64)),             # tiny: capped by the 64-step minimum
    ((1, 100, 64), (1, 100)),            # too short to split
    ((3, 1000, 100), (15, 67)),          # capped at 1000 // 64 = 15 segments
])
def test_scan_plan(shape, expect):
    from selective_state_space_18_amd import ssmscan
    Bsz, Ls, Dm = shape
    S, sl = ssmscan.plan(Bsz, Ls, Dm, 16, compute_units=256)
    assert (S, sl) == expect
    assert (S - 1) * sl < Ls or Ls == 0
    assert S * sl >= Ls


def test_scan_plan_forced_segment_length():
    from selective_state_space_18_amd import ssmscan
    ssmscan.set_option(ssmscan.SSM_OPT_SEGMENT_LEN, 100)
    try:
        assert ssmscan.plan(4, 1000, 64, 16, compute_units=256) == (10, 100)
        assert ssmscan.plan(4, 1001, 64, 16, compute_units=256) == (11, 100)
    finally:
        ssmscan.set_option(ssmscan.SSM_OPT_SEGMENT_LEN, 0)


def test_binding_refuses_cpu_tensors():
    import torch
    from selective_state_space_18_amd import ssmscan
    x = torch.zeros(1, 4, 8)
    with pytest.raises(ValueError):
        ssmscan.scan_fwd(x, x, torch.zeros(8, 4), torch.zeros(1, 4, 4), torch.zeros(1, 4, 4), torch.zeros(8))


@pytest.mark.parametrize("shape,expect", [
    # (Bsz, L, Dm, dtype) on 256 CUs -> (segments, segment length, segments per group, groups)
    ((4, 16384, 5120, 1), (512, 32, 16, 32)),    # Mamba-2.8B-shaped layer
    ((4, 16384, 512, 1), (512, 32, 8, 64)),
    ((1, 130000, 72, 1), (4063, 32, 16, 254)),   # last group holds 15 segments
    ((1, 4900, 64, 0), (307, 16, 2, 154)),       # fp32: 16-step segments; last group holds 1
    ((1, 33000, 100, 1), (1032, 32, 5, 207)),    # last group holds 2
    ((2, 300, 130, 1), (10, 32, 1, 10)),
    ((8, 2048, 1536, 1), (64, 32, 2, 32)),       # Mamba-130M-shaped layer
    ((1, 0, 64, 1), (1, 32, 1, 1)),
])
def test_bwd_plan(shape, expect):
    from selective_state_space_18_amd import ssmscan
    Bsz, Ls, Dm, dt = shape
    got = ssmscan.bwd_plan(Bsz, Ls, Dm, 16, dt, compute_units=256)
    assert got == expect
    S, sl, G, groups = got
    assert groups == -(-S // G) and groups <= 256
    assert S * sl >= Ls and (S - 1) * sl < max(Ls, 1)


def test_bwd_plan_argument_errors(L):
    v = ctypes.c_int64()
    r = ctypes.byref(v)
    assert L.ssm_scan_bwd_plan(1, 8, 64, 16, 2, 256, r, r, r, r) == 3
    assert L.ssm_scan_bwd_plan(1, 8, 64, 5, 1, 256, r, r, r, r) == 4
    assert L.ssm_scan_bwd_plan(1, -8, 64, 16, 1, 256, r, r, r, r) == 2
    assert L.ssm_scan_bwd_plan(1, 8, 64, 16, 1, 256, None, r, r, r) == 1


def test_time_step_span_limits(L):
    """A scan time step of x must stay below 1 GiB, and a backward segment
    (32 steps in bf16, 16 in fp32) too: the kernels address them with 32-bit
    offsets.  The checks come before any pointer is looked at."""
    v = ctypes.c_void_p
    assert scan(L, Bsz=1, Ls=1, Dm=1 << 29, dtype=1) == 2        # 1 GiB per bf16 step
    assert scan(L, Bsz=1, Ls=1, Dm=1 << 28, dtype=0) == 2        # 1 GiB per fp32 step
    assert "1 GiB" in L.ssm_last_error().decode()

    def bwd(Dm, dtype):
        return L.ssm_scan_bwd(*(v(P[i % 10]) for i in range(18)), 1, 1, Dm, 16, dtype, 0, None)

    assert bwd(1 << 24, 1) == 2                                  # 32 steps x 2 B x 2^24 = 1 GiB
    assert "segment" in L.ssm_last_error().decode()
    assert bwd(1 << 24, 0) == 2                                  # 16 steps x 4 B x 2^24 = 1 GiB


def test_noalloc_rejects_oversized_calls_without_a_device(L):
    """ssm_scan_fwd_noalloc's fixed 64 MiB array: a call whose converted B/C
    rows alone (Bsz * L * 2N fp32 values) exceed it is refused before any
    device call; argument errors behave as in ssm_scan_fwd_ex."""
    v = ctypes.c_void_p
    far = [0x10000000000 * (i + 1) for i in range(9)]  # 1 TiB apart: no overlap

    def call(Bsz, Ls, Dm, N=16, dtype=1, x=far[0]):
        return L.ssm_scan_fwd_noalloc(v(x), v(far[1]), v(far[2]), v(far[3]), v(far[4]), v(far[5]), v(None),
                                      v(far[7]), v(far[8]), Bsz, Ls, Dm, N, dtype, None)

    assert call(1, 600000, 64) == 2          # 600000 x 32 x 4 B = 73 MiB of B/C rows
    assert "no-allocation" in L.ssm_last_error().decode()
    assert call(1, 300000, 64, dtype=0) == 2  # fp32 storage: 8-byte rows
    assert call(1, 8, 64, N=3) == 4
    assert call(1, 8, 64, x=0) == 1
    assert call(0, 8, 64) == 0                # nothing to do: no device call


def test_probe_argument_errors(L):
    """The calibration probes validate before launching: unknown kinds, bad
    sizes and NULL buffers are refused without a device call."""
    v = ctypes.c_void_p
    i64 = ctypes.c_int64
    sink = v(P[0])
    assert L.ssm_probe_issue(10, i64(1), i64(1), sink, None, None, None) == 9  # past the step-mix kind
    assert L.ssm_probe_issue(-1, i64(1), i64(1), sink, None, None, None) == 9
    assert L.ssm_probe_issue(9, i64(0), i64(1), sink, None, None, None) == 2
    assert L.ssm_probe_issue(9, i64(1), i64(1), v(None), None, None, None) == 1
    assert L.ssm_probe_hbm(15, sink, i64(1 << 20), None) == 9
    assert L.ssm_probe_hbm(16, sink, i64(24), None) != 0  # not a multiple of 16


def test_missing_library_fails_loudly(tmp_path):
    """With no built library the binding raises; there is no fallback path."""
    code = ("import torch\n"
            "from selective_state_space_18_amd import ssmscan as ss\n"
            "try:\n"
            "    ss.lib()\n"
            "except ImportError as e:\n"
            "    print('raised', e)\n"
            "else:\n"
            "    print('loaded')\n"
            "x = torch.zeros(1, 4, 64, dtype=torch.bfloat16)\n"
            "try:\n"
            "    ss.scan_fwd(x, x, torch.zeros(64, 16), torch.zeros(1, 4, 16, dtype=torch.bfloat16),\n"
            "                torch.zeros(1, 4, 16, dtype=torch.bfloat16), torch.zeros(64))\n"
            "except Exception as e:\n"
            "    print('scan raised', type(e).__name__)\n"
            "else:\n"
            "    print('scan ran')\n")
    env = dict(os.environ, SSMSCAN_LIB=str(tmp_path / "absent" / "libssmscan.so"))
    r = subprocess.run([__import__("sys").executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    assert "raised" in r.stdout and "loaded" not in r.stdout, r.stdout
    assert "scan raised" in r.stdout and "scan ran" not in r.stdout, r.stdout
