"""Build libssmscan.so (HIP, gfx950) in-tree with hipcc.

    python -m selective_state_space_18_amd.build [-v] [--isa DIR]

Objects go to ``_build/`` next to this file; the shared library is written to
``libssmscan.so`` in the package directory, where the binding loads it.
``--isa DIR`` additionally keeps the device assembly (for inspection).
"""
import argparse
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libssmscan.so")

ARCH = "gfx950"
SOURCES = ["abi.cpp", "scan_f32.hip", "scan_f32_packed.hip", "scan_bf16.hip", "scan_bf16_packed.hip",
           "scan_launch.hip", "step_kernel.hip", "bwd_f32.hip", "bwd_f32_packed.hip", "bwd_bf16.hip",
           "bwd_bf16_packed.hip", "cplx_f32.hip", "cplx_bf16.hip", "cbwd_f32.hip", "cbwd_bf16.hip",
           "ssd_f32.hip", "ssd_bf16.hip", "probe.hip", "noalloc.hip"]

# Packed-FP32 instructions are switched off for every device pass.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", CSRC, "-I", INCLUDE]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libssmscan)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False, isa_dir: str = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmd = [cc, *COMMON, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        cmds.append(cmd)
        if isa_dir and src.endswith(".hip"):
            os.makedirs(isa_dir, exist_ok=True)
            asm = os.path.join(isa_dir, os.path.splitext(src)[0] + f"-{ARCH}.s")
            cmds.append([cc, *COMMON, "-x", "hip", "--cuda-device-only", "-S",
                         os.path.join(CSRC, src), "-o", asm])
    with ThreadPoolExecutor(max_workers=min(8, len(cmds))) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB + ".tmp"
    _run([cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


SAN_DIR = os.path.join(BUILD, "san")
SAN_LIB = os.path.join(SAN_DIR, "libssmscan.so")
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]


def build_sanitized(verbose: bool = False) -> str:
    """The library with its host-side argument validation, planning and
    dispatch (abi.cpp) built by g++ with AddressSanitizer and
    UndefinedBehaviorSanitizer, linked with the device objects of the normal
    build (which runs first if they are missing).  For CPU runs with gcc's
    libasan preloaded, the library selected through SSMSCAN_LIB."""
    objs = [os.path.join(BUILD, os.path.splitext(src)[0] + ".o") for src in SOURCES if src != "abi.cpp"]
    if not all(os.path.exists(o) for o in objs):
        build(verbose=verbose)
    os.makedirs(SAN_DIR, exist_ok=True)
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    abi = os.path.join(SAN_DIR, "abi.o")
    _run(["g++", "-std=c++17", "-O1", "-fPIC", *SAN_FLAGS, "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(rocm, "include"),
          "-I", CSRC, "-I", INCLUDE, "-c", os.path.join(CSRC, "abi.cpp"), "-o", abi], verbose)
    tmp = SAN_LIB + ".tmp"
    _run(["g++", "-shared", *SAN_FLAGS, abi, *objs, "-L", os.path.join(rocm, "lib"), "-lamdhip64",
          f"-Wl,-rpath,{os.path.join(rocm, 'lib')}", "-o", tmp], verbose)
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("-v", action="store_true")
    ap.add_argument("--isa", default=None)
    ap.add_argument("--sanitize", action="store_true", help="build the ASan/UBSan host variant instead")
    a = ap.parse_args()
    print(build_sanitized(verbose=a.v) if a.sanitize else build(verbose=a.v, isa_dir=a.isa))
