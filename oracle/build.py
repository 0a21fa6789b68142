"""Build the fp64 reference oracle (test infrastructure) with gcc.

Compiles ``ssm_oracle.c`` into ``liboracle.so`` next to this file: -O2, OpenMP,
no fast-math (the oracle must keep IEEE double semantics).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ssm_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")
# AddressSanitizer + UndefinedBehaviorSanitizer build of the same source, for
# the CPU hygiene run (loaded through SSM_ORACLE_LIB with gcc's libasan
# preloaded).
SAN_LIB = os.path.join(HERE, "_build", "liboracle_san.so")
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]


def build(verbose: bool = False, sanitize: bool = False) -> str:
    out = SAN_LIB if sanitize else LIB
    os.makedirs(os.path.dirname(out), exist_ok=True)
    cmd = ["gcc", "-O1" if sanitize else "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wextra",
           *(SAN_FLAGS if sanitize else []), SRC, "-o", out + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
