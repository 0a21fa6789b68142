"""CPU hygiene run: the library's host code (argument validation, planning,
scratch and dispatch in abi.cpp) and the fp64 oracle, each built with
AddressSanitizer and UndefinedBehaviorSanitizer, run the C-ABI checks and the
oracle pins in a child process with gcc's sanitizer runtimes preloaded.  Any
sanitizer report aborts the child (halt_on_error), which fails this test."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    r = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


@pytest.fixture(scope="module")
def san_env():
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if asan is None or ubsan is None:
        pytest.skip("gcc's sanitizer runtimes are not installed")
    sys.path.insert(0, ROOT)
    from selective_state_space_18_amd import build as lib_build
    from oracle import build as oracle_build
    lib = lib_build.build_sanitized()
    orc = oracle_build.build(sanitize=True)
    env = dict(os.environ)
    env.update(SSMSCAN_LIB=lib, SSM_ORACLE_LIB=orc, LD_PRELOAD=f"{asan}:{ubsan}",
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    return env, lib, orc


def test_sanitized_builds_are_the_ones_loaded(san_env):
    env, lib, orc = san_env
    code = ("import ctypes, oracle\n"
            "from selective_state_space_18_amd import ssmscan\n"
            "ssmscan.lib(); oracle.load()\n"
            "maps = open('/proc/self/maps').read()\n"
            f"assert {lib!r} in maps and {orc!r} in maps and 'libasan' in maps, 'not loaded'\n"
            "print('loaded')\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and "loaded" in r.stdout, r.stdout + r.stderr


def test_abi_checks_and_oracle_pins_under_sanitizers(san_env):
    env, _, _ = san_env
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "tests/test_abi_cpu.py", "tests/test_oracle_pins.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = "\n".join((r.stdout + r.stderr).splitlines()[-30:])
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "failed" not in r.stdout, tail
