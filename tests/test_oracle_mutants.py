"""Plant plausible mistakes in a copy of the oracle (on the CPU) and show that
the pins catch each of them.  The planted copies live in a temporary directory;
the real oracle source is only read."""
import os
import subprocess

import pytest

import _pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "ssm_oracle.c")

# (name, text to replace, replacement)
MUTANTS = [
    ("drop_D_term", "return y + dskip * xt;", "return y;"),
    ("y_uses_old_state",
     "h[n] = abar * h[n] + bbar * xt;\n        y += c[n] * h[n];",
     "y += c[n] * h[n];\n        h[n] = abar * h[n] + bbar * xt;"),
    ("wrong_sign_in_exp", "const double abar = exp(z);", "const double abar = exp(-z);"),
    ("bbar_missing_delta", "bbar = dt * zoh_phi(z) * b[n];", "bbar = zoh_phi(z) * b[n];"),
    ("euler_instead_of_zoh", "bbar = dt * zoh_phi(z) * b[n];", "bbar = dt * b[n];"),
    ("phi_missing_division", "return expm1(z) / z;", "return expm1(z);"),
    ("B_and_C_swapped", "B + r,\n                                        C + r,",
     "C + r,\n                                        B + r,"),
    ("B_C_ignore_batch", "const int64_t r = (b * L + t) * N;", "const int64_t r = t * N;"),
    ("delta_from_channel_0", "step_size(delta[i], bias_d", "step_size(delta[(b * L + t) * Dm], bias_d"),
    ("A_row_of_channel_0_in_scan", "dt, A + d * N, B + r", "dt, A, B + r"),
    ("D_of_channel_0", "C + r, D[d], N, euler);", "C + r, D[0], N, euler);"),
    ("initial_state_ignored", "h[n] = h0 ? h0[(b * Dm + d) * N + n] : 0.0;", "h[n] = 0.0;"),
    ("step_B_ignores_batch", "B + b * N, C + b * N", "B, C + b * N"),
    ("step_A_row_of_channel_0", "dt, A + d * N,\n                                B + b * N",
     "dt, A,\n                                B + b * N"),
    # delta pre-processing and the Euler input term
    ("softplus_flag_ignored", "return (flags & ORACLE_DELTA_SOFTPLUS) ? softplus(v) : v;", "return v;"),
    ("softplus_always_on", "return (flags & ORACLE_DELTA_SOFTPLUS) ? softplus(v) : v;", "return softplus(v);"),
    ("bias_ignored", "const double v = raw + bias;", "const double v = raw;"),
    ("bias_subtracted", "const double v = raw + bias;", "const double v = raw - bias;"),
    ("softplus_positive_branch_drops_v", "return v + log1p(exp(-v));", "return log1p(exp(-v));"),
    ("softplus_naive_tail", "return log1p(exp(v));\n}", "return log(1.0 + exp(v));\n}"),
    ("softplus_naive_overflow", "    if (v > 0.0)\n        return v + log1p(exp(-v));\n", ""),
    ("scan_bias_of_channel_0", "const double bias_d = bias ? bias[d] : 0.0;",
     "const double bias_d = bias ? bias[0] : 0.0;"),
    ("step_bias_of_channel_0", "bias ? bias[d] : 0.0, flags);", "bias ? bias[0] : 0.0, flags);"),
    ("euler_uses_zoh", "            bbar = dt * b[n];\n", "            bbar = dt * zoh_phi(z) * b[n];\n"),
    ("euler_drops_delta", "            bbar = dt * b[n];\n", "            bbar = b[n];\n"),
    ("euler_forward_abar", "const double abar = exp(z);", "const double abar = euler ? 1.0 + z : exp(z);"),
    ("euler_ignored_in_step", "const int euler = (flags & ORACLE_EULER_B) != 0;\n    for (int64_t b",
     "const int euler = 0;\n    for (int64_t b"),
    ("euler_ignored_in_scan", "const int euler = (flags & ORACLE_EULER_B) != 0;\n    const int64_t nchan",
     "const int euler = 0;\n    const int64_t nchan"),
    ("h_final_not_last_state",
     "h_final[(b * Dm + d) * N + n] = h[n];",
     "h_final[(b * Dm + d) * N + n] = h[n] * 0.5 + 0.5 * h[n] * (n == 0 ? 1.0 : 0.999);"),
]


def _build_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutant {name}: pattern must occur exactly once"
    path = tmp_path / f"{name}.c"
    path.write_text(src.replace(old, new))
    lib = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-fopenmp", str(path),
                    "-o", str(lib), "-lm"], check=True)
    return str(lib)


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, name, old, new):
    import oracle
    mut = oracle.Oracle(_build_mutant(tmp_path, name, old, new))
    failed = []
    for check in _pins.ALL_CHECKS:
        try:
            check(mut)
        except AssertionError:
            failed.append(getattr(check, "__name__", "check"))
    assert failed, f"no pin caught the planted mistake '{name}'"
