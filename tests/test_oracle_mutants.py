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
    ("drop_D_term", "y += c[n] * h[n];\n    }\n    return y + dskip * xt;", "y += c[n] * h[n];\n    }\n    return y;"),
    ("y_uses_old_state",
     "h[n] = abar * h[n] + bbar * xt;\n        y += c[n] * h[n];",
     "y += c[n] * h[n];\n        h[n] = abar * h[n] + bbar * xt;"),
    ("wrong_sign_in_exp", "const double abar = exp(z);\n        double bbar;",
     "const double abar = exp(-z);\n        double bbar;"),
    ("bbar_missing_delta", "bbar = dt * zoh_phi(z) * b[n];", "bbar = zoh_phi(z) * b[n];"),
    ("euler_instead_of_zoh", "bbar = dt * zoh_phi(z) * b[n];", "bbar = dt * b[n];"),
    ("phi_missing_division", "return expm1(z) / z;", "return expm1(z);"),
    ("B_and_C_swapped", "B + r,\n                                        C + r,",
     "C + r,\n                                        B + r,"),
    ("B_C_ignore_batch", "const int64_t r = (b * L + t) * N;\n                    const double dt = step_size(delta[i], bias_d, flags);\n                    y[i]",
     "const int64_t r = t * N;\n                    const double dt = step_size(delta[i], bias_d, flags);\n                    y[i]", 0),
    ("delta_from_channel_0", "step_size(delta[i], bias_d, flags);\n                    y[i]",
     "step_size(delta[(b * L + t) * Dm], bias_d, flags);\n                    y[i]", 0),
    ("A_row_of_channel_0_in_scan", "dt, A + d * N, B + r", "dt, A, B + r"),
    ("D_of_channel_0", "C + r, D[d], N, euler);", "C + r, D[0], N, euler);", 0),
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
    ("scan_bias_of_channel_0", "const double bias_d = bias ? bias[d] : 0.0;\n                for (int64_t n = 0; n < N; ++n)\n                    h[n]",
     "const double bias_d = bias ? bias[0] : 0.0;\n                for (int64_t n = 0; n < N; ++n)\n                    h[n]"),
    ("step_bias_of_channel_0", "bias ? bias[d] : 0.0, flags);", "bias ? bias[0] : 0.0, flags);", 0),
    ("euler_uses_zoh", "            bbar = dt * b[n];\n", "            bbar = dt * zoh_phi(z) * b[n];\n"),
    ("euler_drops_delta", "            bbar = dt * b[n];\n", "            bbar = b[n];\n"),
    ("euler_forward_abar", "const double abar = exp(z);\n        double bbar;",
     "const double abar = euler ? 1.0 + z : exp(z);\n        double bbar;"),
    ("euler_ignored_in_step", "const int euler = (flags & ORACLE_EULER_B) != 0;\n    for (int64_t b",
     "const int euler = 0;\n    for (int64_t b", 0),
    ("euler_ignored_in_scan", "const int euler = (flags & ORACLE_EULER_B) != 0;\n    const int64_t nchan",
     "const int euler = 0;\n    const int64_t nchan", 0),
    # backward
    ("bwd_dx_drops_D", "double gx = D[d] * g, gdt = 0.0;", "double gx = 0.0, gdt = 0.0;", 0),
    ("bwd_lambda_uses_C_of_state_0", "lam[n] += C[r + n] * g;", "lam[n] += C[r] * g;", 0),
    ("bwd_zoh_dk_ddelta_missing_abar", "const double dk_ddt = euler ? 1.0 : abar;",
     "const double dk_ddt = euler ? 1.0 : 1.0;"),
    ("bwd_euler_dk_ddelta_is_abar", "const double dk_ddt = euler ? 1.0 : abar;",
     "const double dk_ddt = euler ? abar : abar;"),
    ("bwd_dk_dA_constant", "dt * dt * zoh_dphi(z);", "dt * dt * 0.5;"),
    ("bwd_dphi_series_wrong", "term *= z * (double)(m + 1) / ((double)m * (double)(m + 2));",
     "term *= z / (double)(m + 2);", 0),
    ("bwd_uses_h_t_for_h_prev", "const double hprev = hs[t * N + n];", "const double hprev = hs[(t + 1) * N + n];"),
    ("bwd_dC_uses_h_prev", "myC[r + n] += g * hs[(t + 1) * N + n];", "myC[r + n] += g * hs[t * N + n];"),
    ("bwd_lambda_not_decayed", "                            lam[n] *= abar;\n", ""),
    ("bwd_softplus_chain_missing", "                            gdt *= sigmoid(delta[i] + bias_d);\n",
     "                            gdt *= 1.0;\n", 0),
    ("bwd_sigmoid_without_bias", "gdt *= sigmoid(delta[i] + bias_d);", "gdt *= sigmoid(delta[i]);", 0),
    ("bwd_dB_missing_x", "myB[r + n] += lam[n] * k * x[i];", "myB[r + n] += lam[n] * k;"),
    ("bwd_dA_missing_abar", "dAd[n] += lam[n] * (dt * abar * hprev", "dAd[n] += lam[n] * (dt * hprev"),
    ("bwd_ddelta_missing_A", "gdt += lam[n] * (a[n] * abar * hprev", "gdt += lam[n] * (abar * hprev"),
    ("bwd_dh_final_ignored", "lam[n] = dh_final ? dh_final[(b * Dm + d) * N + n] : 0.0;", "lam[n] = 0.0;"),
    ("bwd_dbias_overwritten", "dbias_d += gdt;", "dbias_d = gdt;", 0),
    ("bwd_forward_ignores_euler", "const double k = euler ? dt : dt * zoh_phi(z);\n                            hs[",
     "const double k = dt * zoh_phi(z);\n                            hs["),
    # complex A
    ("cplx_rotation_sign", "h[2 * n] = abr * hr - abi * hi + kr * u;", "h[2 * n] = abr * hr + abi * hi + kr * u;"),
    ("cplx_no_imag_coupling", "h[2 * n + 1] = abr * hi + abi * hr + ki * u;", "h[2 * n + 1] = abr * hi + ki * u;"),
    ("cplx_y_uses_imag", "y += c[n] * h[2 * n];", "y += c[n] * h[2 * n + 1];"),
    ("cplx_phi_conjugate", "ki = dt * (ei * zr - er * zi) / den;", "ki = dt * (er * zi - ei * zr) / den;"),
    ("cplx_sin_for_cos", "const double abr = mag * cos(zi), abi = mag * sin(zi);",
     "const double abr = mag * sin(zi), abi = mag * cos(zi);"),
    ("cplx_expm1_missing_term", "*er = expm1(zr) * cos(zi) - 2.0 * s * s;", "*er = expm1(zr) * cos(zi);"),
    ("cplx_imag_A_ignored", "zi = dt * a[2 * n + 1];", "zi = 0.0 * a[2 * n + 1];"),
    ("cplx_euler_ignored", "        if (euler) {\n            kr = dt;", "        if (0) {\n            kr = dt;"),
    ("cplx_h0_imag_dropped", "h[k] = h0 ? h0[(b * Dm + d) * 2 * N + k] : 0.0;",
     "h[k] = h0 && (k % 2 == 0) ? h0[(b * Dm + d) * 2 * N + k] : 0.0;"),
    ("cplx_D_of_channel_0", "C + r, D[d], N, euler);", "C + r, D[0], N, euler);", 1),
    ("cplx_euler_ignored_in_scan", "const int euler = (flags & ORACLE_EULER_B) != 0;\n    const int64_t nchan",
     "const int euler = 0;\n    const int64_t nchan", 1),
    # backward of the complex-A scan
    ("cbwd_adjoint_not_conjugated", "lam[n] *= conj(abar);", "lam[n] *= abar;"),
    ("cbwd_G_abar_without_conj", "lam[n] * conj(hprev);", "lam[n] * hprev;"),
    ("cbwd_du_without_conj", "creal(lam[n] * conj(k));", "creal(lam[n] * k);"),
    ("cbwd_dk_dA_not_conjugated", "gk * conj(dt * dt * cdphi(z));", "gk * dt * dt * cdphi(z);"),
    ("cbwd_ddelta_missing_A", "creal(gabar * conj(An * abar));", "creal(gabar * conj(abar));"),
    ("cbwd_dA_missing_abar", "dAd[n] += gabar * conj(dt * abar) + gk", "dAd[n] += gabar * conj(dt) + gk"),
    ("cbwd_euler_dk_ddelta_is_abar", "                                gdt += creal(gk);\n",
     "                                gdt += creal(gk * conj(abar));\n"),
    ("cbwd_dphi_series_wrong", "term *= z * (double)(m + 1) / ((double)m * (double)(m + 2));",
     "term *= z * (double)(m + 1) / ((double)m * (double)(m + 3));", 1),
    ("cbwd_dphi_closed_form_sign", "return (z * cexp(z) - (er + I * ei)) / (z * z);",
     "return (z * cexp(z) + (er + I * ei)) / (z * z);"),
    ("cbwd_C_into_imag_part", "lam[n] += C[r + n] * g;", "lam[n] += I * C[r + n] * g;", 1),
    ("cbwd_dh_final_imag_ignored", "dh_final[j] + I * dh_final[j + 1]", "dh_final[j]"),
    ("cbwd_dh0_imag_dropped", "dh0[j + 1] = cimag(lam[n]);", "dh0[j + 1] = 0.0;"),
    ("cbwd_dC_uses_h_prev", "myC[r + n] += g * hs[(t + 1) * 2 * N + 2 * n];", "myC[r + n] += g * hs[t * 2 * N + 2 * n];"),
    ("cbwd_h0_imag_dropped_in_forward", "hs[k] = h0 ? h0[(b * Dm + d) * 2 * N + k] : 0.0;",
     "hs[k] = h0 && k % 2 == 0 ? h0[(b * Dm + d) * 2 * N + k] : 0.0;"),
    ("h_final_not_last_state",
     "h_final[(b * Dm + d) * N + n] = h[n];",
     "h_final[(b * Dm + d) * N + n] = h[n] * 0.5 + 0.5 * h[n] * (n == 0 ? 1.0 : 0.999);"),
]


def _build_mutant(tmp_path, name, old, new, occurrence=None):
    """Replace `old` by `new` in a copy of the oracle: `old` must occur exactly
    once, or `occurrence` picks one of several (0 = first)."""
    src = open(SRC).read()
    if occurrence is None:
        assert src.count(old) == 1, f"mutant {name}: pattern must occur exactly once"
        start = src.index(old)
    else:
        start = -1
        for _ in range(occurrence + 1):
            start = src.index(old, start + 1)
    path = tmp_path / f"{name}.c"
    path.write_text(src[:start] + new + src[start + len(old):])
    lib = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-fopenmp", str(path),
                    "-o", str(lib), "-lm"], check=True)
    return str(lib)


@pytest.mark.parametrize("mutant", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, mutant):
    import oracle
    name, old, new = mutant[:3]
    occurrence = mutant[3] if len(mutant) > 3 else None
    # one thread: the checks make many tiny calls, and test workers run side by side
    mut = oracle.Oracle(_build_mutant(tmp_path, name, old, new, occurrence), threads=1)
    for check in _pins.ALL_CHECKS:
        try:
            check(mut)
        except AssertionError:
            return  # caught
    pytest.fail(f"no pin caught the planted mistake '{name}'")


# Mistakes in the Python front-end of the scalar-decay layer (head mapping and
# per-head parameters), planted in a subclass of the real oracle.
def _ssd_mutant(kind):
    import numpy as np
    import oracle

    class Broken(oracle.Oracle):
        def scan_ssd(self, x, delta, A, B, C, D, head_dim, h0=None, threads=0, delta_bias=None,
                     delta_softplus=False, euler_b=False):
            x = np.asarray(x)
            Bsz, L, Dm = x.shape
            P = int(head_dim)
            H = Dm // P
            N = np.asarray(B).shape[2]
            A = np.asarray(A, dtype=np.float64)
            delta = np.asarray(delta, dtype=np.float64)
            rep = (lambda a, axis=0: np.tile(a, P) if axis == 0 else np.tile(a, (1, 1, P))) \
                if kind == "heads_interleaved" else (lambda a, axis=0: np.repeat(a, P, axis=axis))
            A_full = rep(A)[:, None] * np.ones((1, N))
            delta_full = rep(delta, 2)
            if kind == "delta_of_head_0":
                delta_full = np.repeat(delta[:, :, :1], Dm, axis=2)
            bias = None
            if delta_bias is not None:
                bias = np.repeat(np.asarray(delta_bias, dtype=np.float64), P)
                if kind == "bias_ignored":
                    bias = None
            if kind == "A_of_head_0":
                A_full = np.full((Dm, N), A[0])
            return self.scan(x, delta_full, A_full, B, C, D, h0=h0, threads=threads, delta_bias=bias,
                             delta_softplus=delta_softplus, euler_b=euler_b)

    return Broken(threads=1)


@pytest.mark.parametrize("kind", ["heads_interleaved", "delta_of_head_0", "bias_ignored", "A_of_head_0"])
def test_pins_catch_ssd_front_end_mistake(kind):
    with pytest.raises(AssertionError):
        _pins.check_ssd_duality(_ssd_mutant(kind))
