"""Pins for the fp64 oracle: checks against what the pages and mathematics fix.

Each ``check_*`` takes an object with the oracle's ``scan``/``step`` interface
and raises AssertionError on a mismatch.  They are run against the real oracle
(tests/test_oracle_pins.py) and against deliberately broken copies of it
(tests/test_oracle_mutants.py) to show that a plausible slip in the oracle
fails at least one of them.

None of these checks re-types the oracle's recurrence: they use the
matrix-exponential (Van Loan) form of the zero-order hold, the unrolled
closed-form sum, the LTI convolution mode, a library IIR filter, exact limits
and invariants, and hand-derived worked examples.
"""
import json
import os

import numpy as np
from scipy.linalg import expm
from scipy.signal import lfilter

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "closed_forms.json")


def rel_err(a, b, floor_frac=0.1):
    """max |a-b| / max(|b|, floor_frac * rms(b)) -- elementwise, RMS-floored."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if b.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(b * b))) if b.size else 0.0
    den = np.maximum(np.abs(b), floor_frac * rms + 1e-300)
    return float(np.max(np.abs(a - b) / den))


# ---------------------------------------------------------------------------
# independent evaluations


def vanloan_zoh(a, dt, b=1.0):
    """(Abar, Bbar) for h' = a h + b u with u held over [0, dt].

    exp(dt * [[a, b], [0, 0]]) = [[Abar, Bbar], [0, 1]] -- the augmented-matrix
    identity for the zero-order hold; it does not use the (e^z - 1)/A formula.
    """
    M = np.array([[a * dt, b * dt], [0.0, 0.0]], dtype=np.float64)
    E = expm(M)
    return E[0, 0], E[0, 1]


def brute_force_scan(x, delta, A, B, C, D, h0=None):
    """Unrolled closed form, O(L^2 N) per channel:

    y_t = sum_{s<=t} sum_n C_t[n] (prod_{s<r<=t} Abar_r[n]) Bbar_s[n] x_s
          + sum_n C_t[n] (prod_{r<=t} Abar_r[n]) h0[n] + D x_t
    """
    Bsz, L, Dm = x.shape
    N = A.shape[1]
    Ab = np.empty((Bsz, L, Dm, N))
    Bb = np.empty((Bsz, L, Dm, N))
    for b in range(Bsz):
        for t in range(L):
            for d in range(Dm):
                for n in range(N):
                    Ab[b, t, d, n], Bb[b, t, d, n] = vanloan_zoh(A[d, n], delta[b, t, d], B[b, t, n])
    y = np.zeros((Bsz, L, Dm))
    hf = np.zeros((Bsz, Dm, N))
    for b in range(Bsz):
        for d in range(Dm):
            for n in range(N):
                for t in range(L):
                    # state h_t as an explicit sum over the inputs s <= t
                    h_t = 0.0
                    for s in range(t + 1):
                        h_t += np.prod(Ab[b, s + 1:t + 1, d, n]) * Bb[b, s, d, n] * x[b, s, d]
                    if h0 is not None:
                        h_t += np.prod(Ab[b, 0:t + 1, d, n]) * h0[b, d, n]
                    y[b, t, d] += C[b, t, n] * h_t
                    if t == L - 1:
                        hf[b, d, n] = h_t
            for t in range(L):
                y[b, t, d] += D[d] * x[b, t, d]
    return y, hf


def random_case(rng, Bsz, L, Dm, N, a_lo=-3.0, a_hi=-0.05):
    x = rng.standard_normal((Bsz, L, Dm))
    delta = np.exp(rng.uniform(np.log(1e-3), np.log(0.5), (Bsz, L, Dm)))
    A = rng.uniform(a_lo, a_hi, (Dm, N))
    B = rng.standard_normal((Bsz, L, N))
    C = rng.standard_normal((Bsz, L, N))
    D = rng.standard_normal(Dm)
    return x, delta, A, B, C, D


# ---------------------------------------------------------------------------
# checks


def check_golden(orc):
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        A = np.array(c["A"], dtype=np.float64)
        N = A.shape[1]
        L = len(c["x"])
        x = np.array(c["x"], dtype=np.float64).reshape(1, L, 1)
        dl = np.array(c["delta"], dtype=np.float64).reshape(1, L, 1)
        B = np.tile(np.array(c["B"], dtype=np.float64).reshape(1, 1, N), (1, L, 1))
        C = np.tile(np.array(c["C"], dtype=np.float64).reshape(1, 1, N), (1, L, 1))
        D = np.array(c["D"], dtype=np.float64)
        y, hf = orc.scan(x, dl, A, B, C, D)
        ey = np.array(c["y"], dtype=np.float64)
        eh = np.array(c["h_final"], dtype=np.float64)
        assert np.allclose(y.reshape(-1), ey, rtol=1e-13, atol=1e-14), (c["name"], y.reshape(-1), ey)
        assert np.allclose(hf.reshape(-1), eh, rtol=1e-13, atol=1e-14), (c["name"], hf.reshape(-1), eh)


def check_brute_force(orc, seed=0, with_h0=False):
    rng = np.random.default_rng(seed)
    x, delta, A, B, C, D = random_case(rng, 2, 9, 3, 4)
    h0 = rng.standard_normal((2, 3, 4)) if with_h0 else None
    y, hf = orc.scan(x, delta, A, B, C, D, h0=h0)
    yb, hb = brute_force_scan(x, delta, A, B, C, D, h0=h0)
    assert rel_err(y, yb) < 1e-11, rel_err(y, yb)
    assert rel_err(hf, hb) < 1e-11, rel_err(hf, hb)


def check_vanloan_step(orc):
    """One step from h=0 with x=1, B=1 gives Bbar; from h=1 with x=0 gives Abar."""
    a_vals = np.array([-20.0, -3.0, -1.0, -0.25, -1e-3, -1e-9, 0.0, 0.5])
    d_vals = np.array([0.0, 1e-6, 1e-3, 0.05, 0.3, 1.0, 2.5])
    Dm, Bsz = len(a_vals), len(d_vals)
    # channel d has A = a_vals[d] (one state); batch row b uses delta = d_vals[b]
    A = a_vals.reshape(Dm, 1)
    x1 = np.ones((Bsz, Dm))
    dl = np.tile(d_vals.reshape(Bsz, 1), (1, Dm))
    ones = np.ones((Bsz, 1))
    zeros = np.zeros((Bsz, 1))
    _, hB = orc.step(x1, dl, A, ones, zeros, np.zeros(Dm), np.zeros((Bsz, Dm, 1)))
    _, hA = orc.step(np.zeros((Bsz, Dm)), dl, A, ones, zeros, np.zeros(Dm), np.ones((Bsz, Dm, 1)))
    for b in range(Bsz):
        for d in range(Dm):
            ea, eb = vanloan_zoh(a_vals[d], d_vals[b], 1.0)
            assert abs(hA[b, d, 0] - ea) <= 1e-14 * max(1.0, abs(ea)), (a_vals[d], d_vals[b], hA[b, d, 0], ea)
            assert abs(hB[b, d, 0] - eb) <= 1e-13 * abs(eb), (a_vals[d], d_vals[b], hB[b, d, 0], eb)


def check_lti_convolution(orc, seed=1):
    """Time-invariant delta, B, C: y = (K * x) + D x with K_k = sum_n C_n Abar_n^k Bbar_n;
    also per state h_n = lfilter([Bbar_n], [1, -Abar_n], x)."""
    rng = np.random.default_rng(seed)
    L, Dm, N = 40, 3, 5
    x = rng.standard_normal((1, L, Dm))
    dch = np.exp(rng.uniform(np.log(1e-2), np.log(0.7), Dm))
    delta = np.tile(dch.reshape(1, 1, Dm), (1, L, 1))
    A = -np.exp(rng.uniform(-2, 1.5, (Dm, N)))
    bvec = rng.standard_normal(N)
    cvec = rng.standard_normal(N)
    B = np.tile(bvec.reshape(1, 1, N), (1, L, 1))
    C = np.tile(cvec.reshape(1, 1, N), (1, L, 1))
    D = rng.standard_normal(Dm)
    y, hf = orc.scan(x, delta, A, B, C, D)
    for d in range(Dm):
        ab = np.exp(dch[d] * A[d])
        bb = np.array([vanloan_zoh(A[d, n], dch[d], bvec[n])[1] for n in range(N)])
        K = np.array([np.sum(cvec * ab ** k * bb) for k in range(L)])
        yc = np.array([np.sum(K[:t + 1][::-1] * x[0, :t + 1, d]) for t in range(L)]) + D[d] * x[0, :, d]
        assert rel_err(y[0, :, d], yc) < 1e-12, rel_err(y[0, :, d], yc)
        hs = np.stack([lfilter([bb[n]], [1.0, -ab[n]], x[0, :, d]) for n in range(N)], axis=1)
        yl = hs @ cvec + D[d] * x[0, :, d]
        assert rel_err(y[0, :, d], yl) < 1e-12
        assert rel_err(hf[0, d], hs[-1]) < 1e-12


def check_a_to_zero_limit(orc):
    """Bbar -> delta*B as A -> 0 (error O(delta^2 |A|)); A == 0 gives delta*B exactly."""
    dt, bval = 0.1, 1.7
    prev = None
    for k in range(3, 13):
        a = -10.0 ** (-k)
        _, h = orc.step(np.ones((1, 1)), np.full((1, 1), dt), np.full((1, 1), a), np.full((1, 1), bval),
                        np.zeros((1, 1)), np.zeros(1), np.zeros((1, 1, 1)))
        err = abs(h[0, 0, 0] - dt * bval)
        bound = 0.5 * dt * dt * abs(a) * bval * 1.01 + 4e-16 * dt * bval
        assert err <= bound, (k, err, bound)
        if prev is not None and k <= 9:
            assert err < prev, (k, err, prev)
        prev = err
    _, h = orc.step(np.ones((1, 1)), np.full((1, 1), dt), np.zeros((1, 1)), np.full((1, 1), bval),
                    np.zeros((1, 1)), np.zeros(1), np.zeros((1, 1, 1)))
    assert h[0, 0, 0] == dt * bval
    _, h = orc.step(np.zeros((1, 1)), np.full((1, 1), dt), np.zeros((1, 1)), np.full((1, 1), bval),
                    np.zeros((1, 1)), np.zeros(1), np.full((1, 1, 1), 0.37))
    assert h[0, 0, 0] == 0.37


def check_delta_zero_persistence(orc, seed=2):
    """delta = 0 from t0 on: the state is held exactly and y_t = C_t h + D x_t."""
    rng = np.random.default_rng(seed)
    x, delta, A, B, C, D = random_case(rng, 2, 16, 3, 4)
    t0 = 6
    delta[:, t0:, :] = 0.0
    y, hf = orc.scan(x, delta, A, B, C, D)
    _, hpre = orc.scan(x[:, :t0], delta[:, :t0], A, B[:, :t0], C[:, :t0], D)
    assert np.array_equal(hf, hpre)
    ye = np.einsum("btn,bdn->btd", C[:, t0:], hpre) + D[None, None, :] * x[:, t0:]
    assert rel_err(y[:, t0:], ye) < 1e-13


def check_pure_decay(orc, seed=3):
    """x = 0: h_L = exp(A * sum_t delta_t) h0 per state."""
    rng = np.random.default_rng(seed)
    Bsz, L, Dm, N = 2, 25, 3, 4
    _, delta, A, B, C, D = random_case(rng, Bsz, L, Dm, N)
    h0 = rng.standard_normal((Bsz, Dm, N))
    y, hf = orc.scan(np.zeros((Bsz, L, Dm)), delta, A, B, C, D, h0=h0)
    tot = delta.sum(axis=1)  # [Bsz, Dm]
    he = np.exp(tot[:, :, None] * A[None, :, :]) * h0
    assert rel_err(hf, he) < 1e-12, rel_err(hf, he)


def check_zoh_exact_for_constant_input(orc, seed=4):
    """Constant x, delta, B and h0 = 0: h after k steps equals the ODE solution
    at time k*delta, B x (exp(A k delta) - 1) / A, for every k."""
    rng = np.random.default_rng(seed)
    L, Dm, N = 12, 4, 3
    xv = rng.standard_normal(Dm)
    dv = rng.uniform(0.01, 0.4, Dm)
    bv = rng.standard_normal(N)
    A = -np.exp(rng.uniform(-1.5, 1.0, (Dm, N)))
    x = np.tile(xv.reshape(1, 1, Dm), (1, L, 1))
    delta = np.tile(dv.reshape(1, 1, Dm), (1, L, 1))
    B = np.tile(bv.reshape(1, 1, N), (1, L, 1))
    for n in range(N):
        C = np.zeros((1, L, N))
        C[..., n] = 1.0
        y, _ = orc.scan(x, delta, A, B, C, np.zeros(Dm))
        for k in range(1, L + 1):
            exact = bv[n] * xv * np.expm1(A[:, n] * k * dv) / A[:, n]
            assert rel_err(y[0, k - 1], exact) < 1e-12


def check_linearity_causality_permutation(orc, seed=5):
    rng = np.random.default_rng(seed)
    Bsz, L, Dm, N = 3, 14, 5, 4
    x1, delta, A, B, C, D = random_case(rng, Bsz, L, Dm, N)
    x2 = rng.standard_normal(x1.shape)
    y1, h1 = orc.scan(x1, delta, A, B, C, D)
    y2, h2 = orc.scan(x2, delta, A, B, C, D)
    y12, h12 = orc.scan(2.0 * x1 - 0.5 * x2, delta, A, B, C, D)
    assert rel_err(y12, 2.0 * y1 - 0.5 * y2) < 1e-11
    assert rel_err(h12, 2.0 * h1 - 0.5 * h2) < 1e-11
    # causality: perturbing x at t' leaves y_{t<t'} bitwise unchanged, changes y_{t'}
    tp = 7
    x3 = x1.copy()
    x3[:, tp] += 1.0
    y3, _ = orc.scan(x3, delta, A, B, C, D)
    assert np.array_equal(y3[:, :tp], y1[:, :tp])
    assert not np.array_equal(y3[:, tp], y1[:, tp])
    # channel and batch permutations permute the outputs (channels are independent)
    pd = rng.permutation(Dm)
    pb = rng.permutation(Bsz)
    yp, hp = orc.scan(x1[pb][:, :, pd], delta[pb][:, :, pd], A[pd], B[pb], C[pb], D[pd])
    assert np.array_equal(yp, y1[pb][:, :, pd])
    assert np.array_equal(hp, h1[pb][:, pd])


def check_step_chain_matches_scan(orc, seed=6):
    """Applying the step L times from h0 reproduces the scan's y and h_final
    (recurrent mode, 'Mamba SSM Nedir?' section 'Ayrik Zamana Gecis')."""
    rng = np.random.default_rng(seed)
    Bsz, L, Dm, N = 2, 10, 3, 4
    x, delta, A, B, C, D = random_case(rng, Bsz, L, Dm, N)
    h0 = rng.standard_normal((Bsz, Dm, N))
    y, hf = orc.scan(x, delta, A, B, C, D, h0=h0)
    h = h0
    for t in range(L):
        yt, h = orc.step(x[:, t], delta[:, t], A, B[:, t], C[:, t], D, h)
        assert rel_err(yt, y[:, t]) < 1e-13
    assert rel_err(h, hf) < 1e-13


def check_split_scan_operator(orc, seed=7):
    """The affine-map composition (a1,b1) o (a2,b2) = (a1 a2, a2 b1 + b2) used to
    carry the state between time chunks: evaluating the scan in arbitrary chunks
    and combining the chunk summaries reproduces the sequential oracle."""
    rng = np.random.default_rng(seed)
    Bsz, L, Dm, N = 1, 37, 2, 3
    x, delta, A, B, C, D = random_case(rng, Bsz, L, Dm, N)
    _, hf = orc.scan(x, delta, A, B, C, D)
    cuts = [0, 5, 6, 19, 31, L]
    carry = np.zeros((Bsz, Dm, N))
    for s, e in zip(cuts[:-1], cuts[1:]):
        _, h_loc = orc.scan(x[:, s:e], delta[:, s:e], A, B[:, s:e], C[:, s:e], D)
        decay = np.exp(delta[:, s:e].sum(axis=1)[:, :, None] * A[None])
        carry = decay * carry + h_loc
    assert rel_err(carry, hf) < 1e-12


# ---------------------------------------------------------------------------
# options: delta = softplus(raw + bias) and the Euler input term Bbar = delta*B


def read_delta(orc, raw, bias=None, softplus=True):
    """The step size the oracle derives from raw (+ bias), read off exactly:
    with A = 0 the input coefficient is delta itself (ZOH limit), so one step
    from h = 0 with x = 1 and B = 1 leaves h = delta."""
    raw = np.asarray(raw, dtype=np.float64).reshape(1, -1)
    Dm = raw.shape[1]
    _, h = orc.step(np.ones((1, Dm)), raw, np.zeros((Dm, 1)), np.ones((1, 1)), np.zeros((1, 1)),
                    np.zeros(Dm), np.zeros((1, Dm, 1)), delta_bias=bias, delta_softplus=softplus)
    return h[0, :, 0]


def check_softplus_closed_forms(orc):
    """softplus(v) = log(1 + e^v): its value at 0, its inverse log(e^u - 1),
    the identity softplus(v) - softplus(-v) = v, the tails e^v (v -> -inf)
    and v (v -> +inf), and numpy's logaddexp(0, v) on a grid."""
    assert abs(read_delta(orc, [0.0])[0] - np.log(2.0)) <= 2e-16
    u = np.array([1e-6, 1e-3, 0.1, 1.0, 5.0, 30.0])
    got = read_delta(orc, np.log(np.expm1(u)))
    assert np.all(np.abs(got - u) <= 1e-14 * u), (got, u)
    v = np.array([0.5, 3.0, 20.0, 40.0])
    pos, neg = read_delta(orc, v), read_delta(orc, -v)
    assert np.all(np.abs((pos - neg) - v) <= 1e-14 * v)
    tail = np.array([-40.0, -100.0, -700.0])
    assert np.all(np.abs(read_delta(orc, tail) - np.exp(tail)) <= 1e-14 * np.exp(tail))
    assert np.array_equal(read_delta(orc, [800.0, 1e4]), np.array([800.0, 1e4]))
    grid = np.linspace(-30.0, 30.0, 121)
    ref = np.logaddexp(0.0, grid)
    assert np.all(np.abs(read_delta(orc, grid) - ref) <= 4e-16 * np.maximum(ref, 1.0))
    # the per-channel bias is added before softplus; without the flag delta = raw + bias
    raw = np.array([0.3, -1.2, 2.0, -0.75])
    bias = np.array([-0.3, 1.2, 0.5, 0.25])
    got = read_delta(orc, raw, bias)
    assert abs(got[0] - np.log(2.0)) <= 2e-16 and abs(got[1] - np.log(2.0)) <= 2e-16
    assert np.allclose(got[2:], np.logaddexp(0.0, raw[2:] + bias[2:]), rtol=1e-15, atol=0)
    assert np.array_equal(read_delta(orc, raw, bias, softplus=False), raw + bias)


def check_fused_delta_matches_precomputed(orc, seed=8):
    """The scan and the step with (raw, bias, softplus) equal the plain ones fed
    delta = logaddexp(0, raw + bias) computed by numpy."""
    rng = np.random.default_rng(seed)
    Bsz, L, Dm, N = 2, 12, 5, 3
    x, _, A, B, C, D = random_case(rng, Bsz, L, Dm, N)
    raw = rng.normal(0.0, 0.5, (Bsz, L, Dm))
    bias = np.log(np.expm1(rng.uniform(1e-3, 0.1, Dm)))
    h0 = rng.standard_normal((Bsz, Dm, N))
    delta = np.logaddexp(0.0, raw + bias[None, None, :])
    for euler in (False, True):
        y1, h1 = orc.scan(x, raw, A, B, C, D, h0=h0, delta_bias=bias, delta_softplus=True, euler_b=euler)
        y2, h2 = orc.scan(x, delta, A, B, C, D, h0=h0, euler_b=euler)
        assert rel_err(y1, y2) < 1e-13 and rel_err(h1, h2) < 1e-13, (euler, rel_err(y1, y2))
        ys, hs = orc.step(x[:, 0], raw[:, 0], A, B[:, 0], C[:, 0], D, h0, delta_bias=bias,
                          delta_softplus=True, euler_b=euler)
        yp, hp = orc.step(x[:, 0], delta[:, 0], A, B[:, 0], C[:, 0], D, h0, euler_b=euler)
        assert rel_err(ys, yp) < 1e-13 and rel_err(hs, hp) < 1e-13


def check_euler_b_closed_forms(orc, seed=9):
    """Euler input term Bbar = delta*B with Abar = exp(delta*A):
    constant inputs give the geometric sum h_k = delta B x (1 - Abar^k)/(1 - Abar);
    time-varying x with constant delta is scipy's lfilter([delta B], [1, -Abar], x);
    A = 0 coincides with the ZOH; with x = 0 (pure decay) it coincides with ZOH."""
    rng = np.random.default_rng(seed)
    L, Dm, N = 15, 4, 3
    xv = rng.standard_normal(Dm)
    dv = rng.uniform(0.01, 0.4, Dm)
    bv = rng.standard_normal(N)
    A = -np.exp(rng.uniform(-1.5, 1.0, (Dm, N)))
    x = np.tile(xv.reshape(1, 1, Dm), (1, L, 1))
    delta = np.tile(dv.reshape(1, 1, Dm), (1, L, 1))
    B = np.tile(bv.reshape(1, 1, N), (1, L, 1))
    for n in range(N):
        C = np.zeros((1, L, N))
        C[..., n] = 1.0
        y, _ = orc.scan(x, delta, A, B, C, np.zeros(Dm), euler_b=True)
        for k in range(1, L + 1):
            z = dv * A[:, n]
            exact = dv * bv[n] * xv * np.expm1(k * z) / np.expm1(z)
            assert rel_err(y[0, k - 1], exact) < 1e-12
    xs = rng.standard_normal((1, L, Dm))
    Ct = np.tile(rng.standard_normal(N).reshape(1, 1, N), (1, L, 1))
    y, hf = orc.scan(xs, delta, A, B, Ct, np.zeros(Dm), euler_b=True)
    for d in range(Dm):
        ab = np.exp(dv[d] * A[d])
        hs = np.stack([lfilter([dv[d] * bv[n]], [1.0, -ab[n]], xs[0, :, d]) for n in range(N)], axis=1)
        assert rel_err(y[0, :, d], hs @ Ct[0, 0]) < 1e-12
        assert rel_err(hf[0, d], hs[-1]) < 1e-12
    xr, dr, _, Br, Cr, Dr = random_case(rng, 2, 9, 3, 4)
    A0 = np.zeros((3, 4))
    ye, he = orc.scan(xr, dr, A0, Br, Cr, Dr, euler_b=True)
    yz, hz = orc.scan(xr, dr, A0, Br, Cr, Dr)
    assert np.array_equal(ye, yz) and np.array_equal(he, hz)
    Ar = -np.exp(rng.uniform(-1.0, 1.0, (3, 4)))
    h0 = rng.standard_normal((2, 3, 4))
    xz = np.zeros_like(xr)
    ye, he = orc.scan(xz, dr, Ar, Br, Cr, Dr, h0=h0, euler_b=True)
    yz, hz = orc.scan(xz, dr, Ar, Br, Cr, Dr, h0=h0)
    assert np.array_equal(ye, yz) and np.array_equal(he, hz)


def check_options_step_chain_matches_scan(orc, seed=10):
    """Recurrent mode with the options on: L steps equal the scan."""
    rng = np.random.default_rng(seed)
    Bsz, L, Dm, N = 2, 8, 3, 4
    x, _, A, B, C, D = random_case(rng, Bsz, L, Dm, N)
    raw = rng.normal(-1.0, 1.0, (Bsz, L, Dm))
    bias = rng.normal(0.0, 0.5, Dm)
    h0 = rng.standard_normal((Bsz, Dm, N))
    opts = dict(delta_bias=bias, delta_softplus=True, euler_b=True)
    y, hf = orc.scan(x, raw, A, B, C, D, h0=h0, **opts)
    h = h0
    for t in range(L):
        yt, h = orc.step(x[:, t], raw[:, t], A, B[:, t], C[:, t], D, h, **opts)
        assert rel_err(yt, y[:, t]) < 1e-13
    assert rel_err(h, hf) < 1e-13


# ---------------------------------------------------------------------------
# backward: finite differences of the forward oracle, adjoint identities


def _bwd_case(rng, opts, Bsz=2, L=7, Dm=3, N=4):
    x, delta, A, B, C, D = random_case(rng, Bsz, L, Dm, N)
    A[0, 1] = 0.0      # exact A = 0 (limit of the ZOH input term and of its derivative)
    A[1, 2] = -1e-7    # tiny A
    h0 = rng.standard_normal((Bsz, Dm, N))
    dy = rng.standard_normal((Bsz, L, Dm))
    dhf = rng.standard_normal((Bsz, Dm, N))
    bias = None
    if opts.get("delta_softplus"):
        delta = rng.normal(-2.0, 1.0, delta.shape)   # raw projection output
        bias = rng.normal(0.0, 0.5, Dm)
    return dict(x=x, delta=delta, A=A, B=B, C=C, D=D, h0=h0), dy, dhf, bias


def _loss(orc, p, dy, dhf, bias, opts):
    y, hf = orc.scan(p["x"], p["delta"], p["A"], p["B"], p["C"], p["D"], h0=p["h0"], delta_bias=bias, **opts)
    return float(np.sum(dy * y) + np.sum(dhf * hf))


def check_bwd_finite_differences(orc, seed=12):
    """Every gradient against central differences of L = <dy, y> + <dhf, h_final>
    computed with the forward oracle, for ZOH, softplus(delta + bias), and the
    Euler input term."""
    for k, opts in enumerate(({}, {"delta_softplus": True}, {"delta_softplus": True, "euler_b": True},
                              {"euler_b": True})):
        rng = np.random.default_rng(seed + k)
        p, dy, dhf, bias = _bwd_case(rng, opts)
        g = orc.scan_bwd(p["x"], p["delta"], p["A"], p["B"], p["C"], p["D"], dy, h0=p["h0"], dh_final=dhf,
                         delta_bias=bias, **opts)
        names = {"x": "dx", "delta": "ddelta", "A": "dA", "B": "dB", "C": "dC", "D": "dD", "h0": "dh0"}
        params = dict(p)
        if bias is not None:
            params["bias"] = bias
            names["bias"] = "dbias"
        scale = max(1.0, max(float(np.max(np.abs(g[v]))) for v in names.values()))
        for name, gname in names.items():
            arr = params[name]
            got = g[gname]
            for idx in np.ndindex(arr.shape):
                old = arr[idx]
                eps = 1e-6 * max(1.0, abs(old))
                arr[idx] = old + eps
                lp = _loss(orc, p, dy, dhf, params.get("bias"), opts)
                arr[idx] = old - eps
                lm = _loss(orc, p, dy, dhf, params.get("bias"), opts)
                arr[idx] = old
                fd = (lp - lm) / (2 * eps)
                assert abs(fd - got[idx]) <= 2e-7 * scale + 1e-6 * abs(fd), (opts, name, idx, fd, got[idx])


def check_bwd_adjoint_identities(orc, seed=16):
    """Exact identities (no differencing): with delta, A fixed the outputs are
    linear in (x, h0), in B when h0 = 0, and y - D x is linear in C, so
    <dy, y(v)> + <dhf, h_final(v)> = <gradient, v> for each of them."""
    rng = np.random.default_rng(seed)
    for opts in ({}, {"euler_b": True}):
        p, dy, dhf, _ = _bwd_case(rng, opts, Bsz=2, L=11, Dm=4, N=5)
        x, delta, A, B, C, D, h0 = (p[k] for k in ("x", "delta", "A", "B", "C", "D", "h0"))
        g = orc.scan_bwd(x, delta, A, B, C, D, dy, h0=h0, dh_final=dhf, **opts)
        y, hf = orc.scan(x, delta, A, B, C, D, h0=h0, **opts)
        lhs = np.sum(dy * y) + np.sum(dhf * hf)
        rhs = np.sum(g["dx"] * x) + np.sum(g["dh0"] * h0)
        assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs)), (opts, lhs, rhs)
        # B: with h0 = 0 the outputs are linear in B
        g0 = orc.scan_bwd(x, delta, A, B, C, D, dy, dh_final=dhf, **opts)
        y0, hf0 = orc.scan(x, delta, A, B, C, D, **opts)
        lhs = np.sum(dy * (y0 - D * x)) + np.sum(dhf * hf0)
        assert abs(lhs - np.sum(g0["dB"] * B)) <= 1e-12 * max(1.0, abs(lhs))
        # C: y - D x is linear in C (h_final does not depend on C)
        lhs = np.sum(dy * (y - D * x))
        assert abs(lhs - np.sum(g["dC"] * C)) <= 1e-12 * max(1.0, abs(lhs))
        # D: dD = sum over (b, t) of dy x
        assert np.allclose(g["dD"], np.sum(dy * x, axis=(0, 1)), rtol=1e-13, atol=1e-13)
        # dC from states computed by the forward on prefixes
        for t in (0, 5, 10):
            _, ht = orc.scan(x[:, :t + 1], delta[:, :t + 1], A, B[:, :t + 1], C[:, :t + 1], D, h0=h0, **opts)
            assert np.allclose(g["dC"][:, t], np.einsum("bd,bdn->bn", dy[:, t], ht), rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# complex diagonal A


def vanloan_complex(a, w, dt, b):
    """(Abar, Bbar) of h' = (a + i w) h + b u as the real 2-state system
    [[a, -w], [w, a]] with input (b, 0): exp of the augmented matrix."""
    M = np.array([[a, -w, b], [w, a, 0.0], [0.0, 0.0, 0.0]], dtype=np.float64) * dt
    E = expm(M)
    return E[0, 0] + 1j * E[1, 0], E[0, 2] + 1j * E[1, 2]


def check_complex_vanloan_step(orc):
    """One step from h = 0 (x = 1) gives Bbar; from h = 1 and h = i (x = 0)
    gives Abar and i Abar, over a grid including a = 0, w = 0 and delta = 0."""
    a_v = [-3.0, -0.5, -1e-6, 0.0]
    w_v = [0.0, 0.3, 2.0, 10.0, -4.0]
    d_v = [0.0, 1e-4, 0.05, 0.7]
    bval = 1.3
    A = np.array([[complex(a, w)] for a in a_v for w in w_v])  # [Dm, 1]
    Dm = A.shape[0]
    for dt in d_v:
        x1, x0 = np.ones((1, Dm)), np.zeros((1, Dm))
        dl = np.full((1, Dm), dt)
        Bm, Cm = np.full((1, 1), bval), np.zeros((1, 1))
        _, hB = orc.step_complex(x1, dl, A, Bm, Cm, np.zeros(Dm), np.zeros((1, Dm, 1), complex))
        _, hA = orc.step_complex(x0, dl, A, Bm, Cm, np.zeros(Dm), np.ones((1, Dm, 1), complex))
        _, hI = orc.step_complex(x0, dl, A, Bm, Cm, np.zeros(Dm), np.full((1, Dm, 1), 1j))
        for k in range(Dm):
            ea, eb = vanloan_complex(A[k, 0].real, A[k, 0].imag, dt, bval)
            # expm's own error grows with the norm of delta * A
            tol = 1e-14 * max(1.0, abs(dt * A[k, 0])) * 4
            assert abs(hA[0, k, 0] - ea) <= tol * max(1.0, abs(ea)), (A[k, 0], dt, hA[0, k, 0], ea)
            assert abs(hI[0, k, 0] - 1j * ea) <= tol * max(1.0, abs(ea))
            assert abs(hB[0, k, 0] - eb) <= 10 * tol * max(abs(eb), 1e-300), (A[k, 0], dt, hB[0, k, 0], eb)


def check_complex_reduces_to_real(orc, seed=20):
    """w = 0: the complex scan is the real scan (imaginary parts stay 0)."""
    rng = np.random.default_rng(seed)
    x, delta, A, B, C, D = random_case(rng, 2, 13, 3, 4)
    h0 = rng.standard_normal((2, 3, 4))
    for opts in ({}, {"euler_b": True}):
        yc, hc = orc.scan_complex(x, delta, A.astype(complex), B, C, D, h0=h0.astype(complex), **opts)
        yr, hr = orc.scan(x, delta, A, B, C, D, h0=h0, **opts)
        assert rel_err(yc, yr) < 1e-14 and rel_err(hc.real, hr) < 1e-14
        assert np.all(hc.imag == 0.0)


def _cbwd_case(rng, opts, Bsz=2, L=7, Dm=3, N=4):
    x, delta, A, B, C, D = random_case(rng, Bsz, L, Dm, N)
    w = rng.normal(0.0, 2.0, A.shape)
    A = A + 1j * w
    A[0, 1] = 0.0          # exact A = 0 (limit of the ZOH input term and of its derivative)
    A[1, 2] = -1e-7 + 3e-8j  # tiny A, inside the series branch of phi'
    A[2, 3] = 0.7j         # pure rotation
    h0 = rng.standard_normal((Bsz, Dm, N)) + 1j * rng.standard_normal((Bsz, Dm, N))
    dy = rng.standard_normal((Bsz, L, Dm))
    dhf = rng.standard_normal((Bsz, Dm, N)) + 1j * rng.standard_normal((Bsz, Dm, N))
    bias = None
    if opts.get("delta_softplus"):
        delta = rng.normal(-2.0, 1.0, delta.shape)
        bias = rng.normal(0.0, 0.5, Dm)
    return dict(x=x, delta=delta, A=A, B=B, C=C, D=D, h0=h0), dy, dhf, bias


def _closs(orc, p, dy, dhf, bias, opts):
    """<dy, y> + Re<dh_final, h_final> (each complex entry as its (re, im) pair)."""
    y, hf = orc.scan_complex(p["x"], p["delta"], p["A"], p["B"], p["C"], p["D"], h0=p["h0"], delta_bias=bias,
                             **opts)
    return float(np.sum(dy * y) + np.sum(dhf.real * hf.real + dhf.imag * hf.imag))


def check_complex_bwd_finite_differences(orc, seed=30):
    """Every gradient of the complex-A scan, real and imaginary parts of A and
    h0 separately, against central differences of the complex forward oracle,
    for ZOH, softplus(delta + bias), and the Euler input term."""
    for k, opts in enumerate(({}, {"delta_softplus": True}, {"delta_softplus": True, "euler_b": True},
                              {"euler_b": True})):
        rng = np.random.default_rng(seed + k)
        p, dy, dhf, bias = _cbwd_case(rng, opts)
        g = orc.scan_complex_bwd(p["x"], p["delta"], p["A"], p["B"], p["C"], p["D"], dy, h0=p["h0"],
                                 dh_final=dhf, delta_bias=bias, **opts)
        grads = {"x": g["dx"], "delta": g["ddelta"], "B": g["dB"], "C": g["dC"], "D": g["dD"],
                 "A.re": g["dA"].real, "A.im": g["dA"].imag, "h0.re": g["dh0"].real, "h0.im": g["dh0"].imag}
        if bias is not None:
            grads["bias"] = g["dbias"]
        scale = max(1.0, max(float(np.max(np.abs(v))) for v in grads.values()))
        for name, got in grads.items():
            base, part = (name.split(".") + [None])[:2]
            shape = (bias if base == "bias" else p[base]).shape
            for idx in np.ndindex(shape):
                def loss_at(delta_v):
                    q = dict(p)
                    bb = bias
                    if base == "bias":
                        bb = bias.copy()
                        bb[idx] += delta_v
                    else:
                        arr = q[base].copy()
                        arr[idx] += delta_v * (1j if part == "im" else 1.0)
                        q[base] = arr
                    return _closs(orc, q, dy, dhf, bb, opts)
                ref = (bias if base == "bias" else p[base])[idx]
                eps = 1e-6 * max(1.0, abs(ref))
                fd = (loss_at(eps) - loss_at(-eps)) / (2 * eps)
                assert abs(fd - got[idx]) <= 2e-7 * scale + 1e-6 * abs(fd), (opts, name, idx, fd, got[idx])


def check_complex_bwd_identities(orc, seed=34):
    """Exact identities: with delta and A fixed the outputs are linear in
    (x, h0), so <dy, y> + Re<dhf, h_final> = <dx, x> + Re<dh0, h0>; and with
    every imaginary part zero the gradients are the real scan's (the real
    backward is pinned on its own) and the adjoint of h0 stays real."""
    rng = np.random.default_rng(seed)
    for opts in ({}, {"euler_b": True}):
        p, dy, dhf, _ = _cbwd_case(rng, opts, Bsz=2, L=11, Dm=4, N=5)
        x, delta, A, B, C, D, h0 = (p[k] for k in ("x", "delta", "A", "B", "C", "D", "h0"))
        g = orc.scan_complex_bwd(x, delta, A, B, C, D, dy, h0=h0, dh_final=dhf, **opts)
        y, hf = orc.scan_complex(x, delta, A, B, C, D, h0=h0, **opts)
        lhs = np.sum(dy * y) + np.sum(dhf.real * hf.real + dhf.imag * hf.imag)
        rhs = np.sum(g["dx"] * x) + np.sum(g["dh0"].real * h0.real + g["dh0"].imag * h0.imag)
        assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs)), (opts, lhs, rhs)
        Ar, h0r, dhfr = A.real.copy(), h0.real.copy(), dhf.real.copy()
        gc = orc.scan_complex_bwd(x, delta, Ar.astype(complex), B, C, D, dy, h0=h0r.astype(complex),
                                  dh_final=dhfr.astype(complex), **opts)
        gr = orc.scan_bwd(x, delta, Ar, B, C, D, dy, h0=h0r, dh_final=dhfr, **opts)
        for k in ("dx", "ddelta", "dB", "dC", "dD"):
            assert rel_err(gc[k], gr[k]) < 1e-12, (opts, k)
        assert rel_err(gc["dA"].real, gr["dA"]) < 1e-11 and rel_err(gc["dh0"].real, gr["dh0"]) < 1e-12
        assert np.all(gc["dh0"].imag == 0.0)


def check_complex_rotation(orc, seed=21):
    """a = 0, x = 0: the state turns by w * sum(delta) at constant modulus."""
    rng = np.random.default_rng(seed)
    Bsz, L, Dm, N = 2, 17, 3, 4
    _, delta, _, B, C, D = random_case(rng, Bsz, L, Dm, N)
    w = rng.uniform(-6, 6, (Dm, N))
    h0 = rng.standard_normal((Bsz, Dm, N)) + 1j * rng.standard_normal((Bsz, Dm, N))
    _, hf = orc.scan_complex(np.zeros((Bsz, L, Dm)), delta, 1j * w, B, C, D, h0=h0)
    expect = h0 * np.exp(1j * w[None] * delta.sum(axis=1)[:, :, None])
    assert np.max(np.abs(hf - expect)) < 1e-13
    assert np.max(np.abs(np.abs(hf) - np.abs(h0))) < 1e-13


def check_complex_exact_for_constant_input(orc, seed=22):
    """Constant x, delta, B, h0 = 0: after k steps the ZOH state is the exact
    ODE solution B x (exp(A k delta) - 1) / A; the Euler term gives the
    geometric sum delta B x (1 - Abar^k) / (1 - Abar)."""
    rng = np.random.default_rng(seed)
    L, Dm, N = 9, 3, 2
    xv, dv = rng.standard_normal(Dm), rng.uniform(0.02, 0.4, Dm)
    bv = rng.standard_normal(N)
    A = -np.exp(rng.uniform(-1, 1, (Dm, N))) + 1j * rng.uniform(-5, 5, (Dm, N))
    x = np.tile(xv.reshape(1, 1, Dm), (1, L, 1))
    dl = np.tile(dv.reshape(1, 1, Dm), (1, L, 1))
    B = np.tile(bv.reshape(1, 1, N), (1, L, 1))
    C = np.zeros((1, L, N))
    for k in range(1, L + 1):
        _, hz = orc.scan_complex(x[:, :k], dl[:, :k], A, B[:, :k], C[:, :k], np.zeros(Dm))
        _, he = orc.scan_complex(x[:, :k], dl[:, :k], A, B[:, :k], C[:, :k], np.zeros(Dm), euler_b=True)
        ex = bv[None, :] * xv[:, None] * np.expm1(A * k * dv[:, None]) / A
        ab = np.exp(A * dv[:, None])
        ee = dv[:, None] * bv[None, :] * xv[:, None] * np.expm1(k * A * dv[:, None]) / np.expm1(A * dv[:, None])
        assert np.max(np.abs(hz[0] - ex)) <= 1e-12 * np.max(np.abs(ex)), k
        assert np.max(np.abs(he[0] - ee)) <= 1e-12 * np.max(np.abs(ee)), k
        _ = ab


def check_complex_lfilter(orc, seed=23):
    """Time-varying x with constant delta, B, C: per state the complex IIR
    filter lfilter([Bbar], [1, -Abar], x) (Abar, Bbar from the real 2-state
    matrix exponential), and y = sum_n C_n Re(h_n) + D x."""
    rng = np.random.default_rng(seed)
    L, Dm, N = 30, 2, 3
    x = rng.standard_normal((1, L, Dm))
    dv = rng.uniform(0.05, 0.5, Dm)
    dl = np.tile(dv.reshape(1, 1, Dm), (1, L, 1))
    A = -np.exp(rng.uniform(-1.5, 0.5, (Dm, N))) + 1j * rng.uniform(-8, 8, (Dm, N))
    bv, cv = rng.standard_normal(N), rng.standard_normal(N)
    B = np.tile(bv.reshape(1, 1, N), (1, L, 1))
    C = np.tile(cv.reshape(1, 1, N), (1, L, 1))
    D = rng.standard_normal(Dm)
    y, hf = orc.scan_complex(x, dl, A, B, C, D)
    for d in range(Dm):
        hs = np.empty((L, N), complex)
        for n in range(N):
            ab, bb = vanloan_complex(A[d, n].real, A[d, n].imag, dv[d], bv[n])
            hs[:, n] = lfilter([bb], [1.0, -ab], x[0, :, d].astype(complex))
        ye = hs.real @ cv + D[d] * x[0, :, d]
        assert rel_err(y[0, :, d], ye) < 1e-12
        assert np.max(np.abs(hf[0, d] - hs[-1])) < 1e-12 * max(1.0, np.max(np.abs(hs[-1])))


def check_complex_step_chain(orc, seed=24):
    rng = np.random.default_rng(seed)
    Bsz, L, Dm, N = 2, 9, 3, 4
    x, _, _, B, C, D = random_case(rng, Bsz, L, Dm, N)
    raw = rng.normal(-1.0, 1.0, (Bsz, L, Dm))
    bias = rng.normal(0.0, 0.5, Dm)
    A = -np.exp(rng.uniform(-1, 1, (Dm, N))) + 1j * rng.uniform(-3, 3, (Dm, N))
    h0 = rng.standard_normal((Bsz, Dm, N)) + 1j * rng.standard_normal((Bsz, Dm, N))
    opts = dict(delta_bias=bias, delta_softplus=True)
    y, hf = orc.scan_complex(x, raw, A, B, C, D, h0=h0, **opts)
    h = h0
    for t in range(L):
        yt, h = orc.step_complex(x[:, t], raw[:, t], A, B[:, t], C[:, t], D, h, **opts)
        assert rel_err(yt, y[:, t]) < 1e-13
    assert np.max(np.abs(h - hf)) < 1e-13 * max(1.0, np.max(np.abs(hf)))



# ---------------------------------------------------------------------------
# scalar decay per head (state-space duality form)


def check_ssd_duality(orc, seed=30):
    """The scalar-decay layer equals its masked-attention form ("Mamba SSM
    Nedir?" page, section "Mamba-2 ve Guncel Gelismeler": the SSM is a form of
    attention).  Per row b and head h, with cum[t] = A[h] * sum_{r<=t} delta_r
    and k_s the one-step input factor (Van Loan's matrix exponential for the
    ZOH rule, delta_s for the Euler rule):
        y[:, d]  = (G o Lmask) x[:, d] + D[d] x[:, d] + exp(cum) * (C h0[d])
        G[t, s]  = (C_t . B_s) k_s,  Lmask[t, s] = exp(cum[t] - cum[s]) for s <= t, else 0
        hL[d]    = exp(cum[L-1]) h0[d] + sum_s exp(cum[L-1] - cum[s]) k_s x_s[d] B_s
    built as dense L x L matrices with numpy.  Covers a head with A = 0,
    heads of several channels, the softplus/bias and Euler options, and h0."""
    rng = np.random.default_rng(seed)
    Bsz, L, H, P, N = 2, 37, 3, 2, 4
    Dm = H * P
    A = np.array([-0.7, 0.0, -2.5])
    x = rng.standard_normal((Bsz, L, Dm))
    B = rng.standard_normal((Bsz, L, N))
    C = rng.standard_normal((Bsz, L, N))
    D = rng.standard_normal(Dm)
    h0 = rng.standard_normal((Bsz, Dm, N))
    cases = [
        (rng.uniform(0.01, 0.5, (Bsz, L, H)), None, False, False, None),
        (rng.uniform(0.01, 0.5, (Bsz, L, H)), None, False, False, h0),
        (0.5 * rng.standard_normal((Bsz, L, H)), rng.uniform(-3.0, 0.0, H), True, True, h0),
        (rng.uniform(0.0, 0.3, (Bsz, L, H)), rng.uniform(0.0, 0.1, H), False, False, h0),
    ]
    for raw, bias, sp, eul, h in cases:
        y, hf = orc.scan_ssd(x, raw, A, B, C, D, P, h0=h, delta_bias=bias, delta_softplus=sp, euler_b=eul)
        y_ref = np.empty_like(x)
        h_ref = np.empty((Bsz, Dm, N))
        causal = np.tril(np.ones((L, L), dtype=bool))
        for b in range(Bsz):
            for hh in range(H):
                v = raw[b, :, hh] + (0.0 if bias is None else bias[hh])
                dt = np.logaddexp(0.0, v) if sp else v
                cum = A[hh] * np.cumsum(dt)
                k = dt.copy() if eul else np.array([vanloan_zoh(A[hh], t)[1] for t in dt])
                G = (C[b] @ B[b].T) * k[None, :]
                Lm = np.where(causal, np.exp(np.where(causal, cum[:, None] - cum[None, :], 0.0)), 0.0)
                M = G * Lm
                for d in range(hh * P, (hh + 1) * P):
                    y_ref[b, :, d] = M @ x[b, :, d] + D[d] * x[b, :, d]
                    h_ref[b, d] = (np.exp(cum[-1] - cum) * k * x[b, :, d]) @ B[b]
                    if h is not None:
                        y_ref[b, :, d] += np.exp(cum) * (C[b] @ h[b, d])
                        h_ref[b, d] += np.exp(cum[-1]) * h[b, d]
        assert rel_err(y, y_ref) < 1e-11, ("ssd y", rel_err(y, y_ref), sp, eul, h is None)
        assert rel_err(hf, h_ref) < 1e-11, ("ssd h_final", rel_err(hf, h_ref), sp, eul, h is None)


ALL_CHECKS = [
    check_golden,
    check_brute_force,
    lambda o: check_brute_force(o, seed=11, with_h0=True),
    check_vanloan_step,
    check_lti_convolution,
    check_a_to_zero_limit,
    check_delta_zero_persistence,
    check_pure_decay,
    check_zoh_exact_for_constant_input,
    check_linearity_causality_permutation,
    check_step_chain_matches_scan,
    check_split_scan_operator,
    check_softplus_closed_forms,
    check_fused_delta_matches_precomputed,
    check_euler_b_closed_forms,
    check_options_step_chain_matches_scan,
    check_bwd_finite_differences,
    check_bwd_adjoint_identities,
    check_complex_vanloan_step,
    check_complex_reduces_to_real,
    check_complex_rotation,
    check_complex_exact_for_constant_input,
    check_complex_lfilter,
    check_complex_step_chain,
    check_complex_bwd_finite_differences,
    check_complex_bwd_identities,
    check_ssd_duality,
]
