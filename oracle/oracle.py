"""ctypes front-end of the fp64 oracle (test infrastructure).

All arrays are numpy float64, C-contiguous; inputs stored on a device in bf16
or fp32 are widened to float64 exactly before they get here.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# SSM_ORACLE_LIB selects another build of the same source (the sanitizer build).
DEFAULT_LIB = os.environ.get("SSM_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")

_dp = ctypes.POINTER(ctypes.c_double)
_i64 = ctypes.c_int64


def _f64(a, shape, name):
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    if tuple(a.shape) != tuple(shape):
        raise ValueError(f"oracle: {name} has shape {a.shape}, expected {shape}")
    return a


def _as_complex(a):
    a = np.asarray(a)
    if np.iscomplexobj(a):
        return a.astype(np.complex128)
    if a.shape[-1] != 2:
        raise ValueError("oracle: expected a complex array or a trailing (re, im) axis")
    return a[..., 0].astype(np.float64) + 1j * a[..., 1].astype(np.float64)


def _pairs(c, shape, name):
    c = np.asarray(c)
    if tuple(c.shape) != tuple(shape):
        raise ValueError(f"oracle: {name} has shape {c.shape}, expected {shape}")
    return np.ascontiguousarray(np.stack([c.real, c.imag], axis=-1).astype(np.float64))


def _flags(delta_softplus, euler_b):
    return (1 if delta_softplus else 0) | (2 if euler_b else 0)


def _ptr(a):
    return a.ctypes.data_as(_dp) if a is not None else None


class Oracle:
    """One loaded copy of the oracle library."""

    def __init__(self, lib_path: str = DEFAULT_LIB, threads: int = 0):
        """threads: default thread count of every call (0: OpenMP's default)."""
        self.threads = int(threads)
        if lib_path == DEFAULT_LIB and not os.path.exists(lib_path):
            from . import build as _build
            _build.build()
        lib = ctypes.CDLL(lib_path)
        lib.ssm_oracle_scan.argtypes = [_dp] * 10 + [_i64] * 4 + [ctypes.c_int, ctypes.c_int]
        lib.ssm_oracle_scan.restype = ctypes.c_int
        lib.ssm_oracle_step.argtypes = [_dp] * 9 + [_i64] * 3 + [ctypes.c_int]
        lib.ssm_oracle_step.restype = ctypes.c_int
        lib.ssm_oracle_scan_bwd.argtypes = [_dp] * 18 + [_i64] * 4 + [ctypes.c_int, ctypes.c_int]
        lib.ssm_oracle_scan_bwd.restype = ctypes.c_int
        lib.ssm_oracle_scan_complex.argtypes = [_dp] * 10 + [_i64] * 4 + [ctypes.c_int, ctypes.c_int]
        lib.ssm_oracle_scan_complex.restype = ctypes.c_int
        lib.ssm_oracle_step_complex.argtypes = [_dp] * 9 + [_i64] * 3 + [ctypes.c_int]
        lib.ssm_oracle_step_complex.restype = ctypes.c_int
        lib.ssm_oracle_scan_complex_bwd.argtypes = [_dp] * 18 + [_i64] * 4 + [ctypes.c_int, ctypes.c_int]
        lib.ssm_oracle_scan_complex_bwd.restype = ctypes.c_int
        lib.ssm_oracle_max_threads.argtypes = []
        lib.ssm_oracle_max_threads.restype = ctypes.c_int
        self.lib = lib
        self.path = lib_path

    def max_threads(self) -> int:
        return int(self.lib.ssm_oracle_max_threads())

    def scan(self, x, delta, A, B, C, D, h0=None, threads: int = 0, delta_bias=None,
             delta_softplus: bool = False, euler_b: bool = False):
        """Sequential fp64 scan.  Returns (y [Bsz,L,Dm], h_final [Bsz,Dm,N]).

        delta_bias [Dm] is added to delta; delta_softplus passes the sum through
        softplus; euler_b uses Bbar = delta*B instead of the ZOH input term."""
        x = np.asarray(x)
        Bsz, L, Dm = x.shape
        N = np.asarray(A).shape[1]
        x = _f64(x, (Bsz, L, Dm), "x")
        delta = _f64(delta, (Bsz, L, Dm), "delta")
        A = _f64(A, (Dm, N), "A")
        B = _f64(B, (Bsz, L, N), "B")
        C = _f64(C, (Bsz, L, N), "C")
        D = _f64(D, (Dm,), "D")
        if h0 is not None:
            h0 = _f64(h0, (Bsz, Dm, N), "h0")
        bias = None if delta_bias is None else _f64(delta_bias, (Dm,), "delta_bias")
        y = np.empty((Bsz, L, Dm), dtype=np.float64)
        hf = np.empty((Bsz, Dm, N), dtype=np.float64)
        rc = self.lib.ssm_oracle_scan(_ptr(x), _ptr(delta), _ptr(bias), _ptr(A), _ptr(B), _ptr(C),
                                      _ptr(D), _ptr(h0), _ptr(y), _ptr(hf),
                                      Bsz, L, Dm, N, _flags(delta_softplus, euler_b), int(threads or self.threads))
        if rc != 0:
            raise RuntimeError(f"ssm_oracle_scan failed with code {rc}")
        return y, hf

    def scan_ssd(self, x, delta, A, B, C, D, head_dim: int, h0=None, threads: int = 0, delta_bias=None,
                 delta_softplus: bool = False, euler_b: bool = False):
        """The scan with one scalar decay per head (the state-space-duality form).

        The bitig.info page on Mamba-3 (section "Karmasik Degerli Durum
        Guncellemesi") says Mamba-2 reduced the state transition to real
        scalars; the "Mamba SSM Nedir?" page (section "Mamba-2 ve Guncel
        Gelismeler") states that model's equivalence with a masked attention.
        Reading: channels form heads of ``head_dim`` consecutive channels; head
        h has one real A[h] for all N states, one delta[b, t, h] per step and
        one bias[h].  That is the selective scan with A[d, n] = A[h(d)] and
        delta[b, t, d] = delta[b, t, h(d)], h(d) = d // head_dim, which is how
        it is evaluated here.  Shapes: x [Bsz,L,Dm], delta [Bsz,L,H], A [H],
        B, C [Bsz,L,N], D [Dm], delta_bias [H], h0 [Bsz,Dm,N].
        Returns (y [Bsz,L,Dm], h_final [Bsz,Dm,N])."""
        x = np.asarray(x)
        Bsz, L, Dm = x.shape
        P = int(head_dim)
        if P <= 0 or Dm % P:
            raise ValueError(f"oracle: Dm={Dm} is not a multiple of head_dim={P}")
        H = Dm // P
        N = np.asarray(B).shape[2]
        delta = _f64(delta, (Bsz, L, H), "delta")
        A = _f64(A, (H,), "A")
        A_full = np.repeat(A, P)[:, None] * np.ones((1, N))
        delta_full = np.repeat(delta, P, axis=2)
        bias = None if delta_bias is None else np.repeat(_f64(delta_bias, (H,), "delta_bias"), P)
        return self.scan(x, delta_full, A_full, B, C, D, h0=h0, threads=threads, delta_bias=bias,
                         delta_softplus=delta_softplus, euler_b=euler_b)

    def scan_complex(self, x, delta, A, B, C, D, h0=None, threads: int = 0, delta_bias=None,
                     delta_softplus: bool = False, euler_b: bool = False):
        """Scan with complex diagonal A.  A: complex [Dm, N] (numpy complex or a
        real [Dm, N, 2] array of (re, im)); h0 complex [Bsz, Dm, N] or None.
        Returns (y [Bsz, L, Dm] real, h_final [Bsz, Dm, N] complex)."""
        x = np.asarray(x)
        Bsz, L, Dm = x.shape
        Ac = _as_complex(A)
        N = Ac.shape[1]
        x = _f64(x, (Bsz, L, Dm), "x")
        delta = _f64(delta, (Bsz, L, Dm), "delta")
        A2 = _pairs(Ac, (Dm, N), "A")
        B = _f64(B, (Bsz, L, N), "B")
        C = _f64(C, (Bsz, L, N), "C")
        D = _f64(D, (Dm,), "D")
        h2 = None if h0 is None else _pairs(_as_complex(h0), (Bsz, Dm, N), "h0")
        bias = None if delta_bias is None else _f64(delta_bias, (Dm,), "delta_bias")
        y = np.empty((Bsz, L, Dm), dtype=np.float64)
        hf = np.empty((Bsz, Dm, N, 2), dtype=np.float64)
        rc = self.lib.ssm_oracle_scan_complex(_ptr(x), _ptr(delta), _ptr(bias), _ptr(A2), _ptr(B), _ptr(C),
                                              _ptr(D), _ptr(h2), _ptr(y), _ptr(hf), Bsz, L, Dm, N,
                                              _flags(delta_softplus, euler_b), int(threads or self.threads))
        if rc != 0:
            raise RuntimeError(f"ssm_oracle_scan_complex failed with code {rc}")
        return y, hf[..., 0] + 1j * hf[..., 1]

    def scan_complex_bwd(self, x, delta, A, B, C, D, dy, h0=None, dh_final=None, delta_bias=None,
                         delta_softplus: bool = False, euler_b: bool = False, want_dBC: bool = True,
                         threads: int = 0):
        """Gradients of the complex-A scan for output gradients dy [Bsz,L,Dm] and,
        if given, dh_final complex [Bsz,Dm,N] (the loss pairs it with h_final as
        Re(conj(dh_final) h_final)).  A, h0 as scan_complex.  Returns a dict with
        dx, ddelta, dD, dbias (if delta_bias is given), dB, dC (if want_dBC), and
        dA [Dm,N], dh0 [Bsz,Dm,N] complex: the gradients of the real and the
        imaginary parts as one complex number."""
        x = np.asarray(x)
        Bsz, L, Dm = x.shape
        Ac = _as_complex(A)
        N = Ac.shape[1]
        x = _f64(x, (Bsz, L, Dm), "x")
        delta = _f64(delta, (Bsz, L, Dm), "delta")
        A2 = _pairs(Ac, (Dm, N), "A")
        B = _f64(B, (Bsz, L, N), "B")
        C = _f64(C, (Bsz, L, N), "C")
        D = _f64(D, (Dm,), "D")
        dy = _f64(dy, (Bsz, L, Dm), "dy")
        h2 = None if h0 is None else _pairs(_as_complex(h0), (Bsz, Dm, N), "h0")
        g2 = None if dh_final is None else _pairs(_as_complex(dh_final), (Bsz, Dm, N), "dh_final")
        bias = None if delta_bias is None else _f64(delta_bias, (Dm,), "delta_bias")
        out = {"dx": np.empty((Bsz, L, Dm)), "ddelta": np.empty((Bsz, L, Dm)), "dD": np.empty(Dm)}
        dA = np.empty((Dm, N, 2))
        dh0 = np.empty((Bsz, Dm, N, 2))
        out["dbias"] = np.empty(Dm) if bias is not None else None
        out["dB"] = np.empty((Bsz, L, N)) if want_dBC else None
        out["dC"] = np.empty((Bsz, L, N)) if want_dBC else None
        rc = self.lib.ssm_oracle_scan_complex_bwd(
            _ptr(x), _ptr(delta), _ptr(bias), _ptr(A2), _ptr(B), _ptr(C), _ptr(D), _ptr(h2), _ptr(dy), _ptr(g2),
            _ptr(out["dx"]), _ptr(out["ddelta"]), _ptr(out["dbias"]), _ptr(dA), _ptr(out["dB"]), _ptr(out["dC"]),
            _ptr(out["dD"]), _ptr(dh0), Bsz, L, Dm, N, _flags(delta_softplus, euler_b), int(threads or self.threads))
        if rc != 0:
            raise RuntimeError(f"ssm_oracle_scan_complex_bwd failed with code {rc}")
        out["dA"] = dA[..., 0] + 1j * dA[..., 1]
        out["dh0"] = dh0[..., 0] + 1j * dh0[..., 1]
        return out

    def step_complex(self, x, delta, A, B, C, D, h, delta_bias=None, delta_softplus: bool = False,
                     euler_b: bool = False):
        """One step with complex A; h complex [Bsz, Dm, N] (not modified).
        Returns (y [Bsz, Dm], h_new complex)."""
        x = np.asarray(x)
        Bsz, Dm = x.shape
        Ac = _as_complex(A)
        N = Ac.shape[1]
        x = _f64(x, (Bsz, Dm), "x")
        delta = _f64(delta, (Bsz, Dm), "delta")
        A2 = _pairs(Ac, (Dm, N), "A")
        B = _f64(B, (Bsz, N), "B")
        C = _f64(C, (Bsz, N), "C")
        D = _f64(D, (Dm,), "D")
        h2 = _pairs(_as_complex(h), (Bsz, Dm, N), "h").copy()
        bias = None if delta_bias is None else _f64(delta_bias, (Dm,), "delta_bias")
        y = np.empty((Bsz, Dm), dtype=np.float64)
        rc = self.lib.ssm_oracle_step_complex(_ptr(x), _ptr(delta), _ptr(bias), _ptr(A2), _ptr(B), _ptr(C),
                                              _ptr(D), _ptr(h2), _ptr(y), Bsz, Dm, N,
                                              _flags(delta_softplus, euler_b))
        if rc != 0:
            raise RuntimeError(f"ssm_oracle_step_complex failed with code {rc}")
        return y, h2[..., 0] + 1j * h2[..., 1]

    def scan_bwd(self, x, delta, A, B, C, D, dy, h0=None, dh_final=None, delta_bias=None,
                 delta_softplus: bool = False, euler_b: bool = False, want_dBC: bool = True,
                 threads: int = 0):
        """Gradients of the scan for output gradients dy [Bsz,L,Dm] (and dh_final
        [Bsz,Dm,N] if given).  Returns a dict with dx, ddelta (for the delta
        input as passed, i.e. the raw value when delta_softplus), dA, dD, dh0,
        dbias (if delta_bias is given) and dB, dC (if want_dBC)."""
        x = np.asarray(x)
        Bsz, L, Dm = x.shape
        N = np.asarray(A).shape[1]
        x = _f64(x, (Bsz, L, Dm), "x")
        delta = _f64(delta, (Bsz, L, Dm), "delta")
        A = _f64(A, (Dm, N), "A")
        B = _f64(B, (Bsz, L, N), "B")
        C = _f64(C, (Bsz, L, N), "C")
        D = _f64(D, (Dm,), "D")
        dy = _f64(dy, (Bsz, L, Dm), "dy")
        h0 = None if h0 is None else _f64(h0, (Bsz, Dm, N), "h0")
        dhf = None if dh_final is None else _f64(dh_final, (Bsz, Dm, N), "dh_final")
        bias = None if delta_bias is None else _f64(delta_bias, (Dm,), "delta_bias")
        out = {"dx": np.empty((Bsz, L, Dm)), "ddelta": np.empty((Bsz, L, Dm)), "dA": np.empty((Dm, N)),
               "dD": np.empty(Dm), "dh0": np.empty((Bsz, Dm, N))}
        out["dbias"] = np.empty(Dm) if bias is not None else None
        out["dB"] = np.empty((Bsz, L, N)) if want_dBC else None
        out["dC"] = np.empty((Bsz, L, N)) if want_dBC else None
        rc = self.lib.ssm_oracle_scan_bwd(
            _ptr(x), _ptr(delta), _ptr(bias), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(h0), _ptr(dy), _ptr(dhf),
            _ptr(out["dx"]), _ptr(out["ddelta"]), _ptr(out["dbias"]), _ptr(out["dA"]), _ptr(out["dB"]),
            _ptr(out["dC"]), _ptr(out["dD"]), _ptr(out["dh0"]), Bsz, L, Dm, N,
            _flags(delta_softplus, euler_b), int(threads or self.threads))
        if rc != 0:
            raise RuntimeError(f"ssm_oracle_scan_bwd failed with code {rc}")
        return out

    def step(self, x, delta, A, B, C, D, h, delta_bias=None, delta_softplus: bool = False,
             euler_b: bool = False):
        """One recurrent step.  Returns (y [Bsz,Dm], h_new [Bsz,Dm,N]); h is not modified.
        The options are those of scan()."""
        x = np.asarray(x)
        Bsz, Dm = x.shape
        N = np.asarray(A).shape[1]
        x = _f64(x, (Bsz, Dm), "x")
        delta = _f64(delta, (Bsz, Dm), "delta")
        A = _f64(A, (Dm, N), "A")
        B = _f64(B, (Bsz, N), "B")
        C = _f64(C, (Bsz, N), "C")
        D = _f64(D, (Dm,), "D")
        hn = _f64(h, (Bsz, Dm, N), "h").copy()
        bias = None if delta_bias is None else _f64(delta_bias, (Dm,), "delta_bias")
        y = np.empty((Bsz, Dm), dtype=np.float64)
        rc = self.lib.ssm_oracle_step(_ptr(x), _ptr(delta), _ptr(bias), _ptr(A), _ptr(B), _ptr(C),
                                      _ptr(D), _ptr(hn), _ptr(y), Bsz, Dm, N,
                                      _flags(delta_softplus, euler_b))
        if rc != 0:
            raise RuntimeError(f"ssm_oracle_step failed with code {rc}")
        return y, hn


_default = None


def load() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def max_threads() -> int:
    return load().max_threads()


def scan(x, delta, A, B, C, D, h0=None, threads: int = 0, **opts):
    return load().scan(x, delta, A, B, C, D, h0=h0, threads=threads, **opts)


def step(x, delta, A, B, C, D, h, **opts):
    return load().step(x, delta, A, B, C, D, h, **opts)


def scan_bwd(x, delta, A, B, C, D, dy, **opts):
    return load().scan_bwd(x, delta, A, B, C, D, dy, **opts)


def scan_complex(x, delta, A, B, C, D, **opts):
    return load().scan_complex(x, delta, A, B, C, D, **opts)


def step_complex(x, delta, A, B, C, D, h, **opts):
    return load().step_complex(x, delta, A, B, C, D, h, **opts)


def scan_complex_bwd(x, delta, A, B, C, D, dy, **opts):
    return load().scan_complex_bwd(x, delta, A, B, C, D, dy, **opts)


def scan_ssd(x, delta, A, B, C, D, head_dim, **opts):
    return load().scan_ssd(x, delta, A, B, C, D, head_dim, **opts)
