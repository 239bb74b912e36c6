"""Float64 CPU oracle for causal linear attention (phi = elu + 1).

TEST INFRASTRUCTURE ONLY: imported by the test-suite, the smoke check and the
benchmark's CPU-baseline leg, never by the library.  It shares no code with
the HIP path.  The arithmetic lives in ``la_oracle.c`` (plain C, float64,
token by token); this module only builds that file, marshals numpy arrays to
float64 and back, and says which routine follows which equation.

Sources: "Transformers are RNNs -- part 2/3" eq. 7-20; the reading notes on
the same paper, section 3.2 eq. 4-6 and appendix A; "Linear Attention/zh",
kernel reformulation and recurrent form.

Every routine here is pinned by the tests in ``tests/test_oracle_pins.py``
(brute force of the quadratic masked definition, a hand-derived worked
example, closed forms, invariants and finite differences).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "la_oracle.c")
_LIB = os.path.join(_HERE, "liblaoracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile la_oracle.c into liblaoracle.so with gcc (OpenMP over heads)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _configure(lib):
    """Declare the C signatures on a loaded oracle library."""
    dp = ctypes.POINTER(ctypes.c_double)
    L = ctypes.c_long
    lib.orc_phi.restype = ctypes.c_double
    lib.orc_phi.argtypes = [ctypes.c_double]
    lib.orc_dphi.restype = ctypes.c_double
    lib.orc_dphi.argtypes = [ctypes.c_double]
    lib.orc_forward_causal.argtypes = [dp] * 9 + [L] * 6
    lib.orc_forward_causal_parallel.argtypes = [dp] * 5 + [L] * 5
    lib.orc_forward_noncausal.argtypes = [dp] * 4 + [L] * 6
    lib.orc_numerator_backward.argtypes = [dp] * 9 + [L] * 3
    lib.orc_backward_causal.argtypes = [dp] * 13 + [L] * 6
    lib.orc_backward_noncausal.argtypes = [dp] * 7 + [L] * 6
    lib.orc_decode_step.argtypes = [dp] * 7 + [L] * 5
    lib.orc_forward_decay.argtypes = [dp] * 10 + [L] * 6
    lib.orc_backward_decay.argtypes = [dp] * 15 + [L] * 6
    lib.orc_feature_performer.argtypes = [dp] * 3 + [L] * 5
    lib.orc_feature_performer_vjp.argtypes = [dp] * 4 + [L] * 5
    lib.orc_feature_poly2.argtypes = [dp] * 2 + [L] * 3
    lib.orc_feature_poly2_vjp.argtypes = [dp] * 3 + [L] * 3
    lib.orc_num_threads.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        build()
        _lib = _configure(ctypes.CDLL(_LIB))
    return _lib


def _f64(x):
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(x):
    if x is None:
        return None
    return x.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def num_threads() -> int:
    return int(_load().orc_num_threads())


def phi(x: float) -> float:
    """eq. 7 with elu's alpha = 1."""
    return float(_load().orc_phi(float(x)))


def dphi(x: float) -> float:
    return float(_load().orc_dphi(float(x)))


def forward_causal(q, k, v, s0=None, z0=None, feature=0):
    """Recurrent form, eq. 10-12.  Returns (O, den, S_N, Z_N) in float64."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, D = q.shape
    M = v.shape[-1]
    if (s0 is None) != (z0 is None):
        raise ValueError("s0 and z0 go together")
    s0 = None if s0 is None else _f64(s0)
    z0 = None if z0 is None else _f64(z0)
    o = np.empty((B, H, N, M))
    den = np.empty((B, H, N))
    s = np.empty((B, H, D, M))
    z = np.empty((B, H, D))
    _load().orc_forward_causal(_ptr(q), _ptr(k), _ptr(v), _ptr(s0), _ptr(z0), _ptr(o), _ptr(den),
                               _ptr(s), _ptr(z), B, H, N, D, M, int(feature))
    return o, den, s, z


def forward_causal_parallel(q, k, v):
    """Quadratic masked form of eq. 9.  Returns (O, den)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, D = q.shape
    M = v.shape[-1]
    o = np.empty((B, H, N, M))
    den = np.empty((B, H, N))
    _load().orc_forward_causal_parallel(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(den), B, H, N, D, M)
    return o, den


def forward_noncausal(q, k, v, feature=0):
    """eq. 5-6: S and Z summed over the whole sequence, reused by every query."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, D = q.shape
    M = v.shape[-1]
    o = np.empty((B, H, N, M))
    _load().orc_forward_noncausal(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, H, N, D, M, int(feature))
    return o


def numerator_backward(p, kf, vb, g, rn=None, return_r0=False):
    """eq. 13-15 for one head on feature-mapped inputs: returns (dP, dKf, dVb), and the gradient R0 of the
    initial state when return_r0 (rn: the final state's upstream gradient [C, Mb], None for zero)."""
    p, kf, vb, g = _f64(p), _f64(kf), _f64(vb), _f64(g)
    N, C = p.shape
    Mb = vb.shape[1]
    rn = None if rn is None else _f64(rn)
    dp_ = np.empty((N, C))
    dk = np.empty((N, C))
    dv = np.empty((N, Mb))
    r0 = np.empty((C, Mb))
    _load().orc_numerator_backward(_ptr(p), _ptr(kf), _ptr(vb), _ptr(g), _ptr(rn), _ptr(dp_), _ptr(dk), _ptr(dv),
                                   _ptr(r0), N, C, Mb)
    return (dp_, dk, dv, r0) if return_r0 else (dp_, dk, dv)


def backward_causal(q, k, v, do, s0=None, z0=None, dsn=None, dzn=None, state_grad=False, feature=0):
    """Gradients of sum(dO * O) + sum(dSN * S_N) + sum(dZN * Z_N) w.r.t. raw Q, K, V (and, with state_grad,
    the initial state).  Returns (dQ, dK, dV) or (dQ, dK, dV, dS0, dZ0)."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, H, N, D = q.shape
    M = v.shape[-1]
    s0 = None if s0 is None else _f64(s0)
    z0 = None if z0 is None else _f64(z0)
    if (dsn is None) != (dzn is None):
        raise ValueError("dsn and dzn go together")
    dsn = None if dsn is None else _f64(dsn)
    dzn = None if dzn is None else _f64(dzn)
    dq = np.empty((B, H, N, D))
    dk = np.empty((B, H, N, D))
    dv = np.empty((B, H, N, M))
    ds0 = np.empty((B, H, D, M)) if state_grad else None
    dz0 = np.empty((B, H, D)) if state_grad else None
    _load().orc_backward_causal(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(s0), _ptr(z0), _ptr(dsn), _ptr(dzn),
                                _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ds0), _ptr(dz0), B, H, N, D, M, int(feature))
    return (dq, dk, dv, ds0, dz0) if state_grad else (dq, dk, dv)


def backward_noncausal(q, k, v, do, feature=0):
    """Gradients of sum(dO * O) for the non-causal forward w.r.t. raw Q, K, V.  Returns (dQ, dK, dV)."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, H, N, D = q.shape
    M = v.shape[-1]
    dq = np.empty((B, H, N, D))
    dk = np.empty((B, H, N, D))
    dv = np.empty((B, H, N, M))
    _load().orc_backward_noncausal(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(dq), _ptr(dk), _ptr(dv),
                                   B, H, N, D, M, int(feature))
    return dq, dk, dv


def decode_step(q, k, v, s, z, log_a=None, feature=0):
    """eq. 18-20 (attention part), decayed by exp(log_a) [B,H] when given.  Returns (y, S_new, Z_new); inputs
    untouched."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    log_a = None if log_a is None else _f64(log_a)
    s = np.array(s, dtype=np.float64, copy=True, order="C")
    z = np.array(z, dtype=np.float64, copy=True, order="C")
    B, H, D = q.shape
    M = v.shape[-1]
    y = np.empty((B, H, M))
    _load().orc_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(log_a), _ptr(s), _ptr(z), _ptr(y), B, H, D, M, int(feature))
    return y, s, z


def forward_decay(q, k, v, log_a, s0=None, z0=None, feature=0):
    """Decayed causal forward (per-token, per-head log-decay log_a [B,H,N]).  Returns (O, den, S_N, Z_N)."""
    q, k, v, log_a = _f64(q), _f64(k), _f64(v), _f64(log_a)
    B, H, N, D = q.shape
    M = v.shape[-1]
    s0 = None if s0 is None else _f64(s0)
    z0 = None if z0 is None else _f64(z0)
    o = np.empty((B, H, N, M))
    den = np.empty((B, H, N))
    s = np.empty((B, H, D, M))
    z = np.empty((B, H, D))
    _load().orc_forward_decay(_ptr(q), _ptr(k), _ptr(v), _ptr(log_a), _ptr(s0), _ptr(z0), _ptr(o), _ptr(den),
                              _ptr(s), _ptr(z), B, H, N, D, M, int(feature))
    return o, den, s, z


def backward_decay(q, k, v, log_a, do, s0=None, z0=None, dsn=None, dzn=None, feature=0):
    """Gradients of sum(dO*O) + sum(dSN*S_N) + sum(dZN*Z_N) for the decayed forward.  Returns
    (dQ, dK, dV, dlogA, dS0, dZ0)."""
    q, k, v, log_a, do = _f64(q), _f64(k), _f64(v), _f64(log_a), _f64(do)
    B, H, N, D = q.shape
    M = v.shape[-1]
    s0 = None if s0 is None else _f64(s0)
    z0 = None if z0 is None else _f64(z0)
    if (dsn is None) != (dzn is None):
        raise ValueError("dsn and dzn go together")
    dsn = None if dsn is None else _f64(dsn)
    dzn = None if dzn is None else _f64(dzn)
    dq = np.empty((B, H, N, D))
    dk = np.empty((B, H, N, D))
    dv = np.empty((B, H, N, M))
    dla = np.empty((B, H, N))
    ds0 = np.empty((B, H, D, M))
    dz0 = np.empty((B, H, D))
    _load().orc_backward_decay(_ptr(q), _ptr(k), _ptr(v), _ptr(log_a), _ptr(do), _ptr(s0), _ptr(z0), _ptr(dsn),
                               _ptr(dzn), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dla), _ptr(ds0), _ptr(dz0),
                               B, H, N, D, M, int(feature))
    return dq, dk, dv, dla, ds0, dz0


def feature_performer(x, w):
    """Positive random features phi(x)_c = exp(w_c . x - |x|^2 / 2) / sqrt(C); x [B,H,N,Din], w [H,C,Din]."""
    x, w = _f64(x), _f64(w)
    B, H, N, Din = x.shape
    C = w.shape[1]
    phi_ = np.empty((B, H, N, C))
    _load().orc_feature_performer(_ptr(x), _ptr(w), _ptr(phi_), B, H, N, Din, C)
    return phi_


def feature_performer_vjp(x, w, dphi_):
    x, w, dphi_ = _f64(x), _f64(w), _f64(dphi_)
    B, H, N, Din = x.shape
    C = w.shape[1]
    dx = np.empty((B, H, N, Din))
    _load().orc_feature_performer_vjp(_ptr(x), _ptr(w), _ptr(dphi_), _ptr(dx), B, H, N, Din, C)
    return dx


def feature_poly2(x, C):
    """Degree-2 polynomial features (1, x, x_a x_b) zero-padded to C; x [..., Din]."""
    x = _f64(x)
    Din = x.shape[-1]
    rows = x.size // Din
    phi_ = np.empty(x.shape[:-1] + (C,))
    _load().orc_feature_poly2(_ptr(x), _ptr(phi_), rows, Din, C)
    return phi_


def feature_poly2_vjp(x, dphi_):
    x, dphi_ = _f64(x), _f64(dphi_)
    Din = x.shape[-1]
    rows = x.size // Din
    dx = np.empty(x.shape)
    _load().orc_feature_poly2_vjp(_ptr(x), _ptr(dphi_), _ptr(dx), rows, Din, dphi_.shape[-1])
    return dx
