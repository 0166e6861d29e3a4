"""fp64 CPU oracle for the selective scan: forward, carried state, decode step and
gradients (ctypes wrapper over oracle.c).

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no
code with the HIP implementation and must never be used as a fallback for it.

What it computes is documented in ``oracle.c``; the pins that tie it to the pages
live in ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

OK = 0
ERR_NULL = -1
ERR_EMPTY = -2
ERR_NONFINITE = -3
ERR_RETAIN = -4
ERR_ALLOC = -5


class OracleError(RuntimeError):
    """Raised when the oracle refuses its inputs; ``code`` is the C status."""

    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: oracle status {code}")
        self.code = code


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (plain C, -O2, OpenMP over independent rows)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        i64 = ctypes.c_int64
        lib.oracle_softplus.argtypes = [ctypes.c_double]
        lib.oracle_softplus.restype = ctypes.c_double
        lib.oracle_silu.argtypes = [ctypes.c_double]
        lib.oracle_silu.restype = ctypes.c_double
        lib.oracle_selective_scan_fwd.argtypes = [i64, i64, i64, i64] + [dp] * 9 + [ctypes.c_int]
        lib.oracle_selective_scan_fwd.restype = ctypes.c_int
        lib.oracle_selective_scan_state.argtypes = [i64, i64, i64, i64] + [dp] * 11 + [ctypes.c_int]
        lib.oracle_selective_scan_state.restype = ctypes.c_int
        lib.oracle_sigmoid.argtypes = [ctypes.c_double]
        lib.oracle_sigmoid.restype = ctypes.c_double
        lib.oracle_selective_scan_bwd.argtypes = [i64, i64, i64, i64] + [dp] * 20 + [ctypes.c_int]
        lib.oracle_selective_scan_bwd.restype = ctypes.c_int
        lib.oracle_causal_conv1d.argtypes = [i64, i64, i64, i64] + [dp] * 4 + [ctypes.c_int] + [dp] * 2
        lib.oracle_causal_conv1d.restype = ctypes.c_int
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def softplus(x: float) -> float:
    return _load().oracle_softplus(float(x))


def silu(x: float) -> float:
    return _load().oracle_silu(float(x))


def sigmoid(x: float) -> float:
    return _load().oracle_sigmoid(float(x))


def max_threads() -> int:
    return _load().oracle_max_threads()


def selective_scan_fwd(u, delta, A, B, C, D=None, z=None, dt_bias=None, nthreads: int = 0) -> np.ndarray:
    """fp64 selective-scan forward.

    u, delta, z: (batch, dim, L); B, C: (batch, N, L); A: (dim, N); D, dt_bias: (dim,).
    Every input is converted to float64 exactly (fp32 and bf16 values are exact in fp64).
    Returns y as float64 (batch, dim, L).
    """
    u, delta, A, B, C = (_f64(x) for x in (u, delta, A, B, C))
    D, z, dt_bias = _f64(D), _f64(z), _f64(dt_bias)
    if u.ndim != 3 or B.ndim != 3:
        raise ValueError("u must be (batch, dim, L) and B (batch, N, L)")
    batch, dim, L = u.shape
    N = B.shape[1]
    if delta.shape != u.shape or (z is not None and z.shape != u.shape):
        raise ValueError("delta and z must match u")
    if B.shape != (batch, N, L) or C.shape != (batch, N, L):
        raise ValueError("B and C must be (batch, N, L)")
    if A.shape != (dim, N):
        raise ValueError("A must be (dim, N)")
    for v in (D, dt_bias):
        if v is not None and v.shape != (dim,):
            raise ValueError("D and dt_bias must be (dim,)")
    y = np.zeros((batch, dim, L), dtype=np.float64)
    code = _load().oracle_selective_scan_fwd(
        batch, L, dim, N, _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C),
        _ptr(D), _ptr(z), _ptr(dt_bias), _ptr(y), int(nthreads))
    if code != OK:
        raise OracleError(code, "selective_scan_fwd")
    return y


def selective_scan_state(u, delta, A, B, C, D=None, z=None, dt_bias=None, h0=None, nthreads: int = 0):
    """fp64 selective scan from state h0 (batch, dim, N; None = zeros).

    Returns (y, h_last): y (batch, dim, L) and the state after the last step.
    """
    u, delta, A, B, C = (_f64(x) for x in (u, delta, A, B, C))
    D, z, dt_bias, h0 = _f64(D), _f64(z), _f64(dt_bias), _f64(h0)
    batch, dim, L = u.shape
    N = B.shape[1]
    if h0 is not None and h0.shape != (batch, dim, N):
        raise ValueError("h0 must be (batch, dim, N)")
    if B.shape != (batch, N, L) or C.shape != (batch, N, L) or A.shape != (dim, N):
        raise ValueError("B, C must be (batch, N, L) and A (dim, N)")
    y = np.zeros((batch, dim, L), dtype=np.float64)
    h_last = np.zeros((batch, dim, N), dtype=np.float64)
    code = _load().oracle_selective_scan_state(
        batch, L, dim, N, _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(dt_bias),
        _ptr(h0), _ptr(y), _ptr(h_last), int(nthreads))
    if code != OK:
        raise OracleError(code, "selective_scan_state")
    return y, h_last


def selective_scan_step(u, delta, A, B, C, D=None, z=None, dt_bias=None, h=None):
    """One recurrent decoding step: u, delta, z (batch, dim); B, C (batch, N); state h
    (batch, dim, N; None = zeros).  Returns (y (batch, dim), new state)."""
    u = _f64(u)
    batch, dim = u.shape
    col = lambda a: None if a is None else _f64(a)[..., None]
    y, h_new = selective_scan_state(col(u), col(delta), A, col(B), col(C), D, col(z), dt_bias, h0=h)
    return y[..., 0], h_new


def selective_scan_bwd(u, delta, A, B, C, D=None, z=None, dt_bias=None, dy=None, h0=None, dh_last=None,
                       nthreads: int = 0) -> dict:
    """fp64 gradients of the scan for the loss sum(dy * y) + sum(dh_last * h_last).

    Shapes as for selective_scan_state; dy (batch, dim, L); dh_last (batch, dim, N)
    or None.  Returns a dict with du, ddelta, dA, dB, dC always, dD if D is given,
    dz if z is given, ddt_bias and dh0 always (ddt_bias is the gradient of the bias
    even when no bias is passed).
    """
    u, delta, A, B, C, dy = (_f64(x) for x in (u, delta, A, B, C, dy))
    D, z, dt_bias, h0, dh_last = (_f64(x) for x in (D, z, dt_bias, h0, dh_last))
    batch, dim, L = u.shape
    N = B.shape[1]
    if dy is None or dy.shape != u.shape:
        raise ValueError("dy must be (batch, dim, L)")
    if B.shape != (batch, N, L) or C.shape != (batch, N, L) or A.shape != (dim, N):
        raise ValueError("B, C must be (batch, N, L) and A (dim, N)")
    for name, v in (("h0", h0), ("dh_last", dh_last)):
        if v is not None and v.shape != (batch, dim, N):
            raise ValueError(f"{name} must be (batch, dim, N)")
    out = {
        "du": np.zeros((batch, dim, L)), "ddelta": np.zeros((batch, dim, L)), "dA": np.zeros((dim, N)),
        "dB": np.zeros((batch, N, L)), "dC": np.zeros((batch, N, L)), "ddt_bias": np.zeros(dim),
        "dh0": np.zeros((batch, dim, N)),
    }
    if D is not None:
        out["dD"] = np.zeros(dim)
    if z is not None:
        out["dz"] = np.zeros((batch, dim, L))
    code = _load().oracle_selective_scan_bwd(
        batch, L, dim, N, _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(dt_bias),
        _ptr(h0), _ptr(dy), _ptr(dh_last), _ptr(out["du"]), _ptr(out["ddelta"]), _ptr(out["dA"]),
        _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out.get("dD")), _ptr(out.get("dz")), _ptr(out["ddt_bias"]),
        _ptr(out["dh0"]), int(nthreads))
    if code != OK:
        raise OracleError(code, "selective_scan_bwd")
    return out


def causal_conv1d(x, w, bias=None, state=None, silu=True):
    """fp64 causal depthwise convolution (width K = w.shape[1]) with optional SiLU.

    x (batch, dim, L); w (dim, K); bias (dim,); state (batch, dim, K-1) = the inputs
    before the sequence, oldest first (None = zeros).  Returns (out, state_out) with
    state_out the last K-1 inputs (the history a following call continues from)."""
    x, w, bias, state = _f64(x), _f64(w), _f64(bias), _f64(state)
    batch, dim, L = x.shape
    K = w.shape[1]
    if w.shape != (dim, K) or (bias is not None and bias.shape != (dim,)):
        raise ValueError("w must be (dim, K) and bias (dim,)")
    if state is not None and state.shape != (batch, dim, K - 1):
        raise ValueError("state must be (batch, dim, K-1)")
    out = np.zeros((batch, dim, L))
    st = np.zeros((batch, dim, max(K - 1, 1)))
    code = _load().oracle_causal_conv1d(batch, L, dim, K, _ptr(x), _ptr(w), _ptr(bias),
                                        _ptr(state) if K > 1 else None, int(bool(silu)), _ptr(out),
                                        _ptr(st) if K > 1 else None)
    if code != OK:
        raise OracleError(code, "causal_conv1d")
    return out, st[..., : K - 1]


def ssd_matrix_form(u, delta, A, B, C, D=None, z=None, dt_bias=None, h0=None):
    """fp64 quadratic form of the scalar-decay scan with one step size per head.

    State space duality (yo3nglau.github.io "Mamba 与状态空间模型：面试问题与推荐回答"
    Q10): when the state matrix is a scalar times the identity, the recurrence
    h_t = a_t h_{t-1} + B_t u_t, y_t = C_t . h_t equals one matrix product of the
    inputs with a causal (lower-triangular) mask whose entries are the read-write
    products C_t . B_s times the decay accumulated between s and t.  Written out for
    head h with step sizes dt_t = softplus(delta[b,h,t] + dt_bias[h]) and decay
    exp(dt_t A[h]) per step (cum_t = sum_{k<=t} dt_k A[h]):

        M[t, s] = (C_t . B_s) * exp(cum_t - cum_s) * dt_s        for s <= t, else 0
        y[p, t] = sum_s M[t, s] u[p, s] + exp(cum_t) C_t . h0[p]
        h_last[p] = exp(cum_{L-1}) h0[p] + sum_s exp(cum_{L-1} - cum_s) dt_s u[p, s] B_s

    then y = (y + D u) * SiLU(z) as in the recurrence.  Shapes: u, z (batch, H*P, L)
    with head h owning channels h*P .. h*P+P-1; delta (batch, H, L); A, dt_bias (H,);
    B, C (batch, N, L); D (H*P,); h0 (batch, H*P, N).  Returns (y, h_last).  Plain
    numpy matrix products over the whole sequence: small L only.
    """
    u, delta, A, B, C = (np.asarray(x, dtype=np.float64) for x in (u, delta, A, B, C))
    D, z, dt_bias, h0 = (None if x is None else np.asarray(x, dtype=np.float64) for x in (D, z, dt_bias, h0))
    batch, dim, L = u.shape
    H = delta.shape[1]
    N = B.shape[1]
    if delta.shape != (batch, H, L) or A.shape != (H,) or dim % H:
        raise ValueError("delta must be (batch, H, L), A (H,) and dim a multiple of H")
    if B.shape != (batch, N, L) or C.shape != (batch, N, L):
        raise ValueError("B and C must be (batch, N, L)")
    P = dim // H
    bias = np.zeros(H) if dt_bias is None else dt_bias
    causal = np.tri(L, dtype=bool)
    y = np.zeros((batch, dim, L))
    h_last = np.zeros((batch, dim, N))
    for b in range(batch):
        G = C[b].T @ B[b]                                   # G[t, s] = C_t . B_s
        for h in range(H):
            dt = np.logaddexp(0.0, delta[b, h] + bias[h])   # softplus
            cum = np.cumsum(dt * A[h])
            diff = cum[:, None] - cum[None, :]
            decay = np.where(causal, np.exp(np.where(causal, diff, 0.0)), 0.0)
            M = G * decay * dt[None, :]
            ch = slice(h * P, (h + 1) * P)
            U = u[b, ch]                                    # (P, L)
            Y = U @ M.T
            last = U @ (B[b] * (np.exp(cum[-1] - cum) * dt)[None, :]).T     # (P, N)
            if h0 is not None:
                Y += (h0[b, ch] @ C[b]) * np.exp(cum)[None, :]
                last += np.exp(cum[-1]) * h0[b, ch]
            y[b, ch] = Y
            h_last[b, ch] = last
    if D is not None:
        y += D[None, :, None] * u
    if z is not None:
        y *= z / (1.0 + np.exp(-z))
    return y, h_last
