"""CPU oracle for the selective-scan forward -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The product path (the HIP library and its binding) never calls it
and shares no code with it.

``scan_fwd`` runs the plain float64 sequential recurrence in ``ss_oracle.c``
(see that file's header for the definition and the passages it follows):

    dt_t = softplus(delta_t + bias)          (optional softplus, optional bias)
    h_t  = exp(dt_t * A) * h_{t-1} + k_t * B_t * u_t      k_t = dt_t, or (exp(dt_t A) - 1) / A (zoh)
                    (or the exponential-trapezoidal rule with ``trapezoid``: see ss_oracle.c)
    y_t  = C_t . h_t + D * u_t               (optional D)
    y_t *= silu(z_t)                         (optional gate)

Inputs may be float32, float64 or bf16 bit patterns (uint16); the oracle decodes
bf16 exactly, so it sees the same values as the GPU.  A, D and delta_bias are
widened exactly to float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ss_oracle.c")
_LIB = os.path.join(_HERE, "libssoracle.so")

_F32, _BF16, _F64 = 0, 1, 2


class _Problem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64), ("channels", ctypes.c_int64), ("length", ctypes.c_int64),
        ("nstate", ctypes.c_int64), ("groups", ctypes.c_int64), ("heads", ctypes.c_int64),
        ("in_dtype", ctypes.c_int32), ("a_per_head", ctypes.c_int32),
        ("d_per_head", ctypes.c_int32), ("softplus", ctypes.c_int32),
        ("u", ctypes.c_void_p), ("delta", ctypes.c_void_p), ("B", ctypes.c_void_p),
        ("C", ctypes.c_void_p), ("z", ctypes.c_void_p),
        ("A", ctypes.c_void_p), ("D", ctypes.c_void_p), ("delta_bias", ctypes.c_void_p),
        ("h0", ctypes.c_void_p), ("zoh", ctypes.c_int32), ("trap", ctypes.c_int32),
    ]


class _Grads(ctypes.Structure):
    _fields_ = [(k, ctypes.c_void_p) for k in ("du", "ddelta", "dA", "dB", "dC", "dD", "dz", "dbias", "dh0")]


def build(force: bool = True) -> str:
    """Compile ss_oracle.c into libssoracle.so with gcc (plain -O2, no fast-math)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-Wall", "-Werror",
                    "-o", tmp, _SRC, "-lm"], check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        build(force=False)
        lib = ctypes.CDLL(_LIB)
        lib.sso_scan_fwd.argtypes = [ctypes.POINTER(_Problem), ctypes.c_void_p, ctypes.c_int64,
                                     ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        lib.sso_scan_fwd.restype = ctypes.c_int
        lib.sso_scan_bwd.argtypes = [ctypes.POINTER(_Problem), ctypes.c_void_p, ctypes.POINTER(_Grads),
                                     ctypes.c_int]
        lib.sso_scan_bwd.restype = ctypes.c_int
        _lib = lib
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _code(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return _BF16
    if a.dtype == np.float32:
        return _F32
    if a.dtype == np.float64:
        return _F64
    raise TypeError("oracle inputs must be float32, float64 or bf16 bits (uint16), got %s" % a.dtype)


def scan_fwd(u: np.ndarray, delta: np.ndarray, A: np.ndarray, B: np.ndarray, C: np.ndarray,
             D: Optional[np.ndarray] = None, z: Optional[np.ndarray] = None,
             delta_bias: Optional[np.ndarray] = None, *, softplus: bool = True,
             rows: Optional[Sequence[int]] = None, h0: Optional[np.ndarray] = None,
             return_state: bool = False, threads: Optional[int] = None, zoh: bool = False,
             trapezoid: bool = False):
    """Float64 reference output.

    Shapes: u, z [batch, channels, L]; delta [batch, heads, L]; A [channels, N] or [heads]
    (scalar decay per head); B, C [batch, groups, N, L]; D [channels] or [heads];
    delta_bias [heads].  ``rows`` selects rows r = b * channels + d (default: all).
    Returns y as [batch, channels, L] when rows is None, else [len(rows), L]; with
    ``return_state`` also the final state [rows, N].  ``h0`` is an optional initial
    state [rows, N].
    """
    u = np.ascontiguousarray(u)
    delta = np.ascontiguousarray(delta)
    B = np.ascontiguousarray(B)
    C = np.ascontiguousarray(C)
    code = _code(u)
    for name, t in (("delta", delta), ("B", B), ("C", C), ("z", z)):
        if t is not None and _code(t) != code:
            raise TypeError("oracle: %s dtype %s differs from u dtype %s" % (name, t.dtype, u.dtype))
    if z is not None:
        z = np.ascontiguousarray(z)
    Bt, Dc, L = u.shape
    H = delta.shape[1]
    G, N = B.shape[1], B.shape[2]
    if delta.shape != (Bt, H, L) or B.shape != (Bt, G, N, L) or C.shape != B.shape:
        raise ValueError("oracle: inconsistent shapes")
    if z is not None and z.shape != u.shape:
        raise ValueError("oracle: z shape")
    A64 = np.ascontiguousarray(A, dtype=np.float64)
    a_per_head = 1 if A64.ndim == 1 else 0
    if a_per_head and A64.shape != (H,):
        raise ValueError("oracle: scalar-decay A must be [heads]")
    if not a_per_head and A64.shape != (Dc, N):
        raise ValueError("oracle: A must be [channels, N]")
    D64 = None if D is None else np.ascontiguousarray(D, dtype=np.float64)
    d_per_head = 0
    if D64 is not None:
        if D64.shape == (Dc,):
            d_per_head = 0
        elif D64.shape == (H,):
            d_per_head = 1
        else:
            raise ValueError("oracle: D must be [channels] or [heads]")
    bias64 = None if delta_bias is None else np.ascontiguousarray(delta_bias, dtype=np.float64)
    if bias64 is not None and bias64.shape != (H,):
        raise ValueError("oracle: delta_bias must be [heads]")
    if rows is None:
        nrows = Bt * Dc
        rows_arr = None
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
        nrows = rows_arr.size
    h0_64 = None
    if h0 is not None:
        h0_64 = np.ascontiguousarray(h0, dtype=np.float64)
        if h0_64.shape != (nrows, N):
            raise ValueError("oracle: h0 must be [rows, N]")
    y = np.empty((nrows, L), dtype=np.float64)
    hf = np.empty((nrows, N), dtype=np.float64) if return_state else None

    def ptr(a):
        return None if a is None else a.ctypes.data

    prob = _Problem(Bt, Dc, L, N, G, H, code, a_per_head, d_per_head, 1 if softplus else 0,
                    ptr(u), ptr(delta), ptr(B), ptr(C), ptr(z), ptr(A64), ptr(D64), ptr(bias64),
                    ptr(h0_64), 1 if zoh else 0, 1 if trapezoid else 0)
    rc = _load().sso_scan_fwd(ctypes.byref(prob), ptr(rows_arr), nrows, ptr(y), ptr(hf),
                              int(threads or default_threads()))
    if rc != 0:
        raise RuntimeError("oracle failed (rc=%d)" % rc)
    if rows is None:
        y = y.reshape(Bt, Dc, L)
    return (y, hf) if return_state else y


def scan_problem(p, *, rows=None, h0=None, return_state=False, threads=None):
    """Run the oracle on a Problem from the seeded input generator."""
    return scan_fwd(p.u, p.delta, p.A, p.B, p.C, p.D, p.z, p.delta_bias, softplus=p.softplus,
                    rows=rows, h0=h0, return_state=return_state, threads=threads,
                    zoh=getattr(p, "zoh", False), trapezoid=getattr(p, "trapezoid", False))


def scan_bwd(u: np.ndarray, delta: np.ndarray, A: np.ndarray, B: np.ndarray, C: np.ndarray,
             D: Optional[np.ndarray] = None, z: Optional[np.ndarray] = None,
             delta_bias: Optional[np.ndarray] = None, *, dy: np.ndarray, softplus: bool = True,
             h0: Optional[np.ndarray] = None, threads: Optional[int] = None) -> dict:
    """Float64 gradients of sum(dy * y) for the forward of ``scan_fwd`` (same arguments; dy is
    [batch, channels, L]).  Returns a dict with du, ddelta, dA, dB, dC and, when the matching
    input is given, dD, dz, ddelta_bias; dh0 [batch * channels, N] is the gradient of the
    initial state.  The definition (the chain rule of the recurrence, reverse in time) is in
    ss_oracle.c."""
    u = np.ascontiguousarray(u)
    delta = np.ascontiguousarray(delta)
    B = np.ascontiguousarray(B)
    C = np.ascontiguousarray(C)
    code = _code(u)
    for name, t in (("delta", delta), ("B", B), ("C", C), ("z", z)):
        if t is not None and _code(t) != code:
            raise TypeError("oracle: %s dtype %s differs from u dtype %s" % (name, t.dtype, u.dtype))
    if z is not None:
        z = np.ascontiguousarray(z)
    Bt, Dc, L = u.shape
    H = delta.shape[1]
    G, N = B.shape[1], B.shape[2]
    if delta.shape != (Bt, H, L) or B.shape != (Bt, G, N, L) or C.shape != B.shape:
        raise ValueError("oracle: inconsistent shapes")
    dy64 = np.ascontiguousarray(dy, dtype=np.float64)
    if dy64.shape != (Bt, Dc, L):
        raise ValueError("oracle: dy must be [batch, channels, L]")
    A64 = np.ascontiguousarray(A, dtype=np.float64)
    a_per_head = 1 if A64.ndim == 1 else 0
    D64 = None if D is None else np.ascontiguousarray(D, dtype=np.float64)
    d_per_head = 1 if (D64 is not None and D64.shape == (H,) and H != Dc) else 0
    bias64 = None if delta_bias is None else np.ascontiguousarray(delta_bias, dtype=np.float64)
    h0_64 = None if h0 is None else np.ascontiguousarray(h0, dtype=np.float64).reshape(Bt * Dc, N)
    out = dict(du=np.empty((Bt, Dc, L)), ddelta=np.empty((Bt, H, L)), dA=np.empty(A64.shape),
               dB=np.empty((Bt, G, N, L)), dC=np.empty((Bt, G, N, L)),
               dD=None if D64 is None else np.empty(D64.shape),
               dz=None if z is None else np.empty((Bt, Dc, L)),
               ddelta_bias=None if bias64 is None else np.empty((H,)), dh0=np.empty((Bt * Dc, N)))

    def ptr(a):
        return None if a is None else a.ctypes.data

    prob = _Problem(Bt, Dc, L, N, G, H, code, a_per_head, d_per_head, 1 if softplus else 0,
                    ptr(u), ptr(delta), ptr(B), ptr(C), ptr(z), ptr(A64), ptr(D64), ptr(bias64),
                    ptr(h0_64), 0, 0)
    grads = _Grads(ptr(out["du"]), ptr(out["ddelta"]), ptr(out["dA"]), ptr(out["dB"]), ptr(out["dC"]),
                   ptr(out["dD"]), ptr(out["dz"]), ptr(out["ddelta_bias"]), ptr(out["dh0"]))
    rc = _load().sso_scan_bwd(ctypes.byref(prob), ptr(dy64), ctypes.byref(grads), int(threads or default_threads()))
    if rc != 0:
        raise RuntimeError("oracle backward failed (rc=%d)" % rc)
    return out


def scan_bwd_problem(p, dy, *, h0=None, threads=None) -> dict:
    """``scan_bwd`` on a Problem from the seeded input generator."""
    return scan_bwd(p.u, p.delta, p.A, p.B, p.C, p.D, p.z, p.delta_bias, dy=dy, softplus=p.softplus,
                    h0=h0, threads=threads)


def conv1d(x: np.ndarray, w: np.ndarray, bias: Optional[np.ndarray] = None, *, state: Optional[np.ndarray] = None,
           silu: bool = False, return_state: bool = False):
    """Float64 causal depthwise convolution (see ss_oracle.c): x [batch, channels, L] (float32,
    float64 or bf16 bits), w [channels, W], bias [channels], state [batch, channels, W - 1] (the
    inputs before t = 0, oldest first).  Returns out [batch, channels, L] (and the last W - 1
    inputs with ``return_state``)."""
    lib = _load()
    if not hasattr(lib, "_conv_bound"):
        lib.sso_conv1d.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                                   ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                   ctypes.c_void_p, ctypes.c_void_p]
        lib.sso_conv1d.restype = ctypes.c_int
        lib._conv_bound = True
    x = np.ascontiguousarray(x)
    Bt, Dc, L = x.shape
    w64 = np.ascontiguousarray(w, dtype=np.float64)
    W = w64.shape[1]
    b64 = None if bias is None else np.ascontiguousarray(bias, dtype=np.float64)
    s64 = None if state is None else np.ascontiguousarray(state, dtype=np.float64).reshape(Bt * Dc, W - 1)
    out = np.empty((Bt, Dc, L))
    so = np.empty((Bt, Dc, max(W - 1, 0)))
    ptr = lambda a: None if a is None else a.ctypes.data
    rc = lib.sso_conv1d(Bt, Dc, L, _code(x), ptr(x), ptr(w64), W, ptr(b64), ptr(s64), 1 if silu else 0, ptr(out),
                        ptr(so))
    if rc != 0:
        raise RuntimeError("oracle conv1d failed (rc=%d)" % rc)
    return (out, so) if return_state else out
