"""CPU oracle (fp64) for causal linear attention, its non-causal and decode
forms, the same forms with other feature maps (DPFP-nu, degree-2 polynomial),
the fast-weight delta rule and the softmax decode baseline.

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package; the GPU library
(``weight_recurrences_amd``) never does, and the two share no code.

The arithmetic lives in ``linattn_oracle.c`` (plain fp64 loops, one function
per form the pages give).  This module only converts inputs to float64 exactly,
calls the C functions through ctypes and returns numpy arrays.  It compiles the
C file with gcc when the shared object is missing or older than its source.

Inputs may be numpy arrays or CPU torch tensors of any float dtype (bf16 and
fp32 values convert to float64 without rounding).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "linattn_oracle.c")
_SO = os.path.join(_HERE, "liblinattn_oracle.so")
_lock = threading.Lock()
_lib = None

_D = ctypes.POINTER(ctypes.c_double)
_I = ctypes.POINTER(ctypes.c_int64)
_i64 = ctypes.c_int64


def build(force: bool = False) -> str:
    """Compile the oracle's C source into ``liblinattn_oracle.so`` (gcc, OpenMP)."""
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-Wall",
             _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    with _lock:
        if _lib is None:
            # LINATTN_ORACLE_LIB names another build of the same source (the
            # sanitizer test loads one built with ASan and UBSan).
            alt = os.environ.get("LINATTN_ORACLE_LIB")
            if not alt:
                build()
            lib = ctypes.CDLL(alt or _SO)
            lib.oracle_phi.restype = ctypes.c_double
            lib.oracle_phi.argtypes = [ctypes.c_double]
            lib.oracle_set_threads.argtypes = [ctypes.c_int]
            lib.oracle_get_threads.restype = ctypes.c_int
            lib.oracle_causal_explicit_rows.argtypes = [_D, _D, _D, _i64, _i64, _i64, _i64, _I, _i64, _D]
            lib.oracle_causal_recurrent.argtypes = [_D, _D, _D, _i64, _i64, _i64, _i64, _D, _D, _D, _D, _D]
            lib.oracle_noncausal_explicit_rows.argtypes = [_D, _D, _D, _i64, _i64, _i64, _i64, _I, _i64, _D]
            lib.oracle_noncausal.argtypes = [_D, _D, _D, _i64, _i64, _i64, _i64, _D, _D, _D]
            lib.oracle_decode_step.argtypes = [_D, _D, _D, _i64, _i64, _i64, _D, _D, _D]
            lib.oracle_deltanet.argtypes = [_D, _D, _D, _D, _i64, _i64, _i64, _i64, _D, _D, _D]
            lib.oracle_softmax_decode.argtypes = [_D, _D, _D, _i64, _i64, _i64, _i64, _i64, _D]
            lib.oracle_fmap_dim.restype = _i64
            lib.oracle_fmap_dim.argtypes = [ctypes.c_int, ctypes.c_int, _i64]
            lib.oracle_fmap.argtypes = [_D, _i64, ctypes.c_int, ctypes.c_int, _D]
            lib.oracle_fmap_causal.argtypes = [_D, _D, _D, _i64, _i64, _i64, _i64, ctypes.c_int, ctypes.c_int,
                                               _D, _D, _D, _D, _D]
            lib.oracle_fmap_noncausal.argtypes = [_D, _D, _D, _i64, _i64, _i64, _i64, ctypes.c_int, ctypes.c_int,
                                                  _D, _D, _D]
            _lib = lib
    return _lib


def f64(x) -> np.ndarray:
    """Exact conversion of a numpy array or CPU torch tensor to C-contiguous float64."""
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor: bf16/fp16/fp32 -> fp32 -> fp64 is exact
        x = x.detach().to("cpu")
        import torch  # local: only when a tensor is passed
        x = x.to(torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _p(a):
    return None if a is None else a.ctypes.data_as(_D)


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def get_threads() -> int:
    return int(_load().oracle_get_threads())


def phi(x: float) -> float:
    """phi(x) = elu(x) + 1 (alpha = 1) in fp64, as the C oracle computes it."""
    return float(_load().oracle_phi(float(x)))


def _split4(q, k, v):
    q, k, v = f64(q), f64(k), f64(v)
    if q.ndim != 4:
        raise ValueError("expected [B, H, N, D] tensors")
    B, H, N, D = q.shape
    M = v.shape[-1]
    assert k.shape == (B, H, N, D) and v.shape == (B, H, N, M)
    return q, k, v, B, H, N, D, M


def causal(q, k, v, S0=None, z0=None, want_output=True):
    """Recurrent causal form, eq.(10)-(12).  Returns (o or None, S, z) as float64:
    o [B,H,N,M], S [B,H,D,M], z [B,H,D]."""
    q, k, v, B, H, N, D, M = _split4(q, k, v)
    S0, z0 = f64(S0), f64(z0)
    o = np.empty((B, H, N, M)) if want_output else None
    S = np.empty((B, H, D, M))
    z = np.empty((B, H, D))
    _load().oracle_causal_recurrent(_p(q), _p(k), _p(v), B * H, N, D, M, _p(S0), _p(z0),
                                    _p(o), _p(S), _p(z))
    return o, S, z


def _rows_arg(rows, BH, N):
    rows = np.asarray(rows, dtype=np.int64)
    if rows.ndim == 1:
        rows = np.broadcast_to(rows, (BH, rows.shape[0]))
    rows = np.ascontiguousarray(rows.reshape(BH, -1))
    if rows.size and (rows.min() < 0 or rows.max() >= N):
        raise ValueError("row index out of range")
    return rows


def causal_explicit(q, k, v, rows=None):
    """Explicit quadratic causal form, eq.(8) with sim = phi(q)^T phi(k).
    ``rows``: 0-based row indices, shared by every head ([R]) or per head
    ([B*H, R]); default all rows.  Returns float64 [B, H, R, M]."""
    q, k, v, B, H, N, D, M = _split4(q, k, v)
    rows = _rows_arg(np.arange(N) if rows is None else rows, B * H, N)
    R = rows.shape[1]
    out = np.empty((B, H, R, M))
    _load().oracle_causal_explicit_rows(_p(q), _p(k), _p(v), B * H, N, D, M,
                                        rows.ctypes.data_as(_I), R, _p(out))
    return out


def noncausal(q, k, v):
    """Non-causal form by associativity, eq.(5)-(6).  Returns (o, S, z) float64."""
    q, k, v, B, H, N, D, M = _split4(q, k, v)
    o = np.empty((B, H, N, M))
    S = np.empty((B, H, D, M))
    z = np.empty((B, H, D))
    _load().oracle_noncausal(_p(q), _p(k), _p(v), B * H, N, D, M, _p(o), _p(S), _p(z))
    return o, S, z


def noncausal_explicit(q, k, v, rows=None):
    """Explicit non-causal form, eq.(4) (sums over all keys).  Returns [B,H,R,M]."""
    q, k, v, B, H, N, D, M = _split4(q, k, v)
    rows = _rows_arg(np.arange(N) if rows is None else rows, B * H, N)
    R = rows.shape[1]
    out = np.empty((B, H, R, M))
    _load().oracle_noncausal_explicit_rows(_p(q), _p(k), _p(v), B * H, N, D, M,
                                           rows.ctypes.data_as(_I), R, _p(out))
    return out


def decode_step(q, k, v, S, z):
    """One RNN step, eq.(18)-(20), on float64 copies of (S, z).
    q, k: [B,H,D]; v: [B,H,M]; S: [B,H,D,M]; z: [B,H,D].
    Returns (o [B,H,M], S_new, z_new)."""
    q, k, v = f64(q), f64(k), f64(v)
    S = f64(S).copy()
    z = f64(z).copy()
    B, H, D = q.shape
    M = v.shape[-1]
    assert S.shape == (B, H, D, M) and z.shape == (B, H, D)
    o = np.empty((B, H, M))
    _load().oracle_decode_step(_p(q), _p(k), _p(v), B * H, D, M, _p(S), _p(z), _p(o))
    return o, S, z


def deltanet(q, k, v, beta, W0=None):
    """Delta-rule fast-weight memory with sum-normalised phi.
    q, k: [B,H,N,D]; v: [B,H,N,M]; beta: [B,H,N]; W0: [B,H,M,D] or None.
    Returns (o [B,H,N,M], W [B,H,M,D]) float64."""
    q, k, v, B, H, N, D, M = _split4(q, k, v)
    beta = f64(beta)
    assert beta.shape == (B, H, N)
    W0 = f64(W0)
    o = np.empty((B, H, N, M))
    W = np.empty((B, H, M, D))
    _load().oracle_deltanet(_p(q), _p(k), _p(v), _p(beta), B * H, N, D, M, _p(W0), _p(o), _p(W))
    return o, W


def softmax_decode(q, k, v, Kc, Vc, L):
    """Softmax attention decode step over a key/value cache ([TR] eq.(2), App. C.1):
    the new key and value are appended at row L of float64 copies of the caches and
    o = softmax(q K^T / sqrt(D)) V over rows 0..L.
    q, k: [B,H,D]; v: [B,H,M]; Kc: [B,H,Lmax,D]; Vc: [B,H,Lmax,M].
    Returns (o [B,H,M], Kc_new, Vc_new) float64."""
    q, k, v = f64(q), f64(k), f64(v)
    Kc = f64(Kc).copy()
    Vc = f64(Vc).copy()
    B, H, D = q.shape
    M = v.shape[-1]
    Lmax = Kc.shape[2]
    assert 0 <= L < Lmax and Kc.shape == (B, H, Lmax, D) and Vc.shape == (B, H, Lmax, M)
    Kc[:, :, L] = k
    Vc[:, :, L] = v
    o = np.empty((B, H, M))
    _load().oracle_softmax_decode(_p(q), _p(Kc), _p(Vc), B * H, L, Lmax, D, M, _p(o))
    return o, Kc, Vc


# Feature maps other than elu + 1 (the C oracle's fmap codes).
DPFP = 1   # DPFP-nu, C = 2 nu D  ([FWP], the DPFP paragraph and its figure)
POLY2 = 2  # degree-2 polynomial, C = D^2  ([TR] §3.2.1)


def fmap_dim(fmap: int, nu: int, D: int) -> int:
    """Feature dimension C of the map (0 for an unknown map)."""
    return int(_load().oracle_fmap_dim(int(fmap), int(nu), int(D)))


def feature_map(x, fmap: int, nu: int = 0):
    """phi(x) for every row of x [..., D]; returns float64 [..., C]."""
    x = f64(x)
    D = x.shape[-1]
    C = fmap_dim(fmap, nu, D)
    rows = np.ascontiguousarray(x.reshape(-1, D))
    out = np.empty((rows.shape[0], C))
    lib = _load()
    for r in range(rows.shape[0]):
        lib.oracle_fmap(_p(rows[r]), D, int(fmap), int(nu), _p(out[r]))
    return out.reshape(x.shape[:-1] + (C,))


def fmap_causal(q, k, v, fmap: int, nu: int = 0, S0=None, z0=None, want_output=True):
    """Recurrent causal form, eq.(10)-(12), with the feature map ``fmap``.
    Returns (o or None [B,H,N,M], S [B,H,C,M], z [B,H,C]) float64."""
    q, k, v, B, H, N, D, M = _split4(q, k, v)
    C = fmap_dim(fmap, nu, D)
    S0, z0 = f64(S0), f64(z0)
    if S0 is not None:
        assert S0.shape == (B, H, C, M) and z0.shape == (B, H, C)
    o = np.empty((B, H, N, M)) if want_output else None
    S = np.empty((B, H, C, M))
    z = np.empty((B, H, C))
    _load().oracle_fmap_causal(_p(q), _p(k), _p(v), B * H, N, D, M, int(fmap), int(nu), _p(S0), _p(z0),
                               _p(o), _p(S), _p(z))
    return o, S, z


def fmap_noncausal(q, k, v, fmap: int, nu: int = 0):
    """Non-causal form, eq.(5)-(6), with the feature map ``fmap``.
    Returns (o [B,H,N,M], S [B,H,C,M], z [B,H,C]) float64."""
    q, k, v, B, H, N, D, M = _split4(q, k, v)
    C = fmap_dim(fmap, nu, D)
    o = np.empty((B, H, N, M))
    S = np.empty((B, H, C, M))
    z = np.empty((B, H, C))
    _load().oracle_fmap_noncausal(_p(q), _p(k), _p(v), B * H, N, D, M, int(fmap), int(nu), _p(o), _p(S), _p(z))
    return o, S, z


from .gradients import causal_bwd  # noqa: E402  (fp64 autograd of the forward definition)
