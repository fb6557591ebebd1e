"""MI355X (gfx950) causal linear attention: thin torch binding over liblinattn.so.

Every function below only checks and marshals arguments: all arithmetic runs
in the library's HIP kernels, enqueued on the current torch stream of the
tensors' device.  torch provides device memory and streams, nothing else.

Method: "Transformers are RNNs" (Katharopoulos et al., 2020), translated page
"線性變換器" — phi = elu + 1 (§3.2.1 eq.(7)), causal form eq.(9)-(12),
non-causal form eq.(5)-(6), RNN step eq.(16)-(20), other feature maps
(§3.2.1: degree-2 polynomial; DPFP-nu from the fast-weight summary); delta-rule fast-weight
memory from the news summary of "Linear Transformers Are Secretly Fast Weight
Programmers" (Schlag et al., 2021), update-rule and normalisation paragraphs.
"""
from __future__ import annotations

import torch

from ._lib import BF16, F32, FMAP_DPFP, FMAP_POLY2, LinAttnError, check, load

__all__ = ["causal", "causal_bwd", "fmap", "fmap_dim", "fmap_workspace_bytes", "FMAP_DPFP", "FMAP_POLY2", "causal_bwd_workspace_bytes", "noncausal", "noncausal_noalloc", "decode_step", "deltanet", "deltanet_decode_step", "causal_workspace_bytes",
           "noncausal_workspace_bytes", "deltanet_workspace_bytes", "LinAttnError", "abi_version"]

_DT = {torch.float32: F32, torch.bfloat16: BF16}


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype}; expected float32 or bfloat16")
    return _DT[t.dtype]


def _dev(*ts):
    dev = ts[0].device
    if dev.type != "cuda":
        raise ValueError("tensors must live on a GPU device (the library has no CPU path)")
    for t in ts:
        if t is None:
            continue
        if t.device != dev:
            raise ValueError("all tensors must be on the same device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    return dev


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(dev):
    return torch.cuda.current_stream(dev).cuda_stream


def abi_version() -> int:
    return int(load().linattn_abi_version())


def causal_workspace_bytes(B, H, N, D, M, dtype) -> int:
    return int(load().linattn_causal_workspace_bytes(B, H, N, D, M, _DT[dtype]))


def noncausal_workspace_bytes(B, H, N, D, M, dtype) -> int:
    return int(load().linattn_noncausal_workspace_bytes(B, H, N, D, M, _DT[dtype]))


def _workspace(nbytes, dev, workspace):
    if nbytes == 0:
        return None
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError("workspace too small")
        return workspace
    return torch.empty(nbytes, dtype=torch.uint8, device=dev)


def causal(q, k, v, *, state=None, return_state=False, output=True, out=None, workspace=None):
    """Causal linear attention, eq.(9)-(12).

    q, k: [B,H,N,D]; v: [B,H,N,M] (float32 or bfloat16, same dtype).
    state: optional (S0 [B,H,D,M], z0 [B,H,D]) float32 initial state.
    Returns o [B,H,N,M] (dtype of q), or (o, (S, z)) with return_state; with
    output=False only the final state (S, z) is computed and returned.
    """
    lib = load()
    dev = _dev(q, k, v)
    B, H, N, D = q.shape
    M = v.shape[-1]
    if k.shape != q.shape or v.shape[:3] != q.shape[:3] or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v shapes/dtypes disagree")
    dt = _dtype_code(q)
    S0 = z0 = None
    if state is not None:
        S0, z0 = state
        _dev(q, S0, z0)
        if S0.dtype != torch.float32 or z0.dtype != torch.float32 or S0.shape != (B, H, D, M) or z0.shape != (B, H, D):
            raise ValueError("state must be float32 S [B,H,D,M] and z [B,H,D]")
    o = None
    if output:
        o = out if out is not None else torch.empty((B, H, N, M), dtype=q.dtype, device=dev)
    S = z = None
    if return_state or not output:
        S = torch.empty((B, H, D, M), dtype=torch.float32, device=dev)
        z = torch.empty((B, H, D), dtype=torch.float32, device=dev)
    need = int(lib.linattn_causal_workspace_bytes(B, H, N, D, M, dt))
    ws = _workspace(need, dev, workspace)
    rc = lib.linattn_causal_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, H, N, D, M, dt,
                                _ptr(S0), _ptr(z0), _ptr(S), _ptr(z), _ptr(ws), need, _stream(dev))
    check(rc, "linattn_causal_fwd")
    if not output:
        return S, z
    return (o, (S, z)) if return_state else o


def fmap_dim(fmap: int, nu: int, D: int) -> int:
    """Feature dimension C of DPFP-nu (2 nu D) or the polynomial map (D^2); 0 if unsupported."""
    return int(load().linattn_fmap_dim(int(fmap), int(nu), int(D)))


def fmap_workspace_bytes(B, H, N, D, M, dtype, fmap, nu=0) -> int:
    return int(load().linattn_fmap_workspace_bytes(B, H, N, D, M, _DT[dtype], int(fmap), int(nu)))


def fmap(q, k, v, feature_map, nu=0, *, causal=True, state=None, return_state=False, output=True, out=None,
         workspace=None):
    """Linear attention with another feature map (linattn_fmap_fwd):
    ``feature_map`` is FMAP_DPFP (order ``nu`` in 1..3) or FMAP_POLY2 (nu = 0).

    q, k: [B,H,N,D]; v: [B,H,N,M] (float32 or bfloat16).  causal selects
    eq.(9)-(12) or eq.(5)-(6).  state: optional (S0 [B,H,C,M], z0 [B,H,C])
    float32 (causal only).  Returns o, or (o, (S, z)) with return_state; with
    output=False only the final (or total) state (S, z).
    """
    lib = load()
    dev = _dev(q, k, v)
    B, H, N, D = q.shape
    M = v.shape[-1]
    if k.shape != q.shape or v.shape[:3] != q.shape[:3] or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v shapes/dtypes disagree")
    dt = _dtype_code(q)
    C = fmap_dim(feature_map, nu, D)
    if C == 0:
        raise LinAttnError(4, "linattn_fmap_fwd")
    S0 = z0 = None
    if state is not None:
        S0, z0 = state
        _dev(q, S0, z0)
        if S0.dtype != torch.float32 or z0.dtype != torch.float32 or S0.shape != (B, H, C, M) or z0.shape != (B, H, C):
            raise ValueError("state must be float32 S [B,H,C,M] and z [B,H,C]")
    o = None
    if output:
        o = out if out is not None else torch.empty((B, H, N, M), dtype=q.dtype, device=dev)
    S = z = None
    if return_state or not output:
        S = torch.empty((B, H, C, M), dtype=torch.float32, device=dev)
        z = torch.empty((B, H, C), dtype=torch.float32, device=dev)
    need = int(lib.linattn_fmap_workspace_bytes(B, H, N, D, M, dt, int(feature_map), int(nu)))
    ws = _workspace(need, dev, workspace)
    rc = lib.linattn_fmap_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, H, N, D, M, dt, int(feature_map), int(nu),
                              1 if causal else 0, _ptr(S0), _ptr(z0), _ptr(S), _ptr(z), _ptr(ws), need,
                              _stream(dev))
    check(rc, "linattn_fmap_fwd")
    if not output:
        return S, z
    return (o, (S, z)) if return_state else o


def causal_bwd_workspace_bytes(B, H, N, D, M, dtype) -> int:
    return int(load().linattn_causal_bwd_workspace_bytes(B, H, N, D, M, _DT[dtype]))


def causal_bwd(q, k, v, dO, *, out=None, workspace=None):
    """Gradients (dq, dk, dv) of sum(dO * causal(q, k, v)) from a zero state.

    q, k: [B,H,N,D]; v, dO: [B,H,N,M] (float32 or bfloat16, one dtype); the
    gradients come back in that dtype.  ``out`` may give (dq, dk, dv)."""
    lib = load()
    dev = _dev(q, k, v, dO)
    B, H, N, D = q.shape
    M = v.shape[-1]
    if k.shape != q.shape or v.shape[:3] != q.shape[:3] or dO.shape != v.shape:
        raise ValueError("q, k [B,H,N,D], v, dO [B,H,N,M] expected")
    if k.dtype != q.dtype or v.dtype != q.dtype or dO.dtype != q.dtype:
        raise ValueError("q, k, v, dO must share a dtype")
    dt = _dtype_code(q)
    if out is not None:
        dq, dk, dv = out
    else:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    need = int(lib.linattn_causal_bwd_workspace_bytes(B, H, N, D, M, dt))
    ws = _workspace(need, dev, workspace)
    rc = lib.linattn_causal_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(dO), _ptr(dq), _ptr(dk), _ptr(dv), B, H, N, D, M,
                                dt, _ptr(ws), need, _stream(dev))
    check(rc, "linattn_causal_bwd")
    return dq, dk, dv


def noncausal(q, k, v, *, out=None, workspace=None):
    """Non-causal linear attention, eq.(5)-(6).  Returns o [B,H,N,M]."""
    lib = load()
    dev = _dev(q, k, v)
    B, H, N, D = q.shape
    M = v.shape[-1]
    if k.shape != q.shape or v.shape[:3] != q.shape[:3] or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v shapes/dtypes disagree")
    dt = _dtype_code(q)
    o = out if out is not None else torch.empty((B, H, N, M), dtype=q.dtype, device=dev)
    need = int(lib.linattn_noncausal_workspace_bytes(B, H, N, D, M, dt))
    ws = _workspace(need, dev, workspace)
    rc = lib.linattn_noncausal_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, H, N, D, M, dt, _ptr(ws), need,
                                   _stream(dev))
    check(rc, "linattn_noncausal_fwd")
    return o


def noncausal_noalloc(q, k, v, *, out=None):
    """Non-causal linear attention through ``linattn_noncausal_fwd_noalloc``: no
    workspace argument and no device allocation inside the call (the library's
    static per-GPU scratch; calls that overlap on one GPU race).  Returns o."""
    lib = load()
    dev = _dev(q, k, v)
    B, H, N, D = q.shape
    M = v.shape[-1]
    if k.shape != q.shape or v.shape[:3] != q.shape[:3] or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v shapes/dtypes disagree")
    dt = _dtype_code(q)
    o = out if out is not None else torch.empty((B, H, N, M), dtype=q.dtype, device=dev)
    _dev(q, o)
    rc = lib.linattn_noncausal_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, H, N, D, M, dt, _stream(dev))
    check(rc, "linattn_noncausal_fwd_noalloc")
    return o


def decode_step(q, k, v, S, z, *, out=None):
    """One RNN step, eq.(18)-(20), updating (S, z) in place.

    q, k: [B,H,D]; v: [B,H,M] (float32 or bfloat16); S [B,H,D,M], z [B,H,D]
    float32.  Returns o [B,H,M] in the dtype of q.
    """
    lib = load()
    dev = _dev(q, k, v, S, z)
    B, H, D = q.shape
    M = v.shape[-1]
    if S.dtype != torch.float32 or z.dtype != torch.float32 or S.shape != (B, H, D, M) or z.shape != (B, H, D):
        raise ValueError("state must be float32 S [B,H,D,M] and z [B,H,D]")
    dt = _dtype_code(q)
    o = out if out is not None else torch.empty((B, H, M), dtype=q.dtype, device=dev)
    rc = lib.linattn_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(S), _ptr(z), B, H, D, M, dt,
                                 _stream(dev))
    check(rc, "linattn_decode_step")
    return o


def softmax_decode_step(q, k, v, Kc, Vc, L, *, out=None):
    """Softmax attention decode step over a key/value cache (the stateful-softmax
    baseline, eq.(2)): k, v are written to row L of the caches and
    o = softmax(q Kc[0..L]^T / sqrt(D)) Vc[0..L] is returned.

    q, k: [B,H,D]; v: [B,H,M]; Kc: [B,H,Lmax,D]; Vc: [B,H,Lmax,M], all of one
    dtype (float32 or bfloat16).  Returns o [B,H,M] in that dtype.
    """
    lib = load()
    dev = _dev(q, k, v, Kc, Vc)
    B, H, D = q.shape
    M = v.shape[-1]
    Lmax = Kc.shape[2]
    if k.shape != q.shape or v.shape[:2] != q.shape[:2] or Kc.shape != (B, H, Lmax, D) or Vc.shape != (B, H, Lmax, M):
        raise ValueError("q, k [B,H,D]; v [B,H,M]; Kc [B,H,Lmax,D]; Vc [B,H,Lmax,M]")
    if len({t.dtype for t in (q, k, v, Kc, Vc)}) != 1:
        raise ValueError("q, k, v and the caches must share one dtype")
    dt = _dtype_code(q)
    o = out if out is not None else torch.empty((B, H, M), dtype=q.dtype, device=dev)
    rc = lib.softmax_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(Kc), _ptr(Vc), B, H, int(L), Lmax, D, M, dt,
                                 _stream(dev))
    check(rc, "softmax_decode_step")
    return o


def deltanet_workspace_bytes(B, H, N, D, M, dtype) -> int:
    return int(load().deltanet_workspace_bytes(B, H, N, D, M, _DT[dtype]))


def deltanet(q, k, v, beta, *, W0=None, return_state=False, out=None, workspace=None):
    """Delta-rule fast-weight memory with sum-normalised phi.

    q, k: [B,H,N,D]; v: [B,H,N,M]; beta: [B,H,N] (same dtype, beta used as
    given); W0: optional float32 [B,H,M,D].  Returns o [B,H,N,M], or
    (o, W [B,H,M,D]) with return_state.
    """
    lib = load()
    dev = _dev(q, k, v, beta, W0)
    B, H, N, D = q.shape
    M = v.shape[-1]
    dt = _dtype_code(q)
    if beta.shape != (B, H, N) or beta.dtype != q.dtype:
        raise ValueError("beta must be [B,H,N] in the dtype of q")
    if W0 is not None and (W0.dtype != torch.float32 or W0.shape != (B, H, M, D)):
        raise ValueError("W0 must be float32 [B,H,M,D]")
    o = out if out is not None else torch.empty((B, H, N, M), dtype=q.dtype, device=dev)
    W = torch.empty((B, H, M, D), dtype=torch.float32, device=dev) if return_state else None
    need = int(lib.deltanet_workspace_bytes(B, H, N, D, M, dt))
    ws = _workspace(need, dev, workspace)
    rc = lib.deltanet_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(o), B, H, N, D, M, dt,
                          _ptr(W0), _ptr(W), _ptr(ws), need, _stream(dev))
    check(rc, "deltanet_fwd")
    return (o, W) if return_state else o


def deltanet_decode_step(q, k, v, beta, W, *, out=None):
    """One delta-rule step (the RNN form of ``deltanet`` for one token),
    updating the memory W in place.

    q, k: [B,H,D]; v: [B,H,M]; beta: [B,H] (float32 or bfloat16, same dtype);
    W [B,H,M,D] float32.  Returns o [B,H,M] in the dtype of q.
    """
    lib = load()
    dev = _dev(q, k, v, beta, W)
    B, H, D = q.shape
    M = v.shape[-1]
    dt = _dtype_code(q)
    if k.shape != q.shape or v.shape[:2] != (B, H) or beta.shape != (B, H):
        raise ValueError("q, k [B,H,D], v [B,H,M], beta [B,H] expected")
    if k.dtype != q.dtype or v.dtype != q.dtype or beta.dtype != q.dtype:
        raise ValueError("q, k, v, beta must share a dtype")
    if W.dtype != torch.float32 or W.shape != (B, H, M, D):
        raise ValueError("W must be float32 [B,H,M,D]")
    o = out if out is not None else torch.empty((B, H, M), dtype=q.dtype, device=dev)
    rc = lib.deltanet_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(o), _ptr(W), B, H, D, M, dt,
                                  _stream(dev))
    check(rc, "deltanet_decode_step")
    return o
