"""fp64 gradients of causal linear attention (test infrastructure only).

The pages ("Transformers are RNNs", translated page "線性變換器", §3.3.1) state
that the gradient of the causal numerator can be computed with cumulative sums
in linear time and constant memory, but print neither the equations nor the
derivation (the appendix is omitted).  The oracle therefore does not restate
any derived formula: it differentiates the forward definition itself with
torch's float64 autograd on the CPU, for the loss L = sum_i dO_i . o_i:

  phi(x) = x + 1 (x > 0), exp(x) otherwise              (§3.2.1 eq.(7))
  S_i = sum_{j<=i} phi(k_j) v_j^T,  z_i = sum_{j<=i} phi(k_j)   (§3.3 eq.(10)-(11))
  o_i = phi(q_i)^T S_i / phi(q_i)^T z_i                  (§3.3 eq.(12))

Two forms are provided and pinned against each other and against central
finite differences in the CPU tests: the recurrent form above (prefix sums,
used for every size) and the explicit masked form of eq.(9) (small sizes).

TEST INFRASTRUCTURE ONLY: only the tests, the smoke check and the benchmark's
CPU baseline use this module; the GPU library never does.
"""
from __future__ import annotations

import numpy as np
import torch


def _t64(x) -> torch.Tensor:
    if isinstance(x, torch.Tensor):
        return x.detach().to(device="cpu", dtype=torch.float64).clone()
    return torch.as_tensor(np.asarray(x, dtype=np.float64)).clone()


def _phi(x: torch.Tensor) -> torch.Tensor:
    # elu(x) + 1 with alpha = 1; both branches meet at x = 0 with slope 1
    return torch.where(x > 0, x + 1.0, torch.exp(torch.clamp(x, max=0.0)))


def causal_forward_recurrent(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor) -> torch.Tensor:
    """o [N, M] of one head from prefix sums (eq.(10)-(12)); differentiable."""
    fq, fk = _phi(q), _phi(k)
    S = torch.cumsum(fk[:, :, None] * v[:, None, :], dim=0)  # [N, D, M]
    z = torch.cumsum(fk, dim=0)                               # [N, D]
    num = torch.einsum("nd,ndm->nm", fq, S)
    den = (fq * z).sum(dim=1, keepdim=True)
    return num / den


def causal_forward_explicit(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor) -> torch.Tensor:
    """o [N, M] of one head from the masked similarity matrix (eq.(9)); differentiable."""
    fq, fk = _phi(q), _phi(k)
    A = torch.tril(fq @ fk.T)                                 # j <= i
    return (A @ v) / A.sum(dim=1, keepdim=True)


def causal_bwd(q, k, v, dO, form: str = "recurrent"):
    """Gradients (dq, dk, dv) of L = sum(dO * o) for q, k [B,H,N,D], v, dO [B,H,N,M].

    Returns float64 numpy arrays of the input shapes."""
    q, k, v, dO = _t64(q), _t64(k), _t64(v), _t64(dO)
    B, H, N, D = q.shape
    M = v.shape[-1]
    fwd = causal_forward_recurrent if form == "recurrent" else causal_forward_explicit
    dq = torch.zeros_like(q)
    dk = torch.zeros_like(k)
    dv = torch.zeros_like(v)
    for b in range(B):
        for h in range(H):
            if N == 0:
                continue
            qh = q[b, h].clone().requires_grad_(True)
            kh = k[b, h].clone().requires_grad_(True)
            vh = v[b, h].clone().requires_grad_(True)
            o = fwd(qh, kh, vh)
            gq, gk, gv = torch.autograd.grad((o * dO[b, h]).sum(), (qh, kh, vh))
            dq[b, h], dk[b, h], dv[b, h] = gq, gk, gv
    return dq.numpy(), dk.numpy(), dv.numpy()


def causal_loss(q, k, v, dO, form: str = "recurrent") -> float:
    """L = sum(dO * o) in float64 (for finite differences)."""
    q, k, v, dO = _t64(q), _t64(k), _t64(v), _t64(dO)
    fwd = causal_forward_recurrent if form == "recurrent" else causal_forward_explicit
    total = 0.0
    with torch.no_grad():
        for b in range(q.shape[0]):
            for h in range(q.shape[1]):
                total += float((fwd(q[b, h], k[b, h], v[b, h]) * dO[b, h]).sum())
    return total


def dq_term_scale(q, k, v, dO) -> np.ndarray:
    """Size of the terms dq is formed from, per (b, h, token) row, float64 [B,H,N].

    For the error bound of the query gradient only (test infrastructure).  By
    the quotient rule on eq.(12), the gradient of L with respect to phi(q_i) is
    (S_i dO_i - z_i (dO_i . o_i)) / den_i with den_i = phi(q_i)^T z_i: two
    vectors that can nearly cancel, so that any float32 evaluation of a row
    carries an error of float32 rounding times their size, however small the
    row itself is.  Returned: || phi'(q_i) * max(|S_i dO_i|, |z_i (dO_i . o_i)|) / den_i ||_inf,
    with phi'(x) = 1 (x > 0), exp(x) otherwise.  The formula is pinned against
    the autograd gradient in the CPU tests.
    """
    q, k, v, dO = _t64(q), _t64(k), _t64(v), _t64(dO)
    B, H, N, D = q.shape
    out = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            if N == 0:
                continue
            fq, fk = _phi(q[b, h]), _phi(k[b, h])
            S = torch.cumsum(fk[:, :, None] * v[b, h][:, None, :], dim=0)   # [N, D, M]
            z = torch.cumsum(fk, dim=0)                                      # [N, D]
            den = (fq * z).sum(dim=1, keepdim=True)
            o = torch.einsum("nd,ndm->nm", fq, S) / den
            t1 = torch.einsum("ndm,nm->nd", S, dO[b, h]).abs()
            t2 = (z * (dO[b, h] * o).sum(dim=1, keepdim=True)).abs()
            dphi = torch.where(q[b, h] > 0, torch.ones_like(fq), torch.exp(torch.clamp(q[b, h], max=0.0)))
            out[b, h] = (dphi * torch.maximum(t1, t2) / den).amax(dim=1).numpy()
    return out


def dq_from_terms(q, k, v, dO) -> np.ndarray:
    """dq from the quotient-rule form above, float64 [B,H,N,D]; used only by the
    CPU pin that ties dq_term_scale's formula to the autograd gradient."""
    q, k, v, dO = _t64(q), _t64(k), _t64(v), _t64(dO)
    B, H, N, D = q.shape
    out = np.zeros((B, H, N, D))
    for b in range(B):
        for h in range(H):
            fq, fk = _phi(q[b, h]), _phi(k[b, h])
            S = torch.cumsum(fk[:, :, None] * v[b, h][:, None, :], dim=0)
            z = torch.cumsum(fk, dim=0)
            den = (fq * z).sum(dim=1, keepdim=True)
            o = torch.einsum("nd,ndm->nm", fq, S) / den
            g = (torch.einsum("ndm,nm->nd", S, dO[b, h]) - z * (dO[b, h] * o).sum(dim=1, keepdim=True)) / den
            dphi = torch.where(q[b, h] > 0, torch.ones_like(fq), torch.exp(torch.clamp(q[b, h], max=0.0)))
            out[b, h] = (dphi * g).numpy()
    return out
