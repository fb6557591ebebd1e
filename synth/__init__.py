"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random numbers; it holds none of the method's
arithmetic.  Both the GPU path and the CPU oracle read the same host tensors it
returns, so parity compares identical input bits.

Recipe: a CPU ``torch.Generator`` seeded with ``seed``; ``torch.randn`` in
float32; tensors drawn in the order q, k, v, then beta; optionally scaled by an
exact power of two in float32; then cast to the storage dtype (bf16 by
round-to-nearest-even).  Delta-rule interpolation weights are
beta = sigmoid(N(0,1)), drawn in float32 and stored in the input dtype.

Workload shapes (the pages' long-sequence and generation workloads; see the
project's design notes for where each comes from):
  causal_small   B=1   H=1  N=256    D=M=32  fp32
  causal_mid     B=4   H=8  N=4096   D=M=64  fp32
  causal_long    B=2   H=16 N=32768  D=M=64  bf16, N(0,1)*0.5 (also run non-causally)
  decode         B=256 H=16 D=M=64, 512-token prefill + 1024 single-token steps, bf16
  deltanet       B=4   H=8  N=4096   D=M=64  fp32, beta=sigmoid(N(0,1))
  deltanet_decode B=256 H=16 D=M=64, 512-token delta-rule prefill + 1024 single-token
                 steps, bf16, beta=sigmoid(N(0,1))
"""
from __future__ import annotations

from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    D: int
    M: int
    dtype: torch.dtype
    scale: float
    seed: int
    steps: int = 0  # decode only: single-token steps after an N-token prefill


WORKLOADS = {
    "causal_small": Workload("causal_small", 1, 1, 256, 32, 32, torch.float32, 1.0, 1001),
    "causal_mid": Workload("causal_mid", 4, 8, 4096, 64, 64, torch.float32, 1.0, 1002),
    "causal_long": Workload("causal_long", 2, 16, 32768, 64, 64, torch.bfloat16, 0.5, 1003),
    "decode": Workload("decode", 256, 16, 512, 64, 64, torch.bfloat16, 1.0, 1004, steps=1024),
    "deltanet": Workload("deltanet", 4, 8, 4096, 64, 64, torch.float32, 1.0, 1005),
    "deltanet_decode": Workload("deltanet_decode", 256, 16, 512, 64, 64, torch.bfloat16, 1.0, 1006, steps=1024),
    # other feature maps (DPFP-nu, degree-2 polynomial) at the fast-weight page's d_key = 64
    "fmap": Workload("fmap", 4, 8, 4096, 64, 64, torch.float32, 1.0, 1007),
}


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def _draw(g, shape, scale, dtype):
    x = torch.randn(*shape, generator=g, dtype=torch.float32)
    if scale != 1.0:
        x = x * scale  # a power of two: exact in float32
    return x.to(dtype)


def qkv(B, H, N, D, M, *, dtype=torch.float32, scale=1.0, seed=0):
    """q, k: [B,H,N,D]; v: [B,H,N,M]; i.i.d. N(0,1)*scale, stored in ``dtype``."""
    g = _gen(seed)
    q = _draw(g, (B, H, N, D), scale, dtype)
    k = _draw(g, (B, H, N, D), scale, dtype)
    v = _draw(g, (B, H, N, M), scale, dtype)
    return q, k, v


def qkv_beta(B, H, N, D, M, *, dtype=torch.float32, scale=1.0, seed=0):
    """q, k, v as ``qkv`` (same draws), then beta = sigmoid(N(0,1)) of shape [B,H,N]."""
    g = _gen(seed)
    q = _draw(g, (B, H, N, D), scale, dtype)
    k = _draw(g, (B, H, N, D), scale, dtype)
    v = _draw(g, (B, H, N, M), scale, dtype)
    beta = torch.sigmoid(torch.randn(B, H, N, generator=g, dtype=torch.float32)).to(dtype)
    return q, k, v, beta


def kv_cache(B, H, L, D, M, *, dtype=torch.bfloat16, scale=1.0, seed=0):
    """Key and value caches of L earlier tokens for the softmax decode baseline:
    Kc [B,H,L,D], Vc [B,H,L,M], i.i.d. N(0,1)*scale."""
    g = _gen(seed)
    Kc = _draw(g, (B, H, L, D), scale, dtype)
    Vc = _draw(g, (B, H, L, M), scale, dtype)
    return Kc, Vc


def decode_steps(B, H, D, M, T, *, dtype=torch.bfloat16, scale=1.0, seed=0):
    """Fresh per-step inputs for T decode steps: q, k [T,B,H,D]; v [T,B,H,M]."""
    g = _gen(seed)
    q = _draw(g, (T, B, H, D), scale, dtype)
    k = _draw(g, (T, B, H, D), scale, dtype)
    v = _draw(g, (T, B, H, M), scale, dtype)
    return q, k, v


def decode_steps_beta(B, H, D, M, T, *, dtype=torch.bfloat16, scale=1.0, seed=0):
    """Per-step inputs for T delta-rule decode steps: q, k [T,B,H,D]; v [T,B,H,M];
    beta [T,B,H] = sigmoid(N(0,1))."""
    g = _gen(seed)
    q = _draw(g, (T, B, H, D), scale, dtype)
    k = _draw(g, (T, B, H, D), scale, dtype)
    v = _draw(g, (T, B, H, M), scale, dtype)
    beta = torch.sigmoid(torch.randn(T, B, H, generator=g, dtype=torch.float32)).to(dtype)
    return q, k, v, beta


def workload_inputs(w: Workload, seed_offset: int = 0):
    """All inputs of a named workload.  Causal/non-causal: (q, k, v);
    deltanet: (q, k, v, beta); decode: (prefill q, k, v, step q, k, v);
    deltanet_decode: (prefill q, k, v, beta, step q, k, v, beta)."""
    s = w.seed + seed_offset
    if w.name == "deltanet_decode":
        pre = qkv_beta(w.B, w.H, w.N, w.D, w.M, dtype=w.dtype, scale=w.scale, seed=s)
        steps = decode_steps_beta(w.B, w.H, w.D, w.M, w.steps, dtype=w.dtype, scale=w.scale, seed=s + 100000)
        return pre + steps
    if w.name == "deltanet":
        return qkv_beta(w.B, w.H, w.N, w.D, w.M, dtype=w.dtype, scale=w.scale, seed=s)
    if w.name == "decode":
        pre = qkv(w.B, w.H, w.N, w.D, w.M, dtype=w.dtype, scale=w.scale, seed=s)
        steps = decode_steps(w.B, w.H, w.D, w.M, w.steps, dtype=w.dtype, scale=w.scale, seed=s + 100000)
        return pre + steps
    return qkv(w.B, w.H, w.N, w.D, w.M, dtype=w.dtype, scale=w.scale, seed=s)


def sample_rows(N: int, BH: int, n_random: int = 64, seed: int = 7):
    """Row indices (0-based) checked against the explicit form at large N:
    1, 2, 64, 65, 1024, 1025, N/2, N (1-based, those that exist) plus
    ``n_random`` seeded random rows per head.  Returns int64 [BH, R]."""
    fixed = sorted({r - 1 for r in (1, 2, 64, 65, 1024, 1025, N // 2, N) if 1 <= r <= N})
    g = _gen(seed)
    rnd = torch.randint(0, N, (BH, n_random), generator=g, dtype=torch.int64)
    fixed_t = torch.tensor(fixed, dtype=torch.int64).expand(BH, len(fixed))
    return torch.cat([fixed_t, rnd], dim=1)
