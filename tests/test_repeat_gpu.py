"""Bitwise repeatability of every entry point on the GPU.

Any summation order is correct within tolerance, but a fixed build must give
the same bits for the same inputs on every run: the cross-block scans fold in
a fixed order whatever the timing, and no kernel accumulates with atomics.
Each case runs the same call twice (from copies of any in/out state) and
compares the raw bits of every result.  Inputs are the workloads' own.
"""
import pytest
import torch

import synth
import weight_recurrences_amd as la

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print("[case]", *a, flush=True)


def gpu(*ts):
    return [t.to(DEV) for t in ts]


def bits(t):
    torch.cuda.synchronize()
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu()
    return t.contiguous().view(torch.int32).cpu()


def same(a, b):
    return torch.equal(bits(a), bits(b))


@pytest.fixture(scope="module")
def long_inputs():
    w = synth.WORKLOADS["causal_long"]
    return w, gpu(*synth.workload_inputs(w))


def test_causal_with_state_repeatable(long_inputs):
    """The variant that publishes float32 states (the state is requested)."""
    w, (q, k, v) = long_inputs
    say("repeat causal with state", w)
    S0 = torch.randn(w.B, w.H, w.D, w.M, device=DEV)
    z0 = torch.rand(w.B, w.H, w.D, device=DEV) * 3
    a = la.causal(q, k, v, state=(S0, z0), return_state=True)
    b = la.causal(q, k, v, state=(S0, z0), return_state=True)
    assert same(a[0], b[0]) and same(a[1][0], b[1][0]) and same(a[1][1], b[1][1])


def test_causal_fp32_repeatable():
    w = synth.WORKLOADS["causal_mid"]
    say("repeat causal fp32", w)
    q, k, v = gpu(*synth.workload_inputs(w))
    a = la.causal(q, k, v, return_state=True)
    b = la.causal(q, k, v, return_state=True)
    assert same(a[0], b[0]) and same(a[1][0], b[1][0]) and same(a[1][1], b[1][1])


def test_noncausal_repeatable(long_inputs):
    w, (q, k, v) = long_inputs
    say("repeat noncausal", w)
    assert same(la.noncausal(q, k, v), la.noncausal(q, k, v))
    q32, k32, v32 = gpu(*synth.workload_inputs(synth.WORKLOADS["causal_mid"]))
    assert same(la.noncausal(q32, k32, v32), la.noncausal(q32, k32, v32))


def _decode_chain(w, S, z, gq, gk, gv, step):
    outs = torch.empty(w.steps, w.B, w.H, w.M, dtype=w.dtype, device=DEV)
    for t in range(w.steps):
        step(gq[t], gk[t], gv[t], S, z, out=outs[t])
    return outs


def test_decode_chain_repeatable():
    """The decode workload's 1024-step chain twice from the same prefill state."""
    w = synth.WORKLOADS["decode"]
    say("repeat decode chain", w)
    q, k, v, sq, sk, sv = synth.workload_inputs(w)
    S, z = la.causal(*gpu(q, k, v), output=False)
    gq, gk, gv = gpu(sq, sk, sv)
    S1, z1, S2, z2 = S.clone(), z.clone(), S.clone(), z.clone()
    o1 = _decode_chain(w, S1, z1, gq, gk, gv, la.decode_step)
    o2 = _decode_chain(w, S2, z2, gq, gk, gv, la.decode_step)
    assert same(o1, o2) and same(S1, S2) and same(z1, z2)


@pytest.mark.parametrize("N", [1000, 4096], ids=["16_chunks", "64_chunks"])
def test_deltanet_repeatable(N):
    """16 chunks (the last one partial) and 64 chunks, from an initial memory,
    outputs and final memory."""
    w = synth.WORKLOADS["deltanet"]
    say("repeat deltanet", N)
    q, k, v, beta = gpu(*synth.qkv_beta(w.B, w.H, N, w.D, w.M, seed=w.seed + N))
    W0 = torch.randn(w.B, w.H, w.M, w.D, device=DEV) * 0.1
    a = la.deltanet(q, k, v, beta, W0=W0, return_state=True)
    b = la.deltanet(q, k, v, beta, W0=W0, return_state=True)
    assert same(a[0], b[0]) and same(a[1], b[1])


def test_deltanet_sequential_repeatable(monkeypatch):
    monkeypatch.setenv("LINATTN_DELTANET_PATH", "sequential")
    w = synth.WORKLOADS["deltanet"]
    say("repeat deltanet sequential", w)
    q, k, v, beta = gpu(*synth.workload_inputs(w))
    a = la.deltanet(q, k, v, beta, return_state=True)
    b = la.deltanet(q, k, v, beta, return_state=True)
    assert same(a[0], b[0]) and same(a[1], b[1])


def test_deltanet_decode_chain_repeatable():
    w = synth.WORKLOADS["deltanet_decode"]
    say("repeat deltanet decode chain", w)
    q, k, v, beta, sq, sk, sv, sb = synth.workload_inputs(w)
    _, W = la.deltanet(*gpu(q, k, v, beta), return_state=True)
    gq, gk, gv, gb = gpu(sq, sk, sv, sb)
    res = []
    for _ in range(2):
        Wc = W.clone()
        outs = torch.empty(w.steps, w.B, w.H, w.M, dtype=w.dtype, device=DEV)
        for t in range(w.steps):
            la.deltanet_decode_step(gq[t], gk[t], gv[t], gb[t], Wc, out=outs[t])
        res.append((outs, Wc))
    assert same(res[0][0], res[1][0]) and same(res[0][1], res[1][1])


def test_causal_bwd_repeatable(long_inputs):
    w, (q, k, v) = long_inputs
    say("repeat causal bwd", w)
    dO = synth.qkv(w.B, w.H, w.N, w.M, w.M, dtype=w.dtype, seed=w.seed + 50)[0].to(DEV)
    a = la.causal_bwd(q, k, v, dO)
    b = la.causal_bwd(q, k, v, dO)
    assert all(same(x, y) for x, y in zip(a, b))
    q32, k32, v32 = gpu(*synth.qkv(1, 3, 9000, 64, 64, scale=0.5, seed=5))
    d32 = synth.qkv(1, 3, 9000, 64, 64, seed=6)[0].to(DEV)
    a = la.causal_bwd(q32, k32, v32, d32)
    b = la.causal_bwd(q32, k32, v32, d32)
    assert all(same(x, y) for x, y in zip(a, b))


@pytest.mark.parametrize("fm,nu", [(la.FMAP_DPFP, 1), (la.FMAP_DPFP, 3), (la.FMAP_POLY2, 0)],
                         ids=["dpfp1", "dpfp3", "poly2"])
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "noncausal"])
def test_fmap_repeatable(fm, nu, causal):
    w = synth.WORKLOADS["fmap"]
    N = w.N if fm == la.FMAP_DPFP else 1024
    say("repeat fmap", fm, nu, causal, N)
    q, k, v = gpu(*synth.qkv(w.B, w.H, N, w.D, w.M, seed=w.seed))
    a = la.fmap(q, k, v, fm, nu, causal=causal, return_state=True)
    b = la.fmap(q, k, v, fm, nu, causal=causal, return_state=True)
    assert same(a[0], b[0]) and same(a[1][0], b[1][0]) and same(a[1][1], b[1][1])


def test_softmax_decode_repeatable():
    w = synth.WORKLOADS["decode"]
    L = 1200
    say("repeat softmax decode", L)
    Kc, Vc = gpu(*synth.kv_cache(w.B, w.H, L + 1, w.D, w.M, dtype=w.dtype, seed=w.seed + 80))
    sq, sk, sv = synth.decode_steps(w.B, w.H, w.D, w.M, 1, dtype=w.dtype, seed=w.seed + 81)
    q, k, v = gpu(sq[0], sk[0], sv[0])
    K1, V1, K2, V2 = Kc.clone(), Vc.clone(), Kc.clone(), Vc.clone()
    a = la.softmax_decode_step(q, k, v, K1, V1, L)
    b = la.softmax_decode_step(q, k, v, K2, V2, L)
    assert same(a, b) and same(K1, K2) and same(V1, V2)
