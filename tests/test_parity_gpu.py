"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Both sides read the same seeded host tensors.  Errors are row-wise relative
(max over rows of ||y - r||_inf / ||r||_inf); tolerances: 1e-4 for float32
inputs, 2e-2 for bfloat16 inputs with float32 accumulation.  States are float32
in every mode and are held to 1e-4 (per matrix, max |err| / max |ref|), also
in bf16 runs: the state update multiplies the exact bf16 values by phi(k)
split into a bf16 head and tail, so the state carries float32-level error.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import gradients
import weight_recurrences_amd as la
from oracle.metrics import grad_rel_err, mat_rel_err, row_rel_err

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}
STATE_TOL = {torch.float32: 1e-4, torch.bfloat16: 1e-4}
DEV = "cuda:0"


def say(*a):
    print("[case]", *a, flush=True)


def gpu(*ts):
    return [None if t is None else t.to(DEV) for t in ts]


def host(t):
    torch.cuda.synchronize()
    return t.detach().to("cpu")


# ---------------------------------------------------------------- causal

@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("D,M", [(32, 32), (32, 64), (64, 32), (64, 64)])
@pytest.mark.parametrize("N", [1, 3, 63, 64, 65, 200, 1000, 2500])
def test_causal_ragged(dtype, D, M, N):
    say("causal", dtype, D, M, N)
    q, k, v = synth.qkv(2, 3, N, D, M, dtype=dtype, seed=N * 7 + D + M)
    o, (S, z) = la.causal(*gpu(q, k, v), return_state=True)
    ro, rS, rz = oracle.causal(q, k, v)
    assert row_rel_err(host(o), ro) < TOL[dtype]
    assert mat_rel_err(host(S), rS) < STATE_TOL[dtype]
    assert mat_rel_err(host(z), rz, 1) < STATE_TOL[dtype]
    # outputs only: the bf16 kernel then forms the state increments from the
    # bf16 head of phi(k) alone
    assert row_rel_err(host(la.causal(*gpu(q, k, v))), ro) < TOL[dtype]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("B,H,N", [(1, 1, 40000), (1, 2, 20000), (3, 100, 700), (2, 5, 9000)])
def test_causal_many_blocks_with_state(dtype, B, H, N):
    """Long sequences over few heads (and many heads over short ones): the
    single-pass kernels then spread one head's blocks over several rounds of
    workgroups, which exercises every look-back case."""
    D, M = 64, 64
    say("causal many blocks", dtype, B, H, N)
    q, k, v = synth.qkv(B, H, N, D, M, dtype=dtype, seed=B * 1000 + H * 10 + N)
    S0 = torch.randn(B, H, D, M, generator=torch.Generator().manual_seed(N)) * 3
    z0 = torch.rand(B, H, D, generator=torch.Generator().manual_seed(N + 1)) * 5
    o, (S, z) = la.causal(*gpu(q, k, v), state=(S0.to(DEV), z0.to(DEV)), return_state=True)
    ro, rS, rz = oracle.causal(q, k, v, S0=S0, z0=z0)
    assert row_rel_err(host(o), ro) < TOL[dtype]
    assert mat_rel_err(host(S), rS) < STATE_TOL[dtype]
    assert mat_rel_err(host(z), rz, 1) < STATE_TOL[dtype]
    o2 = la.causal(*gpu(q, k, v), state=(S0.to(DEV), z0.to(DEV)))
    assert row_rel_err(host(o2), ro) < TOL[dtype]


@pytest.mark.parametrize("dtype,B,H,N,exact", [(torch.bfloat16, 1, 8, 4096, False), (torch.bfloat16, 2, 3, 3000, True),
                                               (torch.bfloat16, 1, 16, 2304, False), (torch.float32, 1, 8, 2000, True),
                                               (torch.float32, 2, 3, 1500, False)],
                         ids=["bf16-8h", "bf16-6h-state", "bf16-16h", "f32-8h-state", "f32-6h"])
def test_causal_lookback_slow_path(monkeypatch, dtype, B, H, N, exact):
    """With a look-back wait bound of 0 every block whose predecessors have not
    published yet takes the slow path and computes their increments directly from
    K and V; the results must still match the oracle (bf16 with and without the
    state, float32, B*H a multiple of 8 and not)."""
    D, M = 64, 64
    say("causal look-back slow path", dtype, B, H, N, exact)
    monkeypatch.setenv("LINATTN_LOOKBACK_SPIN_TICKS", "0")
    q, k, v = synth.qkv(B, H, N, D, M, dtype=dtype, seed=N + H)
    S0 = torch.randn(B, H, D, M, generator=torch.Generator().manual_seed(N)) * 2
    z0 = torch.rand(B, H, D, generator=torch.Generator().manual_seed(N + 1)) * 4
    ro, rS, rz = oracle.causal(q, k, v, S0=S0, z0=z0)
    if exact:
        o, (S, z) = la.causal(*gpu(q, k, v), state=gpu(S0, z0), return_state=True)
        assert mat_rel_err(host(S), rS) < STATE_TOL[dtype]
        assert mat_rel_err(host(z), rz, 1) < STATE_TOL[dtype]
    else:
        o = la.causal(*gpu(q, k, v), state=gpu(S0, z0))
    assert row_rel_err(host(o), ro) < TOL[dtype]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("D,M", [(32, 32), (32, 64), (64, 32), (64, 64)])
@pytest.mark.parametrize("N", [1, 65, 1000, 2500])
def test_causal_blocked_path(monkeypatch, dtype, D, M, N):
    """LINATTN_CAUSAL_PATH=blocked sends causal calls through the three-kernel
    path (block states, block scan, chunked sweep): outputs, final state from an
    initial state, and outputs only, against the oracle."""
    monkeypatch.setenv("LINATTN_CAUSAL_PATH", "blocked")
    say("causal blocked", dtype, D, M, N)
    q, k, v = synth.qkv(2, 3, N, D, M, dtype=dtype, seed=N * 5 + D + 3 * M)
    S0 = torch.randn(2, 3, D, M, generator=torch.Generator().manual_seed(N)) * 2
    z0 = torch.rand(2, 3, D, generator=torch.Generator().manual_seed(N + 1)) * 4
    o, (S, z) = la.causal(*gpu(q, k, v), state=gpu(S0, z0), return_state=True)
    ro, rS, rz = oracle.causal(q, k, v, S0=S0, z0=z0)
    assert row_rel_err(host(o), ro) < TOL[dtype]
    assert mat_rel_err(host(S), rS) < STATE_TOL[dtype]
    assert mat_rel_err(host(z), rz, 1) < STATE_TOL[dtype]
    ro, _, _ = oracle.causal(q, k, v)
    assert row_rel_err(host(la.causal(*gpu(q, k, v))), ro) < TOL[dtype]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_causal_blocked_path_long_head(monkeypatch, dtype):
    """The blocked path over many blocks of one head (its block scan), the long
    workload's head length."""
    monkeypatch.setenv("LINATTN_CAUSAL_PATH", "blocked")
    q, k, v = synth.qkv(1, 2, 32768, 64, 64, dtype=dtype, scale=0.5, seed=77)
    say("causal blocked long head", dtype)
    o = host(la.causal(*gpu(q, k, v)))
    ro, _, _ = oracle.causal(q, k, v)
    assert row_rel_err(o, ro) < (2e-2 if dtype == torch.bfloat16 else 1e-4)


def test_causal_small_workload_all_rows_explicit():
    w = synth.WORKLOADS["causal_small"]
    say(w)
    q, k, v = synth.workload_inputs(w)
    o = la.causal(*gpu(q, k, v))
    assert row_rel_err(host(o), oracle.causal_explicit(q, k, v)) < 1e-4


def test_causal_mid_workload():
    w = synth.WORKLOADS["causal_mid"]
    say(w)
    q, k, v = synth.workload_inputs(w)
    o, (S, z) = la.causal(*gpu(q, k, v), return_state=True)
    o = host(o)
    ro, rS, rz = oracle.causal(q, k, v)
    assert row_rel_err(o, ro) < 1e-4
    assert mat_rel_err(host(S), rS) < 1e-4 and mat_rel_err(host(z), rz, 1) < 1e-4
    rows = synth.sample_rows(w.N, w.B * w.H, n_random=16)
    ex = oracle.causal_explicit(q, k, v, rows=rows)
    got = torch.gather(o.reshape(w.B * w.H, w.N, w.M), 1, rows[..., None].expand(-1, -1, w.M))
    assert row_rel_err(got.reshape(ex.shape), ex) < 1e-4


@pytest.fixture(scope="module")
def long_inputs():
    w = synth.WORKLOADS["causal_long"]
    return w, synth.workload_inputs(w)


def test_causal_long_workload(long_inputs):
    w, (q, k, v) = long_inputs
    say(w)
    o, (S, z) = la.causal(*gpu(q, k, v), return_state=True)
    o = host(o)
    ro, rS, rz = oracle.causal(q, k, v)
    assert row_rel_err(o, ro) < 2e-2
    assert mat_rel_err(host(S), rS) < 1e-4 and mat_rel_err(host(z), rz, 1) < 1e-4
    rows = synth.sample_rows(w.N, w.B * w.H, n_random=32)
    ex = oracle.causal_explicit(q, k, v, rows=rows)
    got = torch.gather(o.reshape(w.B * w.H, w.N, w.M), 1, rows[..., None].expand(-1, -1, w.M))
    assert row_rel_err(got.reshape(ex.shape), ex) < 2e-2


def test_causal_long_workload_outputs_only(long_inputs):
    """The measured configuration: outputs only, no state requested."""
    w, (q, k, v) = long_inputs
    say("outputs only", w)
    o = host(la.causal(*gpu(q, k, v)))
    ro, _, _ = oracle.causal(q, k, v, want_output=True)
    assert row_rel_err(o, ro) < 2e-2
    rows = synth.sample_rows(w.N, w.B * w.H, n_random=32)
    ex = oracle.causal_explicit(q, k, v, rows=rows)
    got = torch.gather(o.reshape(w.B * w.H, w.N, w.M), 1, rows[..., None].expand(-1, -1, w.M))
    assert row_rel_err(got.reshape(ex.shape), ex) < 2e-2


def test_causal_long_repeatable(long_inputs):
    w, (q, k, v) = long_inputs
    say("repeat", w)
    qg, kg, vg = gpu(q, k, v)
    a = host(la.causal(qg, kg, vg))
    b = host(la.causal(qg, kg, vg))
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_noncausal_long_workload(long_inputs):
    w, (q, k, v) = long_inputs
    say("noncausal", w)
    o = host(la.noncausal(*gpu(q, k, v)))
    ro, _, _ = oracle.noncausal(q, k, v)
    assert row_rel_err(o, ro) < 2e-2
    rows = synth.sample_rows(w.N, w.B * w.H, n_random=4)[:, :6]
    ex = oracle.noncausal_explicit(q, k, v, rows=rows)
    got = torch.gather(o.reshape(w.B * w.H, w.N, w.M), 1, rows[..., None].expand(-1, -1, w.M))
    assert row_rel_err(got.reshape(ex.shape), ex) < 2e-2


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("D,M", [(32, 32), (32, 64), (64, 32), (64, 64)])
@pytest.mark.parametrize("N", [1, 65, 1000, 2500])
def test_noncausal_ragged(dtype, D, M, N):
    say("noncausal", dtype, D, M, N)
    q, k, v = synth.qkv(2, 2, N, D, M, dtype=dtype, seed=N + 3 * D + M)
    o = host(la.noncausal(*gpu(q, k, v)))
    ro, _, _ = oracle.noncausal(q, k, v)
    assert row_rel_err(o, ro) < TOL[dtype]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_state_carry_split_sequence(dtype):
    N, D, M = 3000, 64, 64
    say("carry", dtype)
    q, k, v = synth.qkv(1, 4, N, D, M, dtype=dtype, seed=11)
    ro, rS, rz = oracle.causal(q, k, v)
    qg, kg, vg = gpu(q, k, v)
    for P in (1, 700, 2048, 2999):
        S, z = la.causal(qg[:, :, :P].contiguous(), kg[:, :, :P].contiguous(), vg[:, :, :P].contiguous(),
                         output=False)
        # in-place carry: S_out is the same buffer as S0
        S1, z1 = S.clone(), z.clone()
        lib = la._lib.load()
        rest = [t[:, :, P:].contiguous() for t in (qg, kg, vg)]
        o2 = torch.empty_like(rest[2])
        need = la.causal_workspace_bytes(1, 4, N - P, D, M, dtype)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=DEV)
        rc = lib.linattn_causal_fwd(rest[0].data_ptr(), rest[1].data_ptr(), rest[2].data_ptr(), o2.data_ptr(),
                                    1, 4, N - P, D, M, 0 if dtype == torch.float32 else 1,
                                    S1.data_ptr(), z1.data_ptr(), S1.data_ptr(), z1.data_ptr(),
                                    ws.data_ptr(), need, torch.cuda.current_stream().cuda_stream)
        assert rc == 0
        assert row_rel_err(host(o2), ro[:, :, P:]) < TOL[dtype]
        assert mat_rel_err(host(S1), rS) < STATE_TOL[dtype]
        assert mat_rel_err(host(z1), rz, 1) < STATE_TOL[dtype]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_state_only_and_empty_sequences(dtype):
    say("state-only / empty", dtype)
    q, k, v = synth.qkv(3, 2, 777, 32, 64, dtype=dtype, seed=5)
    S0 = torch.randn(3, 2, 32, 64, dtype=torch.float64)
    z0 = torch.rand(3, 2, 32, dtype=torch.float64) * 10
    S0f, z0f = S0.float(), z0.float()
    S, z = la.causal(*gpu(q, k, v), state=(S0f.to(DEV), z0f.to(DEV)), output=False)
    _, rS, rz = oracle.causal(q, k, v, S0=S0f, z0=z0f, want_output=False)
    assert mat_rel_err(host(S), rS) < 1e-4 and mat_rel_err(host(z), rz, 1) < 1e-4
    # N = 0: the final state is the initial state
    e = torch.empty(3, 2, 0, 32, dtype=dtype, device=DEV)
    ev = torch.empty(3, 2, 0, 64, dtype=dtype, device=DEV)
    o, (S, z) = la.causal(e, e, ev, state=(S0f.to(DEV), z0f.to(DEV)), return_state=True)
    assert o.shape == (3, 2, 0, 64)
    assert torch.equal(host(S), S0f) and torch.equal(host(z), z0f)
    o, (S, z) = la.causal(e, e, ev, return_state=True)
    assert torch.count_nonzero(host(S)) == 0 and torch.count_nonzero(host(z)) == 0


def test_causal_one_hot_slots_exact():
    """Keys that select one slot each (phi = e_c exactly in float32): every output
    row is the mean of the small-integer values stored in the query's slot."""
    N, D, M = 300, 32, 32
    say("one-hot")
    g = torch.Generator().manual_seed(3)
    slots = torch.randint(0, D, (N,), generator=g)
    k = torch.full((1, 1, N, D), -200.0)
    k[0, 0, torch.arange(N), slots] = 0.0
    q = torch.full((1, 1, N, D), -200.0)
    q[..., int(slots[0])] = 0.0
    v = torch.randint(-8, 9, (1, 1, N, M), generator=g).float()
    o = host(la.causal(*gpu(q, k, v)))
    want = np.zeros((N, M))
    sel = []
    for i in range(N):
        if slots[i] == slots[0]:
            sel.append(i)
        want[i] = v[0, 0, sel].numpy().mean(axis=0)
    np.testing.assert_allclose(o[0, 0].numpy(), want, rtol=0, atol=1e-5)


# ---------------------------------------------------------------- decode

@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("D,M", [(32, 32), (32, 64), (64, 32), (64, 64)])
def test_decode_steps_small(dtype, D, M):
    B, H, P, T = 3, 5, 40, 6
    say("decode", dtype, D, M)
    q, k, v = synth.qkv(B, H, P, D, M, dtype=dtype, seed=D * M)
    sq, sk, sv = synth.decode_steps(B, H, D, M, T, dtype=dtype, seed=D + M)
    S, z = la.causal(*gpu(q, k, v), output=False)
    _, rS, rz = oracle.causal(q, k, v, want_output=False)
    gq, gk, gv = gpu(sq, sk, sv)
    for t in range(T):
        o = la.decode_step(gq[t], gk[t], gv[t], S, z)
        ro, rS, rz = oracle.decode_step(sq[t], sk[t], sv[t], rS, rz)
        assert row_rel_err(host(o), ro) < TOL[dtype]
    assert mat_rel_err(host(S), rS) < 1e-4 and mat_rel_err(host(z), rz, 1) < 1e-4


def _steps_as_sequence(x, b0, b1):
    """Per-step tensors [T, B, H, X] -> the sequence [B, H, T, X] of batch rows b0:b1."""
    return x[:, b0:b1].permute(1, 2, 0, 3).contiguous()


def test_decode_workload_all_heads():
    """Full decode workload (prefill 512 + 1024 steps on 256 x 16 states, the
    launch sequence the benchmark times), every head at every step, and the
    final fp32 states of every head.  The oracle applies the recurrent form's
    loop body once per step from the prefill state, which is the recurrent form
    run over the steps as a sequence starting from (S0, z0) = the prefill state."""
    w = synth.WORKLOADS["decode"]
    say(w)
    q, k, v, sq, sk, sv = synth.workload_inputs(w)
    S, z = la.causal(*gpu(q, k, v), output=False)
    _, rS, rz = oracle.causal(q, k, v, want_output=False)
    assert mat_rel_err(host(S), rS) < 1e-4 and mat_rel_err(host(z), rz, 1) < 1e-4
    gq, gk, gv = gpu(sq, sk, sv)
    outs = torch.empty(w.steps, w.B, w.H, w.M, dtype=w.dtype, device=DEV)
    for t in range(w.steps):
        la.decode_step(gq[t], gk[t], gv[t], S, z, out=outs[t])
    outs, S, z = host(outs), host(S), host(z)
    step = 32
    for b0 in range(0, w.B, step):
        b1 = min(w.B, b0 + step)
        say("decode oracle, sequences", b0, b1)
        ro, rS_b, rz_b = oracle.causal(*(_steps_as_sequence(x, b0, b1) for x in (sq, sk, sv)),
                                       S0=rS[b0:b1], z0=rz[b0:b1])
        assert row_rel_err(_steps_as_sequence(outs, b0, b1), ro) < 2e-2, (b0, b1)
        assert mat_rel_err(S[b0:b1], rS_b) < 1e-4, (b0, b1)
        assert mat_rel_err(z[b0:b1], rz_b, 1) < 1e-4, (b0, b1)


# ---------------------------------------------------------------- delta rule

@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("D,M", [(32, 32), (32, 64), (64, 32), (64, 64)])
@pytest.mark.parametrize("N", [1, 5, 64, 65, 130])
def test_deltanet_ragged(dtype, D, M, N):
    say("deltanet", dtype, D, M, N)
    q, k, v, beta = synth.qkv_beta(2, 3, N, D, M, dtype=dtype, seed=N + D * M)
    W0 = torch.randn(2, 3, M, D) * 0.1
    o, W = la.deltanet(*gpu(q, k, v, beta), W0=W0.to(DEV), return_state=True)
    ro, rW = oracle.deltanet(q, k, v, beta, W0=W0)
    assert row_rel_err(host(o), ro) < TOL[dtype]
    assert mat_rel_err(host(W), rW) < 1e-4


@pytest.mark.parametrize("D,M", [(32, 64), (64, 32), (64, 64)])
@pytest.mark.parametrize("N", [1025, 1088, 1470, 2113])
def test_deltanet_many_chunks(D, M, N):
    """17 to 34 chunks of 64 tokens with a partial last chunk (1 to 63 tokens),
    from an initial memory, with the final memory written over it."""
    dtype = torch.float32
    say("deltanet many chunks", D, M, N)
    q, k, v, beta = synth.qkv_beta(1, 3, N, D, M, dtype=dtype, seed=N + 7 * D + M)
    W0 = torch.randn(1, 3, M, D, generator=torch.Generator().manual_seed(N)) * 0.1
    qg, kg, vg, bg = gpu(q, k, v, beta)
    Wg = W0.to(DEV)
    o, W = la.deltanet(qg, kg, vg, bg, W0=Wg, return_state=True)
    ro, rW = oracle.deltanet(q, k, v, beta, W0=W0)
    assert row_rel_err(host(o), ro) < TOL[dtype]
    assert mat_rel_err(host(W), rW) < 1e-4
    # the final memory written over the initial one (W_out == W0), through the C ABI
    lib = la._lib.load()
    need = la.deltanet_workspace_bytes(1, 3, N, D, M, dtype)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    o2 = torch.empty_like(o)
    rc = lib.deltanet_fwd(qg.data_ptr(), kg.data_ptr(), vg.data_ptr(), bg.data_ptr(), o2.data_ptr(), 1, 3, N, D, M,
                          0, Wg.data_ptr(), Wg.data_ptr(), ws.data_ptr(), need, torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    assert torch.equal(host(o2), host(o)) and torch.equal(host(Wg), host(W))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("D,M", [(32, 32), (32, 64), (64, 32), (64, 64)])
@pytest.mark.parametrize("N", [1, 5, 64, 65, 130, 1000])
def test_deltanet_sequential_path(monkeypatch, dtype, D, M, N):
    """LINATTN_DELTANET_PATH=sequential runs the token-by-token kernel (one chain
    of wavefront reductions per row of W): outputs and final memory from an
    initial memory, with the final memory written over the initial one."""
    monkeypatch.setenv("LINATTN_DELTANET_PATH", "sequential")
    say("deltanet sequential", dtype, D, M, N)
    q, k, v, beta = synth.qkv_beta(2, 3, N, D, M, dtype=dtype, seed=N + 3 * D * M)
    W0 = torch.randn(2, 3, M, D, generator=torch.Generator().manual_seed(N)) * 0.1
    ro, rW = oracle.deltanet(q, k, v, beta, W0=W0)
    qg, kg, vg, bg = gpu(q, k, v, beta)
    lib = la._lib.load()
    dt = 0 if dtype == torch.float32 else 1
    need = lib.deltanet_workspace_bytes(2, 3, N, D, M, dt)
    assert need == 0  # the token-by-token kernel keeps everything in registers
    Wg = W0.to(DEV)
    o = torch.empty(2, 3, N, M, dtype=dtype, device=DEV)
    rc = lib.deltanet_fwd(qg.data_ptr(), kg.data_ptr(), vg.data_ptr(), bg.data_ptr(), o.data_ptr(), 2, 3, N, D, M,
                          dt, Wg.data_ptr(), Wg.data_ptr(), None, 0, torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    assert row_rel_err(host(o), ro) < TOL[dtype]
    assert mat_rel_err(host(Wg), rW) < 1e-4


def test_deltanet_sequential_path_workload(monkeypatch):
    """The token-by-token kernel on the full delta-rule workload (B=4 H=8 N=4096)."""
    monkeypatch.setenv("LINATTN_DELTANET_PATH", "sequential")
    w = synth.WORKLOADS["deltanet"]
    say("deltanet sequential", w)
    q, k, v, beta = synth.workload_inputs(w)
    o, W = la.deltanet(*gpu(q, k, v, beta), return_state=True)
    ro, rW = oracle.deltanet(q, k, v, beta)
    assert row_rel_err(host(o), ro) < 1e-4
    assert mat_rel_err(host(W), rW) < 1e-4


def test_deltanet_workload():
    w = synth.WORKLOADS["deltanet"]
    say(w)
    q, k, v, beta = synth.workload_inputs(w)
    o, W = la.deltanet(*gpu(q, k, v, beta), return_state=True)
    ro, rW = oracle.deltanet(q, k, v, beta)
    assert row_rel_err(host(o), ro) < 1e-4
    assert mat_rel_err(host(W), rW) < 1e-4


def test_deltanet_exact_recall_and_inplace_memory():
    """One-hot keys at beta = 1 store and overwrite slots exactly; W_out may be W0."""
    D, M, N = 64, 64, 200
    say("deltanet recall")
    g = torch.Generator().manual_seed(4)
    slots = torch.randint(0, D, (N,), generator=g)
    k = torch.full((1, 1, N, D), -200.0)
    k[0, 0, torch.arange(N), slots] = 0.0
    v = torch.randint(-8, 9, (1, 1, N, M), generator=g).float()
    q = k.clone()
    beta = torch.ones(1, 1, N)
    Wg = torch.zeros(1, 1, M, D, device=DEV)
    lib = la._lib.load()
    qg, kg, vg, bg = gpu(q, k, v, beta)
    o = torch.empty(1, 1, N, M, device=DEV)
    need = lib.deltanet_workspace_bytes(1, 1, N, D, M, 0)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=DEV)
    rc = lib.deltanet_fwd(qg.data_ptr(), kg.data_ptr(), vg.data_ptr(), bg.data_ptr(), o.data_ptr(), 1, 1, N, D, M,
                          0, Wg.data_ptr(), Wg.data_ptr(), ws.data_ptr(), need, torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    # reading the slot just written returns exactly the value written
    np.testing.assert_allclose(host(o)[0, 0].numpy(), v[0, 0].numpy(), rtol=0, atol=1e-5)
    W = host(Wg)[0, 0]
    for c in range(D):
        last = [i for i in range(N) if slots[i] == c]
        want = v[0, 0, last[-1]] if last else torch.zeros(M)
        np.testing.assert_allclose(W[:, c].numpy(), want.numpy(), rtol=0, atol=1e-5)


def test_deltanet_empty_sequence_copies_memory():
    say("deltanet empty")
    W0 = torch.randn(2, 2, 32, 32, device=DEV)
    e = torch.empty(2, 2, 0, 32, device=DEV)
    o, W = la.deltanet(e, e, e, torch.empty(2, 2, 0, device=DEV), W0=W0, return_state=True)
    assert torch.equal(host(W), host(W0))


# ------------------------------------------------------- delta-rule decode step

def _oracle_delta_step(q, k, v, beta, W):
    """One oracle step: the sequence oracle on a length-1 sequence."""
    o, W2 = oracle.deltanet(q[:, :, None], k[:, :, None], v[:, :, None], beta[:, :, None], W0=W)
    return o[:, :, 0], W2


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("D,M", [(32, 32), (32, 64), (64, 32), (64, 64)])
def test_deltanet_decode_steps_small(dtype, D, M):
    """Prefill a memory with the sequence kernel, then T single steps (B*H = 15,
    a partial workgroup of wavefronts), each against the oracle."""
    B, H, P, T = 3, 5, 40, 6
    say("deltanet decode", dtype, D, M)
    q, k, v, beta = synth.qkv_beta(B, H, P, D, M, dtype=dtype, seed=D * M + 1)
    sq, sk, sv, sb = synth.decode_steps_beta(B, H, D, M, T, dtype=dtype, seed=D + M + 1)
    W0 = torch.randn(B, H, M, D) * 0.1
    _, W = la.deltanet(*gpu(q, k, v, beta), W0=W0.to(DEV), return_state=True)
    _, rW = oracle.deltanet(q, k, v, beta, W0=W0)
    gq, gk, gv, gb = gpu(sq, sk, sv, sb)
    for t in range(T):
        o = la.deltanet_decode_step(gq[t], gk[t], gv[t], gb[t], W)
        ro, rW = _oracle_delta_step(sq[t], sk[t], sv[t], sb[t], rW)
        assert row_rel_err(host(o), ro) < TOL[dtype], t
        assert mat_rel_err(host(W), rW) < 1e-4, t


def test_deltanet_decode_equals_sequence():
    """N decode steps from W0 give the sequence path's outputs and memory.  The
    decode step is plain fp32; the chunked sequence path forms its products from
    bf16 head + tail operands (about 2^-17 relative per operand, the tail x tail
    term dropped), so the two agree to the bound both are held to against the
    oracle."""
    B, H, N, D, M = 2, 4, 70, 64, 64
    say("deltanet decode vs sequence")
    q, k, v, beta = synth.qkv_beta(B, H, N, D, M, seed=77)
    W0 = (torch.randn(B, H, M, D) * 0.1).to(DEV)
    o_seq, W_seq = la.deltanet(*gpu(q, k, v, beta), W0=W0, return_state=True)
    W = W0.clone()
    gq, gk, gv, gb = gpu(q, k, v, beta)
    outs = [la.deltanet_decode_step(gq[:, :, t].contiguous(), gk[:, :, t].contiguous(), gv[:, :, t].contiguous(),
                                    gb[:, :, t].contiguous(), W) for t in range(N)]
    o_dec = torch.stack(outs, dim=2)
    assert row_rel_err(host(o_dec), host(o_seq).double()) < 1e-4
    assert mat_rel_err(host(W), host(W_seq).double()) < 1e-4


def test_deltanet_decode_workload_all_heads():
    """Full delta-rule decode workload (512-token prefill + 1024 steps on 256 x 16
    memories, the launch sequence the benchmark times): every head at every step
    and every final memory.  The oracle is the rule token by token over the
    steps taken as a sequence, from the oracle's own prefill memory."""
    w = synth.WORKLOADS["deltanet_decode"]
    say(w)
    q, k, v, beta, sq, sk, sv, sb = synth.workload_inputs(w)
    _, W = la.deltanet(*gpu(q, k, v, beta), return_state=True)
    _, rW = oracle.deltanet(q, k, v, beta)
    assert mat_rel_err(host(W), rW) < 1e-4
    gq, gk, gv, gb = gpu(sq, sk, sv, sb)
    outs = torch.empty(w.steps, w.B, w.H, w.M, dtype=w.dtype, device=DEV)
    for t in range(w.steps):
        la.deltanet_decode_step(gq[t], gk[t], gv[t], gb[t], W, out=outs[t])
    outs, W = host(outs), host(W)
    step = 32
    for b0 in range(0, w.B, step):
        b1 = min(w.B, b0 + step)
        say("deltanet decode oracle, sequences", b0, b1)
        bseq = sb[:, b0:b1].permute(1, 2, 0).contiguous()
        ro, rW_b = oracle.deltanet(*(_steps_as_sequence(x, b0, b1) for x in (sq, sk, sv)), bseq, W0=rW[b0:b1])
        assert row_rel_err(_steps_as_sequence(outs, b0, b1), ro) < 2e-2, (b0, b1)
        assert mat_rel_err(W[b0:b1], rW_b) < 1e-4, (b0, b1)


# ------------------------------------------------------------- causal backward

BWD_TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def _zero_rows(shape, name):
    """Rows of a gradient that are identically zero: o_1 = v_1 whatever q_1 is, so
    dq of the first token vanishes, and with a single token dk vanishes too."""
    mask = np.zeros(shape[:-1], dtype=bool)
    if name == "dq" or (name == "dk" and shape[-2] == 1):
        mask[..., 0] = True
    return mask


def _bwd_compare(grads, refs, tol, label=(), dq_floor=None):
    """Row-wise (per b, h, token) relative error of dq, dk and dv.  Rows that are
    identically zero are measured against the largest gradient element.  A row of
    dq is the difference of two terms that can nearly cancel (S_i dO_i and
    z_i (dO_i . o_i), over den_i); with ``dq_floor`` (their size per row) each dq
    row is measured against the larger of itself and those terms, the error any
    float32 evaluation makes (a plain float32 autograd of the definition misses
    1e-4 of the row by itself on such rows)."""
    scale = max(np.abs(r).max() for r in refs)
    for got, ref, name in zip(grads, refs, ("dq", "dk", "dv")):
        floor = dq_floor if name == "dq" else None
        e = grad_rel_err(got, ref, _zero_rows(ref.shape, name), scale, floor)
        assert e < tol, (*label, name, e)


def _bwd_check(q, k, v, dO, dtype):
    grads = [host(t) for t in la.causal_bwd(*gpu(q, k, v, dO))]
    _bwd_compare(grads, oracle.causal_bwd(q, k, v, dO), BWD_TOL[dtype],
                 dq_floor=gradients.dq_term_scale(q, k, v, dO))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("D,M", [(32, 32), (32, 64), (64, 32), (64, 64)])
@pytest.mark.parametrize("N", [1, 63, 64, 65, 300, 2500])
def test_causal_bwd_ragged(dtype, D, M, N):
    """Every size class: a single token, chunk edges, several chunks and blocks."""
    say("causal bwd", dtype, D, M, N)
    q, k, v = synth.qkv(2, 2, N, D, M, dtype=dtype, scale=0.5, seed=N + D + 2 * M)
    dO = synth.qkv(2, 2, N, M, M, dtype=dtype, seed=N + 7)[0]
    _bwd_check(q, k, v, dO, dtype)


def test_causal_bwd_many_blocks():
    """Many blocks per head (the prefix and suffix scans across blocks)."""
    q, k, v = synth.qkv(1, 3, 9000, 64, 64, dtype=torch.float32, scale=0.5, seed=5)
    dO = synth.qkv(1, 3, 9000, 64, 64, seed=6)[0]
    say("causal bwd many blocks")
    _bwd_check(q, k, v, dO, torch.float32)


def test_causal_bwd_long_workload_sampled_head():
    """The long bf16 workload (B=2 H=16 N=32768 D=M=64), every head computed on
    the GPU; two heads checked in full against the oracle."""
    w = synth.WORKLOADS["causal_long"]
    say("causal bwd long", w)
    q, k, v = synth.workload_inputs(w)
    dO = synth.qkv(w.B, w.H, w.N, w.M, w.M, dtype=w.dtype, seed=w.seed + 50)[0]
    grads = [host(t) for t in la.causal_bwd(*gpu(q, k, v, dO))]
    for b, h in ((0, 3), (1, 15)):
        sel = (slice(b, b + 1), slice(h, h + 1))
        _bwd_compare([g[sel] for g in grads], oracle.causal_bwd(q[sel], k[sel], v[sel], dO[sel]),
                     BWD_TOL[w.dtype], (b, h))


# ---------------------------------------------------------------- softmax decode baseline

def _softmax_inputs(B, H, L, Lmax, D, M, dtype, seed):
    q, k, v = synth.decode_steps(B, H, D, M, 1, dtype=dtype, seed=seed)
    Kc, Vc = synth.kv_cache(B, H, Lmax, D, M, dtype=dtype, seed=seed + 1)
    return q[0], k[0], v[0], Kc, Vc


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("D,M", [(32, 32), (32, 64), (64, 32), (64, 64)])
@pytest.mark.parametrize("L", [0, 1, 31, 32, 33, 127, 128, 129, 1000])
def test_softmax_decode_ragged(dtype, D, M, L):
    say("softmax decode", dtype, D, M, L)
    q, k, v, Kc, Vc = _softmax_inputs(2, 3, L, L + 5, D, M, dtype, seed=L * 3 + D + M)
    Kg, Vg = gpu(Kc, Vc)
    o = la.softmax_decode_step(*gpu(q, k, v), Kg, Vg, L)
    ro, rK, rV = oracle.softmax_decode(q, k, v, Kc, Vc, L)
    assert row_rel_err(host(o), ro) < TOL[dtype]
    # row L now holds k and v; every other row is unchanged
    assert torch.equal(host(Kg)[:, :, L], k) and torch.equal(host(Vg)[:, :, L], v)
    keep = [j for j in range(L + 5) if j != L]
    assert torch.equal(host(Kg)[:, :, keep], Kc[:, :, keep]) and torch.equal(host(Vg)[:, :, keep], Vc[:, :, keep])


def test_softmax_decode_steps_append():
    """A prefill cache, then steps that each append and attend: every output
    against the oracle run on the caches it has built itself."""
    B, H, D, M, P, T = 3, 4, 64, 64, 37, 70
    dtype = torch.bfloat16
    Kc, Vc = synth.kv_cache(B, H, P + T, D, M, dtype=dtype, seed=11)
    sq, sk, sv = synth.decode_steps(B, H, D, M, T, dtype=dtype, seed=12)
    Kg, Vg = gpu(Kc, Vc)
    rK, rV = Kc, Vc
    for t in range(T):
        say("softmax decode step", t)
        o = la.softmax_decode_step(*gpu(sq[t], sk[t], sv[t]), Kg, Vg, P + t)
        ro, rK, rV = oracle.softmax_decode(sq[t], sk[t], sv[t], rK, rV, P + t)
        assert row_rel_err(host(o), ro) < 2e-2
    assert torch.equal(host(Kg).double(), torch.from_numpy(rK)) and torch.equal(host(Vg).double(), torch.from_numpy(rV))


def test_softmax_decode_workload_shape():
    """The decode workload's shape: 256 sequences x 16 heads, D = M = 64, bf16, at
    the first and last context lengths of its 512 + 1024 tokens (every head)."""
    w = synth.WORKLOADS["decode"]
    Lmax = w.N + w.steps
    Kc, Vc = synth.kv_cache(w.B, w.H, Lmax, w.D, w.M, dtype=w.dtype, seed=w.seed + 70)
    Kg, Vg = gpu(Kc, Vc)
    sq, sk, sv = synth.decode_steps(w.B, w.H, w.D, w.M, 2, dtype=w.dtype, seed=w.seed + 71)
    for t, L in enumerate([w.N, Lmax - 1]):
        say("softmax decode workload", L)
        o = la.softmax_decode_step(*gpu(sq[t], sk[t], sv[t]), Kg, Vg, L)
        ro, _, _ = oracle.softmax_decode(sq[t], sk[t], sv[t], Kc, Vc, L)
        Kc[:, :, L], Vc[:, :, L] = sk[t], sv[t]
        assert row_rel_err(host(o), ro) < 2e-2
