"""GPU parity of linear attention with the other feature maps (DPFP-nu and the
degree-2 polynomial map) through the C ABI, against the CPU oracle.

Both sides read the same seeded host tensors.  Outputs: row-wise relative
error (max over rows of ||y - r||_inf / ||r||_inf), 1e-4 for float32 inputs and
2e-2 for bfloat16 inputs (float32 arithmetic, one rounding of the output).
States are float32 and held to 1e-4 per matrix.  With DPFP a row can have no
weight at all (no query-key pair shares an active pair of components): both
sides then give 0/0 = NaN, and the NaN positions must agree.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import weight_recurrences_amd as la
from oracle.metrics import mat_rel_err, row_rel_err

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}
STATE_TOL = 1e-4
DEV = "cuda:0"
MAPS = [(la.FMAP_DPFP, 1), (la.FMAP_DPFP, 2), (la.FMAP_DPFP, 3), (la.FMAP_POLY2, 0)]
MAP_IDS = ["dpfp1", "dpfp2", "dpfp3", "poly2"]
ORACLE_MAP = {la.FMAP_DPFP: oracle.DPFP, la.FMAP_POLY2: oracle.POLY2}


def say(*a):
    print("[case]", *a, flush=True)


def gpu(*ts):
    return [None if t is None else t.to(DEV) for t in ts]


def host(t):
    torch.cuda.synchronize()
    return t.detach().to("cpu")


def check_rows(got, ref, tol):
    """NaN rows (0/0 with DPFP) must coincide; the rest within tol."""
    got = got.double().numpy()
    nan_g, nan_r = np.isnan(got).any(axis=-1), np.isnan(ref).any(axis=-1)
    assert np.array_equal(nan_g, nan_r), f"NaN rows differ: {nan_g.sum()} vs {nan_r.sum()}"
    keep = ~nan_r
    if keep.any():
        assert row_rel_err(torch.from_numpy(got[keep]), ref[keep]) < tol


@pytest.mark.parametrize("fm,nu", MAPS, ids=MAP_IDS)
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("D,M", [(32, 32), (32, 64), (64, 32), (64, 64)])
@pytest.mark.parametrize("N", [1, 63, 200, 700])
def test_fmap_causal_ragged(fm, nu, dtype, D, M, N):
    if fm == la.FMAP_POLY2 and D == 64 and N > 200:
        N = 200  # the fp64 oracle at C = 4096 is slow; 200 still spans four chunks
    say("fmap causal", fm, nu, dtype, D, M, N)
    q, k, v = synth.qkv(2, 2, N, D, M, dtype=dtype, seed=N * 13 + D + M + 7 * nu + 100 * fm)
    o, (S, z) = la.fmap(*gpu(q, k, v), fm, nu, return_state=True)
    ro, rS, rz = oracle.fmap_causal(q, k, v, ORACLE_MAP[fm], nu)
    check_rows(host(o), ro, TOL[dtype])
    assert mat_rel_err(host(S), rS) < STATE_TOL
    assert mat_rel_err(host(z), rz, 1) < STATE_TOL


@pytest.mark.parametrize("fm,nu", MAPS, ids=MAP_IDS)
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("N", [1, 100, 513])
def test_fmap_noncausal(fm, nu, dtype, N):
    D, M = (32, 64) if fm == la.FMAP_POLY2 else (64, 64)
    say("fmap noncausal", fm, nu, dtype, N)
    q, k, v = synth.qkv(1, 3, N, D, M, dtype=dtype, seed=N + 5 * nu + 50 * fm)
    o, (S, z) = la.fmap(*gpu(q, k, v), fm, nu, causal=False, return_state=True)
    ro, rS, rz = oracle.fmap_noncausal(q, k, v, ORACLE_MAP[fm], nu)
    check_rows(host(o), ro, TOL[dtype])
    assert mat_rel_err(host(S), rS) < STATE_TOL
    assert mat_rel_err(host(z), rz, 1) < STATE_TOL
    # the last causal row sees every key
    oc = la.fmap(*gpu(q, k, v), fm, nu)
    check_rows(host(oc)[:, :, -1:], ro[:, :, -1:], TOL[dtype])


@pytest.mark.parametrize("fm,nu", MAPS, ids=MAP_IDS)
def test_fmap_state_carry_in_place(fm, nu):
    """A sequence cut in two, the second call starting from the first call's
    state and writing its final state over it (S_out == S0)."""
    B, H, N, D, M, cut = 2, 2, 450, 32, 64, 170
    dtype = torch.float32
    say("fmap carry", fm, nu)
    q, k, v = synth.qkv(B, H, N, D, M, dtype=dtype, seed=77 + nu + 10 * fm)
    ro, rS, rz = oracle.fmap_causal(q, k, v, ORACLE_MAP[fm], nu)
    qg, kg, vg = gpu(q, k, v)
    o1, (S, z) = la.fmap(qg[:, :, :cut].contiguous(), kg[:, :, :cut].contiguous(), vg[:, :, :cut].contiguous(),
                         fm, nu, return_state=True)
    C = la.fmap_dim(fm, nu, D)
    ws = torch.empty(la.fmap_workspace_bytes(B, H, N - cut, D, M, dtype, fm, nu), dtype=torch.uint8, device=DEV)
    o2 = torch.empty(B, H, N - cut, M, device=DEV)
    q2, k2, v2 = (t[:, :, cut:].contiguous() for t in (qg, kg, vg))
    lib = la._lib.load()
    rc = lib.linattn_fmap_fwd(q2.data_ptr(), k2.data_ptr(), v2.data_ptr(), o2.data_ptr(), B, H, N - cut, D, M, 0,
                              fm, nu, 1, S.data_ptr(), z.data_ptr(), S.data_ptr(), z.data_ptr(), ws.data_ptr(),
                              ws.numel(), torch.cuda.current_stream().cuda_stream)
    assert rc == 0 and S.shape == (B, H, C, M)
    check_rows(host(torch.cat([o1, o2], dim=2)), ro, TOL[dtype])
    assert mat_rel_err(host(S), rS) < STATE_TOL
    assert mat_rel_err(host(z), rz, 1) < STATE_TOL


@pytest.mark.parametrize("fm,nu", MAPS, ids=MAP_IDS)
def test_fmap_empty_and_state_only(fm, nu):
    B, H, D, M = 2, 3, 32, 32
    C = la.fmap_dim(fm, nu, D)
    say("fmap empty", fm, nu)
    S0 = torch.randn(B, H, C, M, generator=torch.Generator().manual_seed(3))
    z0 = torch.rand(B, H, C, generator=torch.Generator().manual_seed(4))
    q, k, v = synth.qkv(B, H, 0, D, M, dtype=torch.float32, seed=5)
    S, z = la.fmap(*gpu(q, k, v), fm, nu, state=gpu(S0, z0), output=False)
    assert torch.equal(host(S), S0) and torch.equal(host(z), z0)
    # state only (o = NULL) over a real sequence
    q, k, v = synth.qkv(B, H, 300, D, M, dtype=torch.bfloat16, seed=6)
    S, z = la.fmap(*gpu(q, k, v), fm, nu, state=gpu(S0, z0), output=False)
    _, rS, rz = oracle.fmap_causal(q, k, v, ORACLE_MAP[fm], nu, S0=S0, z0=z0, want_output=False)
    assert mat_rel_err(host(S), rS) < STATE_TOL and mat_rel_err(host(z), rz, 1) < STATE_TOL


@pytest.mark.parametrize("fm,nu", [(la.FMAP_DPFP, 1), (la.FMAP_DPFP, 3), (la.FMAP_POLY2, 0)],
                         ids=["dpfp1", "dpfp3", "poly2"])
def test_fmap_workload_shape(fm, nu):
    """The feature-map workload's shape, B=4 H=8 N=4096 D=M=64 float32, in the
    launch configuration the benchmark times, every row of every head against the
    oracle (the polynomial map's oracle takes about half a minute on 8 threads)."""
    w = synth.WORKLOADS["fmap"]
    say("fmap workload", fm, nu)
    q, k, v = synth.qkv(w.B, w.H, w.N, w.D, w.M, dtype=w.dtype, seed=w.seed)
    o = host(la.fmap(*gpu(q, k, v), fm, nu))
    ro, _, _ = oracle.fmap_causal(q, k, v, ORACLE_MAP[fm], nu)
    check_rows(o, ro, TOL[w.dtype])
