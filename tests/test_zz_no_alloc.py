"""The allocation-free non-causal entry point (linattn_noncausal_fwd_noalloc)
against the entry point it varies (linattn_noncausal_fwd), through the C ABI.

Two calls in a row on the same GPU, the second with a smaller input, so the
second runs on scratch that still holds the first call's partial states; both
must equal the workspace entry point's output bit for bit (same kernels, same
partition) and the oracle within the dtype's tolerance.  A problem larger than
the static scratch is refused before anything is enqueued.
"""
import pytest
import torch

import oracle
import synth
import weight_recurrences_amd as la
from oracle.metrics import row_rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}
LIMIT = 32 << 20


def _dt(dtype):
    return 0 if dtype == torch.float32 else 1


def _with_workspace(lib, q, k, v, dtype):
    B, H, N, D = q.shape
    M = v.shape[-1]
    need = lib.linattn_noncausal_workspace_bytes(B, H, N, D, M, _dt(dtype))
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=DEV)
    o = torch.empty(B, H, N, M, dtype=dtype, device=DEV)
    rc = lib.linattn_noncausal_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), B, H, N, D, M, _dt(dtype),
                                   ws.data_ptr(), need, torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    return o


def _noalloc(lib, q, k, v, dtype):
    B, H, N, D = q.shape
    M = v.shape[-1]
    o = torch.empty(B, H, N, M, dtype=dtype, device=DEV)
    rc = lib.linattn_noncausal_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), B, H, N, D, M,
                                           _dt(dtype), torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    return o


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_noalloc_matches_workspace_entry_point(dtype):
    lib = la._lib.load()
    # the long workload's shape, then a smaller ragged one on the same scratch
    shapes = [(2, 16, 32768, 64, 64), (1, 3, 1000, 32, 64)] if dtype == torch.bfloat16 else \
             [(4, 8, 4096, 64, 64), (1, 3, 1000, 32, 64)]
    for i, (B, H, N, D, M) in enumerate(shapes):
        print("[case] noalloc", dtype, (B, H, N, D, M), flush=True)
        assert lib.linattn_noncausal_workspace_bytes(B, H, N, D, M, _dt(dtype)) <= LIMIT
        q, k, v = synth.qkv(B, H, N, D, M, dtype=dtype, scale=0.5, seed=300 + i)
        qg, kg, vg = (t.to(DEV) for t in (q, k, v))
        got = _noalloc(lib, qg, kg, vg, dtype)
        want = _with_workspace(lib, qg, kg, vg, dtype)
        torch.cuda.synchronize()
        assert torch.equal(got.cpu().view(torch.int16 if dtype == torch.bfloat16 else torch.int32),
                           want.cpu().view(torch.int16 if dtype == torch.bfloat16 else torch.int32))
        if N <= 4096:
            ro, _, _ = oracle.noncausal(q, k, v)
            assert row_rel_err(got.cpu(), ro) < TOL[dtype]
        la.noncausal_noalloc(qg, kg, vg, out=got)   # the Python binding reaches the same entry point
        torch.cuda.synchronize()
        assert torch.equal(got, want)


def test_noalloc_refuses_problems_beyond_the_scratch():
    lib = la._lib.load()
    B, H, N, D, M = 64, 64, 1, 64, 64
    assert lib.linattn_noncausal_workspace_bytes(B, H, N, D, M, 1) > LIMIT
    q = torch.zeros(B, H, N, D, dtype=torch.bfloat16, device=DEV)
    k, v = torch.zeros_like(q), torch.zeros(B, H, N, M, dtype=torch.bfloat16, device=DEV)
    o = torch.full((B, H, N, M), 7.0, dtype=torch.bfloat16, device=DEV)
    rc = lib.linattn_noncausal_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), B, H, N, D, M, 1,
                                           torch.cuda.current_stream().cuda_stream)
    assert rc == 7  # LINATTN_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((o == 7.0).all())  # nothing was enqueued
