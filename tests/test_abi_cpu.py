"""C-ABI contract tests that need no GPU.

The library must load on a machine without a GPU, export every function that
include/linattn.h declares, and reject invalid arguments with the documented
status code before it touches the HIP runtime.  The pointers used here are
fake addresses; every case below is built to fail validation, so nothing is
ever launched.  The tests skip where a GPU is visible, so that a validation
bug could never turn a fake address into a kernel argument there.
"""
import ctypes

import pytest
import torch

from weight_recurrences_amd import _lib

OK, NULL, SHAPE, DTYPE, UNSUP, ALIGN, ALIAS, WS = 0, 1, 2, 3, 4, 5, 6, 7

gpu_visible = torch.cuda.device_count() > 0
no_gpu = pytest.mark.skipif(gpu_visible, reason="fake-pointer validation runs only where no GPU is visible")

A = 1 << 32  # fake, 16-byte aligned, far-apart base addresses
Q, K, V, O, S0, Z0, SO, ZO, WSP, BETA = (A * (i + 1) for i in range(10))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_exports_every_declared_function(lib):
    names = _lib.header_functions()
    assert set(names) == set(_lib.SIGNATURES), names
    for name in names:
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_version_and_status_strings(lib):
    assert lib.linattn_abi_version() == 4
    for code, name in _lib.STATUS.items():
        assert lib.linattn_status_str(code).decode() == name
    assert lib.linattn_status_str(99).decode() == "LINATTN_ERR_UNKNOWN"


def _single_pass_ws(BH, N, D, M, tblk):
    """Workspace of the single-pass causal kernels: one 8-byte flag per block,
    two published states per block (the register image of S, then z, in floats,
    rounded up to 256 bytes), and room for a private copy of the initial state."""
    up = lambda x: (x + 255) // 256 * 256
    nblk = (N + tblk - 1) // tblk
    tmw = (M // 16) // (4 // (D // 16))
    slot = up((4 * tmw * 4 * 64 + D) * 4)
    return up(BH * nblk * 8) + 2 * BH * nblk * slot + up(BH * (D * M + D) * 4)


def test_workspace_sizes(lib):
    # long bf16 workload, single-pass kernel: 32 heads x 128 blocks of 256 tokens; one
    # 8-byte flag per block, two published states of (64*64 + 64) floats per block,
    # and room for a private copy of the initial state
    flags = 32 * 128 * 8
    slot = (64 * 64 + 64) * 4
    init = 32 * (64 * 64 + 64) * 4
    assert lib.linattn_causal_workspace_bytes(2, 16, 32768, 64, 64, 1) == flags + 2 * 32 * 128 * slot + init
    assert lib.linattn_causal_workspace_bytes(2, 16, 32768, 64, 64, 1) == _single_pass_ws(32, 32768, 64, 64, 256)
    # float32 causal, single-pass kernel with blocks of 256 tokens
    assert lib.linattn_causal_workspace_bytes(2, 16, 32768, 64, 64, 0) == _single_pass_ws(32, 32768, 64, 64, 256)
    assert lib.linattn_causal_workspace_bytes(1, 1, 256, 32, 32, 0) == _single_pass_ws(1, 256, 32, 32, 256)
    assert lib.linattn_causal_workspace_bytes(3, 1, 100, 32, 64, 0) == _single_pass_ws(3, 100, 32, 64, 256)
    assert lib.linattn_noncausal_workspace_bytes(1, 1, 256, 32, 32, 0) == 2 * (32 * 32 + 32) * 4
    # delta rule, per chunk of 64 tokens: kh as bf16 head and tail (64 x D x 4 bytes) and
    # T as bf16 head and tail in six 64-lane operand blocks of 32 bytes per lane
    rec64, rec32 = 64 * 64 * 4 + 6 * 64 * 32, 64 * 32 * 4 + 6 * 64 * 32
    assert lib.deltanet_workspace_bytes(4, 8, 4096, 64, 64, 0) == 32 * 64 * rec64
    assert lib.deltanet_workspace_bytes(1, 2, 1024, 64, 64, 0) == 2 * 16 * rec64
    assert lib.deltanet_workspace_bytes(1, 1, 65, 32, 64, 1) == 2 * rec32
    assert lib.deltanet_workspace_bytes(4, 8, 0, 64, 64, 0) == 0
    for bad in [(1, 1, 256, 48, 32, 0), (1, 1, 256, 32, 32, 5), (-1, 1, 4, 32, 32, 0)]:
        assert lib.linattn_causal_workspace_bytes(*bad) == 0
        assert lib.linattn_noncausal_workspace_bytes(*bad) == 0
        assert lib.deltanet_workspace_bytes(*bad) == 0


def causal(lib, q=Q, k=K, v=V, o=O, B=1, H=2, N=4096, D=64, M=64, dt=1, s0=None, z0=None, so=None, zo=None,
           ws=WSP, wsb=1 << 30):
    return lib.linattn_causal_fwd(q, k, v, o, B, H, N, D, M, dt, s0, z0, so, zo, ws, wsb, None)


@no_gpu
def test_causal_validation(lib):
    assert causal(lib, dt=2) == DTYPE
    assert causal(lib, D=48) == UNSUP
    assert causal(lib, M=128) == UNSUP
    assert causal(lib, D=16) == UNSUP
    assert causal(lib, B=-1) == SHAPE
    assert causal(lib, N=-5) == SHAPE
    assert causal(lib, D=0) == SHAPE
    assert causal(lib, B=1 << 16, H=1 << 16) == SHAPE
    assert causal(lib, q=None) == NULL
    assert causal(lib, s0=S0) == NULL           # z0 missing
    assert causal(lib, so=SO) == NULL           # z_out missing
    assert causal(lib, q=Q + 8) == ALIGN
    assert causal(lib, s0=S0 + 4, z0=Z0) == ALIGN
    assert causal(lib, ws=None) == WS
    need = lib.linattn_causal_workspace_bytes(1, 2, 4096, 64, 64, 1)
    assert need > 0 and causal(lib, wsb=need - 1) == WS
    assert causal(lib, o=Q) == ALIAS            # output on top of q
    assert causal(lib, o=V + 4096) == ALIAS     # partial overlap with v
    assert causal(lib, o=WSP) == ALIAS          # output inside the workspace
    assert causal(lib, s0=S0, z0=Z0, so=S0 + 16, zo=ZO) == ALIAS  # partial state overlap
    assert causal(lib, so=K, zo=ZO) == ALIAS    # state output over an input
    assert causal(lib, ws=K) == ALIAS           # workspace over an input


@no_gpu
def test_empty_problems_are_no_ops(lib):
    # nothing to compute and no state to write: OK without launching anything
    assert causal(lib, B=0) == OK
    assert causal(lib, q=None, k=None, v=None, o=None, N=0, ws=None, wsb=0) == OK
    assert lib.linattn_noncausal_fwd(None, None, None, None, 3, 2, 0, 64, 64, 1, None, 0, None) == OK
    assert lib.linattn_decode_step(None, None, None, None, None, None, 0, 16, 64, 64, 1, None) == OK
    assert lib.deltanet_fwd(None, None, None, None, None, 0, 8, 100, 64, 64, 0, None, None, None, 0, None) == OK
    assert lib.deltanet_fwd(None, None, None, None, None, 2, 8, 0, 64, 64, 0, None, None, None, 0, None) == OK
    assert lib.deltanet_decode_step(None, None, None, None, None, None, 0, 16, 64, 64, 1, None) == OK


@no_gpu
def test_noncausal_validation(lib):
    f = lib.linattn_noncausal_fwd
    need = lib.linattn_noncausal_workspace_bytes(2, 16, 32768, 64, 64, 1)
    args = [Q, K, V, O, 2, 16, 32768, 64, 64, 1, WSP, need, None]
    bad = list(args); bad[3] = None
    assert f(*bad) == NULL
    bad = list(args); bad[9] = 7
    assert f(*bad) == DTYPE
    bad = list(args); bad[10] = None
    assert f(*bad) == WS
    bad = list(args); bad[11] = need - 4
    assert f(*bad) == WS
    bad = list(args); bad[3] = K
    assert f(*bad) == ALIAS
    bad = list(args); bad[0] = Q + 2
    assert f(*bad) == ALIGN


@no_gpu
def test_noncausal_noalloc_validation(lib):
    """The allocation-free variant validates like linattn_noncausal_fwd and refuses,
    before any HIP call, a problem whose workspace exceeds the static scratch."""
    f = lib.linattn_noncausal_fwd_noalloc
    limit = 32 << 20
    assert lib.linattn_noncausal_workspace_bytes(2, 16, 32768, 64, 64, 1) <= limit
    args = [Q, K, V, O, 2, 16, 32768, 64, 64, 1, None]
    bad = list(args); bad[3] = None
    assert f(*bad) == NULL
    bad = list(args); bad[9] = 7
    assert f(*bad) == DTYPE
    bad = list(args); bad[7] = 48
    assert f(*bad) == UNSUP
    bad = list(args); bad[3] = K
    assert f(*bad) == ALIAS
    bad = list(args); bad[0] = Q + 2
    assert f(*bad) == ALIGN
    assert lib.linattn_noncausal_workspace_bytes(64, 64, 4096, 64, 64, 1) > limit
    big = list(args); big[4], big[5], big[6] = 64, 64, 4096
    assert f(*big) == WS
    assert f(None, None, None, None, 2, 16, 0, 64, 64, 1, None) == OK


@no_gpu
def test_decode_validation(lib):
    f = lib.linattn_decode_step
    args = [Q, K, V, O, S0, Z0, 256, 16, 64, 64, 1, None]
    bad = list(args); bad[4] = None
    assert f(*bad) == NULL
    bad = list(args); bad[3] = S0 + 64
    assert f(*bad) == ALIAS
    bad = list(args); bad[5] = S0 + 1024
    assert f(*bad) == ALIAS        # z inside S
    bad = list(args); bad[8] = 128
    assert f(*bad) == UNSUP
    bad = list(args); bad[1] = K + 12
    assert f(*bad) == ALIGN


@no_gpu
def test_deltanet_validation(lib):
    f = lib.deltanet_fwd
    need = lib.deltanet_workspace_bytes(4, 8, 4096, 64, 64, 0)
    args = [Q, K, V, BETA, O, 4, 8, 4096, 64, 64, 0, S0, SO, WSP, need, None]
    bad = list(args); bad[3] = None
    assert f(*bad) == NULL
    bad = list(args); bad[12] = S0 + 256
    assert f(*bad) == ALIAS        # partial overlap of W_out and W0
    bad = list(args); bad[4] = BETA
    assert f(*bad) == ALIAS
    bad = list(args); bad[12] = Q
    assert f(*bad) == ALIAS        # memory output over q
    bad = list(args); bad[8] = 33
    assert f(*bad) == UNSUP
    bad = list(args); bad[10] = -1
    assert f(*bad) == DTYPE
    bad = list(args); bad[13] = None
    assert f(*bad) == WS
    bad = list(args); bad[14] = need - 16
    assert f(*bad) == WS
    bad = list(args); bad[13] = K
    assert f(*bad) == ALIAS        # workspace over k
    bad = list(args); bad[4] = WSP + 64
    assert f(*bad) == ALIAS        # output inside the workspace


@no_gpu
def test_causal_bwd_validation(lib):
    f = lib.linattn_causal_bwd
    need = lib.linattn_causal_bwd_workspace_bytes(2, 16, 32768, 64, 64, 1)
    assert need > 0
    DQ, DK, DV, DO = SO, ZO, Z0, S0
    args = [Q, K, V, DO, DQ, DK, DV, 2, 16, 32768, 64, 64, 1, WSP, need, None]
    bad = list(args); bad[3] = None
    assert f(*bad) == NULL
    bad = list(args); bad[13] = None
    assert f(*bad) == WS
    bad = list(args); bad[14] = need - 16
    assert f(*bad) == WS
    bad = list(args); bad[4] = Q
    assert f(*bad) == ALIAS        # dq over q
    bad = list(args); bad[5] = DQ + 64
    assert f(*bad) == ALIAS        # dk overlapping dq
    bad = list(args); bad[13] = V
    assert f(*bad) == ALIAS        # workspace over v
    bad = list(args); bad[10] = 48
    assert f(*bad) == UNSUP
    bad = list(args); bad[6] = DV + 8
    assert f(*bad) == ALIGN
    assert f(None, None, None, None, None, None, None, 2, 16, 0, 64, 64, 1, None, 0, None) == OK


@no_gpu
def test_deltanet_decode_validation(lib):
    f = lib.deltanet_decode_step
    args = [Q, K, V, BETA, O, S0, 256, 16, 64, 64, 1, None]
    bad = list(args); bad[5] = None
    assert f(*bad) == NULL
    bad = list(args); bad[3] = None
    assert f(*bad) == NULL
    bad = list(args); bad[4] = S0 + 64
    assert f(*bad) == ALIAS        # o inside W
    bad = list(args); bad[5] = BETA
    assert f(*bad) == ALIAS        # W over beta
    bad = list(args); bad[9] = 48
    assert f(*bad) == UNSUP
    bad = list(args); bad[10] = 2
    assert f(*bad) == DTYPE
    bad = list(args); bad[2] = V + 4
    assert f(*bad) == ALIGN


def test_binding_refuses_cpu_tensors():
    import weight_recurrences_amd as la
    x = torch.zeros(1, 1, 4, 32)
    with pytest.raises(ValueError, match="GPU"):
        la.causal(x, x, x)


@no_gpu
def test_softmax_decode_validation(lib):
    f = lib.softmax_decode_step
    # q, k, v, o small; caches far apart (fake device addresses, never dereferenced)
    args = [Q, K, V, O, S0, SO, 256, 16, 700, 1536, 64, 64, 1, None]
    bad = list(args); bad[4] = None
    assert f(*bad) == NULL
    bad = list(args); bad[8] = 1536        # L must be below Lmax
    assert f(*bad) == SHAPE
    bad = list(args); bad[8] = -1
    assert f(*bad) == SHAPE
    bad = list(args); bad[12] = 5
    assert f(*bad) == DTYPE
    bad = list(args); bad[10] = 48
    assert f(*bad) == UNSUP
    bad = list(args); bad[3] = S0 + 64     # o inside the key cache
    assert f(*bad) == ALIAS
    bad = list(args); bad[5] = S0 + 4096   # value cache overlaps the key cache
    assert f(*bad) == ALIAS
    bad = list(args); bad[0] = Q + 8
    assert f(*bad) == ALIGN
    assert f(None, None, None, None, None, None, 0, 16, 0, 1, 64, 64, 1, None) == OK


def fmapc(lib, q=Q, k=K, v=V, o=O, B=1, H=2, N=4096, D=64, M=64, dt=1, fm=1, nu=1, causal=1, s0=None, z0=None,
          so=None, zo=None, ws=WSP, wsb=1 << 34):
    return lib.linattn_fmap_fwd(q, k, v, o, B, H, N, D, M, dt, fm, nu, causal, s0, z0, so, zo, ws, wsb, None)


def test_fmap_dims(lib):
    assert lib.linattn_fmap_dim(1, 1, 64) == 128 and lib.linattn_fmap_dim(1, 3, 32) == 192
    assert lib.linattn_fmap_dim(2, 0, 64) == 4096 and lib.linattn_fmap_dim(2, 0, 32) == 1024
    for fm, nu, D in ((1, 0, 64), (1, 4, 64), (2, 1, 64), (3, 1, 64), (0, 0, 64), (1, 1, 48)):
        assert lib.linattn_fmap_dim(fm, nu, D) == 0
    # workspace: block records plus the totals; 0 for unsupported maps
    assert lib.linattn_fmap_workspace_bytes(1, 2, 4096, 64, 64, 1, 1, 1) > 0
    assert lib.linattn_fmap_workspace_bytes(1, 2, 4096, 64, 64, 1, 1, 4) == 0
    assert lib.linattn_fmap_workspace_bytes(1, 2, 4096, 64, 48, 1, 2, 0) == 0


@no_gpu
def test_fmap_validation(lib):
    assert fmapc(lib, fm=3) == UNSUP
    assert fmapc(lib, nu=0) == UNSUP
    assert fmapc(lib, fm=2, nu=1) == UNSUP
    assert fmapc(lib, causal=0, s0=S0, z0=Z0) == UNSUP  # no initial state in the non-causal form
    assert fmapc(lib, dt=2) == DTYPE
    assert fmapc(lib, D=48) == UNSUP
    assert fmapc(lib, N=-1) == SHAPE
    assert fmapc(lib, k=None) == NULL
    assert fmapc(lib, s0=S0) == NULL
    assert fmapc(lib, q=Q + 8) == ALIGN
    assert fmapc(lib, ws=None) == WS
    need = lib.linattn_fmap_workspace_bytes(1, 2, 4096, 64, 64, 1, 1, 1)
    assert fmapc(lib, wsb=need - 1) == WS
    assert fmapc(lib, o=K + 64) == ALIAS
    assert fmapc(lib, so=V, zo=ZO) == ALIAS
    assert fmapc(lib, s0=S0, z0=Z0, so=S0 + 16, zo=ZO) == ALIAS
    assert fmapc(lib, ws=Q) == ALIAS
    # nothing to compute
    assert fmapc(lib, B=0) == OK
    assert fmapc(lib, q=None, k=None, v=None, o=None, N=0, ws=None, wsb=0) == OK
