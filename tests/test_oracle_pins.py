"""Pins of the CPU oracle against what the pages and the mathematics fix.

Nothing here compares the oracle with a retyped copy of itself.  Each test is
one of: a hand-derived fixture (tests/golden), the pure-Python brute force of
eq.(3)/(8) (a different computation from the recurrent form), a closed form
of a special case, an invariant of the method, a library routine the special
case reduces to (torch's elu, numpy matmul), or an identity between two
different forms the pages give.

Sources: "Transformers are RNNs" (Katharopoulos et al., 2020), translated page
"線性變換器", §3.2-§3.4; news summary of "Linear Transformers Are Secretly Fast
Weight Programmers" (Schlag et al., 2021), capacity / update-rule /
normalisation paragraphs.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import brute
from oracle.metrics import row_rel_err, mat_rel_err

HERE = os.path.dirname(os.path.abspath(__file__))
GOLD = json.load(open(os.path.join(HERE, "golden", "handworked.json")))


def rnd(shape, seed, scale=1.0):
    g = np.random.default_rng(seed)
    return g.standard_normal(shape) * scale


def phi_lib(x):
    """elu(x) + 1 through torch's own elu (an independent implementation)."""
    t = torch.as_tensor(np.asarray(x, dtype=np.float64))
    return (torch.nn.functional.elu(t, alpha=1.0) + 1.0).numpy()


# ---------------------------------------------------------------- phi, eq.(7)

def test_phi_closed_forms():
    assert oracle.phi(0.0) == 1.0
    for x in [1e-300, 1e-12, 0.25, 1.0, 3.5, 1e6]:
        assert oracle.phi(x) == 1.0 + x  # x + 1 exactly on the positive branch
    xs = np.concatenate([-np.logspace(-12, 2.8, 200), np.linspace(-5, 5, 401)])
    got = np.array([oracle.phi(x) for x in xs])
    # torch evaluates (exp(x) - 1) + 1, exact only to an absolute ulp of 1
    np.testing.assert_allclose(got, phi_lib(xs), rtol=1e-14, atol=2.3e-16)
    # on the negative branch phi is exp(x) to full relative accuracy
    neg = xs[xs <= 0]
    np.testing.assert_allclose(got[xs <= 0], [math.exp(x) for x in neg], rtol=1e-15, atol=0)


def test_phi_positive_and_continuous():
    xs = np.linspace(-700, 700, 14001)
    got = np.array([oracle.phi(x) for x in xs])
    assert np.all(got > 0)
    assert abs(oracle.phi(-1e-13) - 1.0) < 1e-12 and abs(oracle.phi(1e-13) - 1.0) < 1e-12
    # very negative inputs keep relative accuracy: phi(-200) = exp(-200)
    assert oracle.phi(-200.0) == pytest.approx(math.exp(-200.0), rel=1e-15)


# ------------------------------------------------------- golden hand-worked

def _t4(x):
    a = np.asarray(x, dtype=np.float64)
    return a[None, None]


@pytest.mark.parametrize("case", GOLD["causal"], ids=lambda c: c["name"])
def test_golden_causal(case):
    q, k, v = _t4(case["q"]), _t4(case["k"]), _t4(case["v"])
    o, _, _ = oracle.causal(q, k, v)
    np.testing.assert_allclose(o[0, 0], np.asarray(case["o"]), rtol=1e-14, atol=1e-14)
    oe = oracle.causal_explicit(q, k, v)
    np.testing.assert_allclose(oe[0, 0], np.asarray(case["o"]), rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("case", GOLD["deltanet"], ids=lambda c: c["name"])
def test_golden_deltanet(case):
    q, k, v = _t4(case["q"]), _t4(case["k"]), _t4(case["v"])
    beta = np.asarray(case["beta"], dtype=np.float64)[None, None]
    o, _ = oracle.deltanet(q, k, v, beta)
    np.testing.assert_allclose(o[0, 0], np.asarray(case["o"]), rtol=1e-14, atol=1e-14)


# ------------------------------------------------- causal: brute force eq.(8)

SHAPES = [(1, 1), (4, 3), (3, 5), (8, 8), (32, 16)]


@pytest.mark.parametrize("D,M", SHAPES)
def test_causal_forms_match_bruteforce(D, M):
    N = 17
    q = rnd((1, 2, N, D), 1 + D)
    k = rnd((1, 2, N, D), 2 + D)
    v = rnd((1, 2, N, M), 3 + D)
    o_rec, _, _ = oracle.causal(q, k, v)
    o_exp = oracle.causal_explicit(q, k, v)
    for h in range(2):
        ref = np.array(brute.attention(q[0, h].tolist(), k[0, h].tolist(), v[0, h].tolist(), causal=True))
        assert row_rel_err(o_rec[0, h], ref) < 1e-12
        assert row_rel_err(o_exp[0, h], ref) < 1e-12


def test_recurrent_equals_explicit_small_workload():
    """eq.(12) == eq.(9) on every row of the smallest workload's shape."""
    q = rnd((1, 1, 256, 32), 11)
    k = rnd((1, 1, 256, 32), 12)
    v = rnd((1, 1, 256, 32), 13)
    o_rec, _, _ = oracle.causal(q, k, v)
    o_exp = oracle.causal_explicit(q, k, v)
    assert row_rel_err(o_rec, o_exp) < 1e-12


def test_state_is_sum_of_outer_products():
    """eq.(10)-(11) at i = N: S = phi(K)^T V, z = sum_j phi(k_j) (numpy matmul)."""
    q, k, v = rnd((2, 3, 40, 6), 1), rnd((2, 3, 40, 6), 2), rnd((2, 3, 40, 5), 3)
    _, S, z = oracle.causal(q, k, v)
    pk = phi_lib(k)
    S_ref = np.einsum("bhnd,bhnm->bhdm", pk, v)
    np.testing.assert_allclose(S, S_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(z, pk.sum(axis=2), rtol=1e-12, atol=1e-12)


# ------------------------------------------------- causal: closed forms

def test_constant_keys_give_prefix_mean():
    N, D, M = 50, 8, 5
    q = rnd((1, 1, N, D), 21)
    k = np.broadcast_to(rnd((1, 1, 1, D), 22), (1, 1, N, D)).copy()
    v = rnd((1, 1, N, M), 23)
    o, _, _ = oracle.causal(q, k, v)
    ref = np.cumsum(v[0, 0], axis=0) / np.arange(1, N + 1)[:, None]
    assert row_rel_err(o[0, 0], ref) < 1e-12


def test_D1_weighted_prefix_mean_independent_of_q():
    N, M = 60, 4
    k = rnd((1, 1, N, 1), 31)
    v = rnd((1, 1, N, M), 32)
    w = phi_lib(k[0, 0, :, 0])
    ref = np.cumsum(w[:, None] * v[0, 0], axis=0) / np.cumsum(w)[:, None]
    for seed in (33, 34):
        q = rnd((1, 1, N, 1), seed, 3.0)
        o, _, _ = oracle.causal(q, k, v)
        assert row_rel_err(o[0, 0], ref) < 1e-12


def test_constant_query_components_cancel():
    """If every component of q_i is equal, phi(q_i) is a multiple of the ones
    vector and the weights become s_j = sum_d phi(k_j)_d (even for q = -100)."""
    N, D, M = 40, 6, 3
    k = rnd((1, 1, N, D), 41)
    v = rnd((1, 1, N, M), 42)
    s = phi_lib(k[0, 0]).sum(axis=1)
    ref = np.cumsum(s[:, None] * v[0, 0], axis=0) / np.cumsum(s)[:, None]
    for c in (-100.0, 0.0, 2.5):
        q = np.full((1, 1, N, D), c)
        o, _, _ = oracle.causal(q, k, v)
        assert np.all(np.isfinite(o))
        assert row_rel_err(o[0, 0], ref) < 1e-12


def test_one_hot_keys_exact_slot_means():
    N, D, M = 64, 8, 4
    g = np.random.default_rng(51)
    slots = g.integers(0, D, size=N)
    c = int(slots[0])
    k = np.full((1, 1, N, D), -200.0)
    k[0, 0, np.arange(N), slots] = 0.0
    q = np.full((1, 1, N, D), -200.0)
    q[..., c] = 0.0
    v = g.integers(-8, 9, size=(1, 1, N, M)).astype(np.float64)
    o, _, _ = oracle.causal(q, k, v)
    for i in range(N):
        sel = [j for j in range(i + 1) if slots[j] == c]
        ref = v[0, 0, sel].mean(axis=0)
        np.testing.assert_allclose(o[0, 0, i], ref, rtol=1e-13, atol=1e-13)


def test_first_row_is_first_value():
    q, k, v = rnd((2, 2, 9, 4), 61), rnd((2, 2, 9, 4), 62), rnd((2, 2, 9, 7), 63)
    o, _, _ = oracle.causal(q, k, v)
    np.testing.assert_allclose(o[:, :, 0], v[:, :, 0], rtol=1e-14, atol=1e-15)
    o1, _, _ = oracle.causal(q[:, :, :1], k[:, :, :1], v[:, :, :1])
    np.testing.assert_allclose(o1[:, :, 0], v[:, :, 0], rtol=1e-14, atol=1e-15)


def test_convex_combination_bounds_and_affine_equivariance():
    N, D, M = 80, 5, 6
    q, k, v = rnd((1, 2, N, D), 71, 2.0), rnd((1, 2, N, D), 72, 2.0), rnd((1, 2, N, M), 73)
    o, _, _ = oracle.causal(q, k, v)
    lo = np.minimum.accumulate(v, axis=2)
    hi = np.maximum.accumulate(v, axis=2)
    assert np.all(o >= lo - 1e-12) and np.all(o <= hi + 1e-12)
    a = -1.75
    b = rnd((M,), 74)
    o2, _, _ = oracle.causal(q, k, a * v + b)
    assert row_rel_err(o2, a * o + b) < 1e-11


def test_state_carry_split_sequence():
    N, D, M = 70, 6, 4
    q, k, v = rnd((1, 2, N, D), 81), rnd((1, 2, N, D), 82), rnd((1, 2, N, M), 83)
    o, S, z = oracle.causal(q, k, v)
    for P in (1, 23, 69):
        _, S1, z1 = oracle.causal(q[:, :, :P], k[:, :, :P], v[:, :, :P], want_output=False)
        o2, S2, z2 = oracle.causal(q[:, :, P:], k[:, :, P:], v[:, :, P:], S0=S1, z0=z1)
        assert row_rel_err(o2, o[:, :, P:]) < 1e-12
        assert mat_rel_err(S2, S) < 1e-12 and mat_rel_err(z2, z, 1) < 1e-12


def test_decode_steps_equal_causal_rows():
    """The RNN form eq.(16)-(20) reproduces eq.(12) token by token."""
    P, T, D, M = 12, 9, 5, 3
    q, k, v = rnd((2, 2, P + T, D), 91), rnd((2, 2, P + T, D), 92), rnd((2, 2, P + T, M), 93)
    o_ref, S_ref, z_ref = oracle.causal(q, k, v)
    _, S, z = oracle.causal(q[:, :, :P], k[:, :, :P], v[:, :, :P], want_output=False)
    for t in range(T):
        ot, S, z = oracle.decode_step(q[:, :, P + t], k[:, :, P + t], v[:, :, P + t], S, z)
        assert row_rel_err(ot, o_ref[:, :, P + t]) < 1e-12
    assert mat_rel_err(S, S_ref) < 1e-12 and mat_rel_err(z, z_ref, 1) < 1e-12


def test_decode_from_zero_state_returns_value():
    q, k, v = rnd((3, 2, 4), 94), rnd((3, 2, 4), 95), rnd((3, 2, 6), 96)
    o, S, z = oracle.decode_step(q, k, v, np.zeros((3, 2, 4, 6)), np.zeros((3, 2, 4)))
    np.testing.assert_allclose(o, v, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(z, phi_lib(k), rtol=1e-14)


# ------------------------------------------------- non-causal, eq.(4)-(6)

@pytest.mark.parametrize("D,M", [(1, 1), (4, 3), (8, 8)])
def test_noncausal_forms_match_bruteforce(D, M):
    N = 15
    q, k, v = rnd((1, 1, N, D), 101 + D), rnd((1, 1, N, D), 102 + D), rnd((1, 1, N, M), 103 + D)
    o, S, z = oracle.noncausal(q, k, v)
    oe = oracle.noncausal_explicit(q, k, v)
    ref = np.array(brute.attention(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(), causal=False))
    assert row_rel_err(o[0, 0], ref) < 1e-12
    assert row_rel_err(oe[0, 0], ref) < 1e-12


def test_noncausal_permutation_properties_and_last_row():
    N, D, M = 45, 7, 5
    q, k, v = rnd((1, 2, N, D), 111), rnd((1, 2, N, D), 112), rnd((1, 2, N, M), 113)
    o, S, z = oracle.noncausal(q, k, v)
    perm = np.random.default_rng(114).permutation(N)
    o_kv, _, _ = oracle.noncausal(q, k[:, :, perm], v[:, :, perm])
    assert row_rel_err(o_kv, o) < 1e-12          # joint permutation of (k, v) pairs
    o_q, _, _ = oracle.noncausal(q[:, :, perm], k, v)
    assert row_rel_err(o_q, o[:, :, perm]) < 1e-12  # equivariant in query order
    oc, Sc, zc = oracle.causal(q, k, v)
    assert row_rel_err(oc[:, :, -1], o[:, :, -1]) < 1e-12
    assert mat_rel_err(Sc, S) < 1e-12


# ------------------------------------------------- delta rule

def _one_hot(idx, D, n_lead=(1, 1)):
    x = np.full(n_lead + (len(idx), D), -200.0)
    x[..., np.arange(len(idx)), idx] = 0.0
    return x


def test_delta_D1_is_exponential_moving_average():
    N, M = 50, 3
    g = np.random.default_rng(121)
    q, k = rnd((1, 1, N, 1), 122), rnd((1, 1, N, 1), 123)
    v = rnd((1, 1, N, M), 124)
    beta = g.uniform(0, 1, size=(1, 1, N))
    W0 = rnd((1, 1, M, 1), 125)
    o, W = oracle.deltanet(q, k, v, beta, W0=W0)
    w = W0[0, 0, :, 0].copy()
    for i in range(N):
        w = (1 - beta[0, 0, i]) * w + beta[0, 0, i] * v[0, 0, i]
        np.testing.assert_allclose(o[0, 0, i], w, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(W[0, 0, :, 0], w, rtol=1e-12, atol=1e-13)


def test_delta_exact_recall_and_overwrite():
    D, M = 6, 3
    g = np.random.default_rng(131)
    slots = [2, 0, 5, 2]
    vals = g.integers(-9, 10, size=(4, M)).astype(np.float64)
    k = _one_hot(slots, D)
    v = vals[None, None]
    beta = np.ones((1, 1, 4))
    # query slot 2 after every write: first v0, then v0, v0, then the overwrite v3
    q = _one_hot([2, 2, 2, 2], D)
    o, W = oracle.deltanet(q, k, v, beta)
    np.testing.assert_allclose(o[0, 0, :3], np.repeat(vals[:1], 3, axis=0), rtol=0, atol=1e-12)
    np.testing.assert_allclose(o[0, 0, 3], vals[3], rtol=0, atol=1e-12)  # not vals[0] + vals[3]
    # every slot returns what was last written to it
    for s, want in [(0, vals[1]), (5, vals[2]), (2, vals[3]), (1, np.zeros(M))]:
        np.testing.assert_allclose(W[0, 0] @ np.eye(D)[s], want, rtol=0, atol=1e-12)


def test_delta_repeated_writes_closed_form():
    D, M, T = 4, 2, 12
    b = 0.3
    vv = np.array([2.0, -5.0])
    k = _one_hot([1] * T, D)
    q = _one_hot([1] * T, D)
    v = np.broadcast_to(vv, (1, 1, T, M)).copy()
    o, _ = oracle.deltanet(q, k, v, np.full((1, 1, T), b))
    for t in range(1, T + 1):
        np.testing.assert_allclose(o[0, 0, t - 1], (1 - (1 - b) ** t) * vv, rtol=1e-12, atol=1e-13)


def test_delta_beta_zero_keeps_initial_memory():
    N, D, M = 20, 5, 4
    q, k, v = rnd((1, 2, N, D), 141), rnd((1, 2, N, D), 142), rnd((1, 2, N, M), 143)
    W0 = rnd((1, 2, M, D), 144)
    o, W = oracle.deltanet(q, k, v, np.zeros((1, 2, N)), W0=W0)
    # remove-then-write with vnew = vbar is the identity up to an ulp per step
    np.testing.assert_allclose(W, W0, rtol=0, atol=1e-14)
    pq = phi_lib(q)
    qh = pq / pq.sum(axis=-1, keepdims=True)
    np.testing.assert_allclose(o, np.einsum("bhmd,bhnd->bhnm", W0, qh), rtol=1e-12, atol=1e-13)
    o0, W0z = oracle.deltanet(q, k, v, np.zeros((1, 2, N)))
    assert np.all(o0 == 0) and np.all(W0z == 0)


def test_delta_fresh_slots_match_additive_rule():
    D, M = 8, 3
    g = np.random.default_rng(151)
    slots = [3, 0, 7, 5, 1]
    beta = g.uniform(0, 1, size=(1, 1, len(slots)))
    v = rnd((1, 1, len(slots), M), 152)
    k = _one_hot(slots, D)
    _, W = oracle.deltanet(k, k, v, beta)
    ref = sum(beta[0, 0, j] * np.outer(v[0, 0, j], np.eye(D)[s]) for j, s in enumerate(slots))
    np.testing.assert_allclose(W[0, 0], ref, rtol=1e-12, atol=1e-13)


def test_delta_affine_product_form():
    """Each step is the affine map W -> W (I - b kh kh^T) + b v kh^T, so
    W_N = W0 P_1..N + sum_j b_j v_j kh_j^T P_{j+1}..N with P the ordered product
    of (I - b kh kh^T); evaluated here as a sum over j of matrix products."""
    N, D, M = 9, 4, 3
    g = np.random.default_rng(161)
    q, k, v = rnd((1, 1, N, D), 162), rnd((1, 1, N, D), 163), rnd((1, 1, N, M), 164)
    beta = g.uniform(0, 1, size=(1, 1, N))
    W0 = rnd((1, 1, M, D), 165)
    o, W = oracle.deltanet(q, k, v, beta, W0=W0)
    pk = phi_lib(k[0, 0])
    kh = pk / pk.sum(axis=1, keepdims=True)
    A = [np.eye(D) - beta[0, 0, j] * np.outer(kh[j], kh[j]) for j in range(N)]

    def prod(a, b):
        P = np.eye(D)
        for j in range(a, b):
            P = P @ A[j]
        return P

    ref = W0[0, 0] @ prod(0, N)
    for j in range(N):
        ref = ref + beta[0, 0, j] * np.outer(v[0, 0, j], kh[j]) @ prod(j + 1, N)
    np.testing.assert_allclose(W[0, 0], ref, rtol=1e-12, atol=1e-12)


def test_delta_rows_are_independent():
    N, D, M = 25, 5, 6
    g = np.random.default_rng(171)
    q, k, v = rnd((1, 1, N, D), 172), rnd((1, 1, N, D), 173), rnd((1, 1, N, M), 174)
    beta = g.uniform(0, 1, size=(1, 1, N))
    o, W = oracle.deltanet(q, k, v, beta)
    perm = g.permutation(M)
    o2, W2 = oracle.deltanet(q, k, v[..., perm], beta)
    np.testing.assert_allclose(o2, o[..., perm], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(W2, W[:, :, perm, :], rtol=1e-14, atol=1e-15)


def test_nan_propagates():
    q, k, v = rnd((1, 1, 5, 3), 181), rnd((1, 1, 5, 3), 182), rnd((1, 1, 5, 2), 183)
    v[0, 0, 2, 1] = np.nan
    o, _, _ = oracle.causal(q, k, v)
    assert np.all(np.isfinite(o[0, 0, :2])) and np.isnan(o[0, 0, 2:, 1]).all()


# ------------------------------------------- gradients (§3.3.1; equations not printed)

def _bwd_inputs(B, H, N, D, M, seed):
    return (rnd((B, H, N, D), seed), rnd((B, H, N, D), seed + 1), rnd((B, H, N, M), seed + 2),
            rnd((B, H, N, M), seed + 3))


def test_bwd_matches_central_finite_differences():
    """Every input element: autograd of the oracle against (L(x+h) - L(x-h)) / 2h."""
    from oracle import gradients
    q, k, v, dO = _bwd_inputs(1, 2, 6, 3, 2, 11)
    dq, dk, dv = gradients.causal_bwd(q, k, v, dO)
    h = 1e-6
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = xp, xm
            fd = (gradients.causal_loss(args_p["q"], args_p["k"], args_p["v"], dO)
                  - gradients.causal_loss(args_m["q"], args_m["k"], args_m["v"], dO)) / (2 * h)
            assert abs(fd - grad[idx]) < 1e-6 * max(1.0, abs(grad[idx])), (name, idx, fd, grad[idx])


def test_bwd_recurrent_and_explicit_forms_agree():
    """Autograd through the prefix sums (eq.(10)-(12)) and through the masked matrix (eq.(9))."""
    from oracle import gradients
    q, k, v, dO = _bwd_inputs(2, 2, 50, 8, 5, 21)
    r = gradients.causal_bwd(q, k, v, dO, form="recurrent")
    e = gradients.causal_bwd(q, k, v, dO, form="explicit")
    for a, b in zip(r, e):
        assert mat_rel_err(a, b) < 1e-12


def test_bwd_single_token_passes_values_through():
    """N = 1: o = v whatever q, k, so dv = dO and dq = dk = 0."""
    q, k, v, dO = _bwd_inputs(2, 3, 1, 8, 5, 31)
    dq, dk, dv = oracle.causal_bwd(q, k, v, dO)
    np.testing.assert_allclose(dv, dO, rtol=1e-14, atol=1e-14)
    assert np.abs(dq).max() < 1e-13 and np.abs(dk).max() < 1e-13


def test_bwd_first_query_gradient_vanishes():
    """o_1 = v_1 for any q_1 and q_1 enters no later output, so dq_1 = 0 at every N
    (the GPU tests treat that row as identically zero); no other row of dq is."""
    q, k, v, dO = _bwd_inputs(2, 2, 50, 8, 6, 33)
    dq, _, _ = oracle.causal_bwd(q, k, v, dO)
    assert np.abs(dq[:, :, 0]).max() < 1e-14 * np.abs(dq).max()
    assert np.abs(dq[:, :, 1:]).max(axis=-1).min() > 1e-6 * np.abs(dq).max()


def test_bwd_quotient_rule_form_and_term_scale():
    """The query gradient as the quotient rule writes it, (S_i dO_i - z_i (dO_i . o_i)) / den_i
    times phi'(q_i), equals the autograd gradient; the term scale the GPU tests use
    as a floor bounds every row (a difference of two terms is at most twice the
    larger) and is far above the row where the two terms cancel."""
    from oracle import gradients
    q, k, v, dO = _bwd_inputs(2, 2, 60, 8, 5, 35)
    dq, _, _ = oracle.causal_bwd(q, k, v, dO)
    assert mat_rel_err(gradients.dq_from_terms(q, k, v, dO), dq) < 1e-12
    scale = gradients.dq_term_scale(q, k, v, dO)
    rows = np.abs(dq).max(axis=-1)
    assert np.all(rows <= 2.0 * scale * (1 + 1e-12))
    assert np.all(scale[:, :, 0] > 1e6 * rows[:, :, 0])   # the first token: terms cancel exactly


def test_bwd_is_causal():
    """dq_i depends on keys and values j <= i only; dk_j, dv_j on output gradients i >= j only."""
    q, k, v, dO = _bwd_inputs(1, 2, 40, 6, 4, 41)
    dq, dk, dv = oracle.causal_bwd(q, k, v, dO)
    k2, v2 = k.copy(), v.copy()
    k2[:, :, 25:] += 1.0
    v2[:, :, 25:] -= 2.0
    dq2, _, _ = oracle.causal_bwd(q, k2, v2, dO)
    np.testing.assert_allclose(dq2[:, :, :25], dq[:, :, :25], rtol=1e-12, atol=1e-14)
    dO2 = dO.copy()
    dO2[:, :, :25] *= -3.0
    _, dk2, dv2 = oracle.causal_bwd(q, k, v, dO2)
    np.testing.assert_allclose(dk2[:, :, 25:], dk[:, :, 25:], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dv2[:, :, 25:], dv[:, :, 25:], rtol=1e-12, atol=1e-14)


def test_bwd_invariants_of_the_normalised_form():
    """o_i is a convex combination of v_1..v_i with weights homogeneous of degree 0 in phi(q_i):
    (a) the derivative along phi(q_i) vanishes: sum_d dphi(q)_id phi(q)_id = 0;
    (b) shifting every v by c shifts every o by c: dq, dk do not change and sum_j dv_j = sum_i dO_i."""
    q, k, v, dO = _bwd_inputs(2, 2, 30, 5, 3, 51)
    dq, dk, dv = oracle.causal_bwd(q, k, v, dO)
    dphi = np.where(q > 0, 1.0, np.exp(np.minimum(q, 0.0)))
    fq = phi_lib(q)
    radial = (dq / dphi * fq).sum(axis=-1)
    assert np.abs(radial).max() < 1e-12 * max(1.0, np.abs(dq).max())
    dq2, dk2, _ = oracle.causal_bwd(q, k, v + np.array([0.7, -1.3, 2.0]), dO)
    assert mat_rel_err(dq2, dq) < 1e-12 and mat_rel_err(dk2, dk) < 1e-12
    np.testing.assert_allclose(dv.sum(axis=2), dO.sum(axis=2), rtol=1e-12, atol=1e-12)


# ------------------------------------------------ softmax decode baseline
# The "stateful softmax" comparison baseline ([TR] Appendix C.1): softmax
# attention, [TR] §3.1 eq.(2), of one new token over a key/value cache.

def _cache(B, H, L, Lmax, D, M, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, D))
    k = rng.standard_normal((B, H, D))
    v = rng.standard_normal((B, H, M))
    Kc = rng.standard_normal((B, H, Lmax, D))
    Vc = rng.standard_normal((B, H, Lmax, M))
    return q, k, v, Kc, Vc


@pytest.mark.parametrize("D,M", [(4, 3), (8, 8), (32, 64)])
def test_softmax_decode_matches_bruteforce(D, M):
    q, k, v, Kc, Vc = _cache(2, 2, 9, 12, D, M, seed=D + M)
    o, K2, V2 = oracle.softmax_decode(q, k, v, Kc, Vc, 9)
    for b in range(2):
        for h in range(2):
            ref = brute.softmax_row(list(q[b, h]), [list(r) for r in K2[b, h, :10]], [list(r) for r in V2[b, h, :10]])
            assert np.abs(o[b, h] - np.array(ref)).max() < 1e-12
    # the append writes exactly the new row and leaves the others
    assert np.array_equal(K2[:, :, 9], k) and np.array_equal(V2[:, :, 9], v)
    assert np.array_equal(np.delete(K2, 9, axis=2), np.delete(Kc, 9, axis=2))


def test_softmax_decode_first_token_returns_value():
    q, k, v, Kc, Vc = _cache(3, 2, 0, 4, 8, 5, seed=1)
    o, _, _ = oracle.softmax_decode(q, k, v, Kc, Vc, 0)
    assert np.array_equal(o, v)


def test_softmax_decode_constant_keys_give_mean():
    q, k, v, Kc, Vc = _cache(2, 3, 7, 10, 16, 6, seed=2)
    Kc[:, :, :7] = k[:, :, None, :]
    o, _, V2 = oracle.softmax_decode(q, k, v, Kc, Vc, 7)
    assert np.abs(o - V2[:, :, :8].mean(axis=2)).max() < 1e-12


def test_softmax_decode_shift_and_scale_properties():
    q, k, v, Kc, Vc = _cache(2, 2, 11, 16, 8, 4, seed=3)
    o, _, V2 = oracle.softmax_decode(q, k, v, Kc, Vc, 11)
    # adding one vector to every key adds the same constant to every score
    u = np.random.default_rng(4).standard_normal(8)
    o2, _, _ = oracle.softmax_decode(q, k + u, v, Kc + u, Vc, 11)
    assert np.abs(o2 - o).max() < 1e-12
    # outputs are convex combinations of the values
    lo, hi = V2[:, :, :12].min(axis=2), V2[:, :, :12].max(axis=2)
    assert (o >= lo - 1e-12).all() and (o <= hi + 1e-12).all()
    # affine in the values
    o3, _, _ = oracle.softmax_decode(q, k, 2.0 * v - 1.0, Kc, 2.0 * Vc - 1.0, 11)
    assert np.abs(o3 - (2.0 * o - 1.0)).max() < 1e-12


def test_softmax_decode_dominant_key_and_scaling():
    # q = a e_0 with key e_0 at row 3 and zero keys elsewhere: the weight of row 3
    # against each other row is exp(a / sqrt(D)); with a / sqrt(D) = 60 the output
    # is v_3 to within exp(-60) relative.
    D, M, L = 16, 4, 6
    q, k, v, Kc, Vc = _cache(1, 1, L, 8, D, M, seed=5)
    Kc[:] = 0.0
    k[:] = 0.0
    Kc[0, 0, 3, 0] = 1.0
    q[:] = 0.0
    q[0, 0, 0] = 60.0 * math.sqrt(D)
    o, _, _ = oracle.softmax_decode(q, k, v, Kc, Vc, L)
    assert np.abs(o[0, 0] - Vc[0, 0, 3]).max() < 1e-20 * np.abs(Vc).max() + 1e-24
    # with score gap exactly log 3 between row 3 and the six others: weight 3/9
    q[0, 0, 0] = math.log(3.0) * math.sqrt(D)
    o, _, V2 = oracle.softmax_decode(q, k, v, Kc, Vc, L)
    others = [j for j in range(L + 1) if j != 3]
    expect = (3.0 * V2[0, 0, 3] + V2[0, 0, others].sum(axis=0)) / 9.0
    assert np.abs(o[0, 0] - expect).max() < 1e-12


# ------------------------------------------------ other feature maps
# [TR] §3.2.1: any feature map phi of dimension C; the degree-2 polynomial
# kernel has an exact one with C = D^2.  [FWP] DPFP paragraph: DPFP-nu raises
# the dot-product dimension to 2 nu D (formula not printed; reading in the
# oracle's header).

FMAPS = [(oracle.DPFP, 1), (oracle.DPFP, 2), (oracle.DPFP, 3), (oracle.POLY2, 0)]
FM_GOLD = json.load(open(os.path.join(HERE, "golden", "feature_maps.json")))


def _sim_fn(fmap, nu):
    if fmap == oracle.DPFP:
        return lambda a, b: brute.dpfp_sim(a, b, nu)
    return brute.poly2_sim


@pytest.mark.parametrize("case", FM_GOLD["dpfp"], ids=lambda c: c["name"])
def test_dpfp_golden(case):
    got = oracle.feature_map(np.array(case["x"]), oracle.DPFP, case["nu"])
    assert np.array_equal(got, np.array(case["phi"]))


@pytest.mark.parametrize("case", FM_GOLD["poly2"], ids=lambda c: c["name"])
def test_poly2_golden(case):
    got = oracle.feature_map(np.array(case["x"]), oracle.POLY2)
    assert np.array_equal(got, np.array(case["phi"]))


@pytest.mark.parametrize("case", FM_GOLD["causal"], ids=lambda c: c["name"])
def test_fmap_causal_golden(case):
    fmap = oracle.DPFP if case["fmap"] == "dpfp" else oracle.POLY2
    q, k, v = (np.array(case[x])[None, None] for x in ("q", "k", "v"))
    o, _, _ = oracle.fmap_causal(q, k, v, fmap, case["nu"])
    np.testing.assert_allclose(o[0, 0], np.array(case["o"]), rtol=1e-14, atol=0)


def test_fmap_dimensions():
    for D in (2, 3, 32, 64):
        for nu in (1, 2, 3):
            assert oracle.fmap_dim(oracle.DPFP, nu, D) == 2 * nu * D
        assert oracle.fmap_dim(oracle.POLY2, 0, D) == D * D
    assert oracle.fmap_dim(7, 1, 64) == 0


def test_poly2_closed_form():
    # phi(q).phi(k) = (q.k)^2: numpy's dot, squared, against the feature vectors
    for D, seed in ((5, 1), (32, 2), (64, 3)):
        q, k = rnd((8, D), seed), rnd((8, D), seed + 10)
        fq, fk = oracle.feature_map(q, oracle.POLY2), oracle.feature_map(k, oracle.POLY2)
        expect = np.einsum("id,jd->ij", q, k) ** 2
        np.testing.assert_allclose(fq @ fk.T, expect, rtol=1e-12, atol=1e-12)


def test_dpfp_properties():
    x = rnd((50, 6), 4)
    for nu in (1, 2, 3):
        f = oracle.feature_map(x, oracle.DPFP, nu)
        assert f.shape == (50, 12 * nu) and (f >= 0).all()
        # degree-2 homogeneity for c > 0
        np.testing.assert_allclose(oracle.feature_map(2.5 * x, oracle.DPFP, nu), 6.25 * f, rtol=1e-14)
        # x -> -x swaps the two halves of r: each 2D block turns by D
        fneg = oracle.feature_map(-x, oracle.DPFP, nu)
        blocks = f.reshape(50, nu, 12)
        np.testing.assert_array_equal(fneg.reshape(50, nu, 12), np.roll(blocks, -6, axis=2))
        # DPFP-nu extends DPFP-(nu-1)
        if nu > 1:
            np.testing.assert_array_equal(f[:, :12 * (nu - 1)], oracle.feature_map(x, oracle.DPFP, nu - 1))
    # the figure: a generic 2-d point has exactly one non-zero of four, and the
    # non-zero slot is its quadrant, so points in different quadrants are orthogonal
    p = rnd((200, 2), 5)
    f = oracle.feature_map(p, oracle.DPFP, 1)
    assert ((f > 0).sum(axis=1) == 1).all()
    quad = np.where(p[:, 0] > 0, np.where(p[:, 1] > 0, 0, 3), np.where(p[:, 1] > 0, 1, 2))
    assert np.array_equal(f.argmax(axis=1), quad)
    np.testing.assert_allclose(f.max(axis=1), np.abs(p[:, 0] * p[:, 1]), rtol=1e-15)


def test_dpfp_pair_sum_agrees_with_features():
    # the pair-sum form of the brute force against the feature vectors of the C oracle
    q, k = rnd((6, 5), 6), rnd((6, 5), 7)
    for nu in (1, 2, 3):
        fq, fk = oracle.feature_map(q, oracle.DPFP, nu), oracle.feature_map(k, oracle.DPFP, nu)
        for i in range(6):
            for j in range(6):
                assert abs(fq[i] @ fk[j] - brute.dpfp_sim(list(q[i]), list(k[j]), nu)) < 1e-12


@pytest.mark.parametrize("fmap,nu", FMAPS)
def test_fmap_causal_and_noncausal_match_bruteforce(fmap, nu):
    B, H, N, D, M = 1, 2, 7, 4, 3
    q, k, v = rnd((B, H, N, D), 8), rnd((B, H, N, D), 9), rnd((B, H, N, M), 10)
    if fmap == oracle.DPFP:
        q, k = np.abs(q) + 0.1, np.abs(k) + 0.1  # one quadrant: no all-zero weight row
    o, S, z = oracle.fmap_causal(q, k, v, fmap, nu)
    onc, Snc, znc = oracle.fmap_noncausal(q, k, v, fmap, nu)
    for h in range(H):
        args = ([list(r) for r in q[0, h]], [list(r) for r in k[0, h]], [list(r) for r in v[0, h]])
        ref = np.array(brute.attention(*args, causal=True, sim_fn=_sim_fn(fmap, nu)))
        refnc = np.array(brute.attention(*args, causal=False, sim_fn=_sim_fn(fmap, nu)))
        assert np.abs(o[0, h] - ref).max() < 1e-12
        assert np.abs(onc[0, h] - refnc).max() < 1e-12
    # the last causal row sees every key; both forms end in the same state
    np.testing.assert_allclose(o[:, :, -1], onc[:, :, -1], rtol=1e-12)
    np.testing.assert_allclose(S, Snc, rtol=1e-12)
    np.testing.assert_allclose(z, znc, rtol=1e-12)


@pytest.mark.parametrize("fmap,nu", FMAPS)
def test_fmap_state_split_and_sums(fmap, nu):
    B, H, N, D, M = 2, 1, 20, 4, 5
    q, k, v = rnd((B, H, N, D), 11), rnd((B, H, N, D), 12), rnd((B, H, N, M), 13)
    o, S, z = oracle.fmap_causal(q, k, v, fmap, nu)
    fk = oracle.feature_map(k, fmap, nu)
    # S = phi(K)^T V and z = column sums of phi(K) (numpy matmul)
    np.testing.assert_allclose(S, np.swapaxes(fk, -1, -2) @ v, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(z, fk.sum(axis=2), rtol=1e-12, atol=1e-12)
    # carrying the state across a split reproduces the whole sequence
    m = 9
    o1, S1, z1 = oracle.fmap_causal(q[:, :, :m], k[:, :, :m], v[:, :, :m], fmap, nu)
    o2, S2, z2 = oracle.fmap_causal(q[:, :, m:], k[:, :, m:], v[:, :, m:], fmap, nu, S0=S1, z0=z1)
    np.testing.assert_allclose(np.concatenate([o1, o2], axis=2), o, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S2, S, rtol=1e-12, atol=1e-12)


def test_fmap_invariances():
    B, H, N, D, M = 1, 2, 12, 6, 4
    q, k, v = rnd((B, H, N, D), 14), rnd((B, H, N, D), 15), rnd((B, H, N, M), 16)
    # polynomial: (q.k)^2 is even in q and scales as c^2 in every key
    o, _, _ = oracle.fmap_causal(q, k, v, oracle.POLY2)
    flip = np.where(np.arange(N)[None, None, :, None] % 2 == 0, -q, q)
    o2, _, _ = oracle.fmap_causal(flip, 3.0 * k, v, oracle.POLY2)
    np.testing.assert_allclose(o2, o, rtol=1e-10, atol=1e-12)
    # DPFP: negating every q and k permutes both feature vectors alike; positive
    # scaling of q cancels between numerator and denominator
    qa, ka = np.abs(q) * np.sign(q[..., :1]), np.abs(k) * np.sign(q[..., :1])  # shared sign pattern
    for nu in (1, 2, 3):
        o, _, _ = oracle.fmap_causal(qa, ka, v, oracle.DPFP, nu)
        o2, _, _ = oracle.fmap_causal(-2.0 * qa, -ka, v, oracle.DPFP, nu)
        np.testing.assert_allclose(o2, o, rtol=1e-10, atol=1e-12)
    # outputs are convex combinations of the values seen so far
    for fmap, nu in FMAPS:
        qa2, ka2 = (np.abs(q), np.abs(k)) if fmap == oracle.DPFP else (q, k)
        o, _, _ = oracle.fmap_causal(qa2, ka2, v, fmap, nu)
        lo = np.minimum.accumulate(v, axis=2)
        hi = np.maximum.accumulate(v, axis=2)
        assert (o >= lo - 1e-12).all() and (o <= hi + 1e-12).all()
