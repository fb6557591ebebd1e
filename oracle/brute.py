"""Pure-Python brute force of the generalised attention of eq.(3), for tiny N,
with the elu + 1 map and with the similarity functions of the other feature
maps (DPFP-nu, degree-2 polynomial) written without their feature vectors.

TEST INFRASTRUCTURE ONLY (used by the oracle's own tests).

This is the oracle's own check: it evaluates [Transformers are RNNs
(Katharopoulos et al., 2020), translated page "線性變換器", §3.1 eq.(3) and
§3.3 eq.(8)] term by term with sim(q, k) = sum_d phi(q_d) phi(k_j,d), where
phi is written from the elu definition (alpha = 1) with Python's math module.
It shares no code with the C oracle: no loops over states, no prefix sums.
"""
import math


def elu_plus_one(x: float) -> float:
    """elu(x) + 1 from elu's definition: x for x > 0, alpha*(exp(x) - 1) otherwise."""
    elu = x if x > 0 else (math.exp(x) - 1.0)
    return elu + 1.0


def sim(qi, kj):
    return sum(elu_plus_one(a) * elu_plus_one(b) for a, b in zip(qi, kj))


def dpfp_sim(qi, kj, nu):
    """DPFP-nu similarity as a sum over index pairs, without feature vectors:
    with r(x) = (relu(x), relu(-x)) of length 2D, sum over n = 1..nu and
    i < 2D of r_i(q) r_{i+n}(q) r_i(k) r_{i+n}(k), indices mod 2D ([FWP], DPFP
    paragraph; reading of the unprinted formula)."""
    def r(x):
        return [max(a, 0.0) for a in x] + [max(-a, 0.0) for a in x]
    rq, rk = r(qi), r(kj)
    L = len(rq)
    return math.fsum(rq[i] * rq[(i + n) % L] * rk[i] * rk[(i + n) % L]
                     for n in range(1, nu + 1) for i in range(L))


def poly2_sim(qi, kj):
    """Degree-2 polynomial kernel, (q.k)^2 ([TR] §3.2.1)."""
    return math.fsum(a * b for a, b in zip(qi, kj)) ** 2


def attention(q, k, v, causal=True, sim_fn=sim):
    """q, k: lists of N lists of D floats; v: N lists of M floats.
    Returns N lists of M floats: sum_j sim(q_i,k_j) v_j / sum_j sim(q_i,k_j),
    with j <= i when causal (inclusive mask) and all j otherwise.  ``sim_fn``
    defaults to phi(q).phi(k) with phi = elu + 1."""
    n = len(q)
    m_dim = len(v[0])
    out = []
    for i in range(n):
        last = i + 1 if causal else n
        weights = [sim_fn(q[i], k[j]) for j in range(last)]
        total = math.fsum(weights)
        row = [math.fsum(weights[j] * v[j][m] for j in range(last)) / total for m in range(m_dim)]
        out.append(row)
    return out


def softmax_row(q, keys, values):
    """Softmax attention of one query, [TR] §3.1 eq.(2), term by term:
    weight_j = exp(q . k_j / sqrt(D)) / sum_i exp(q . k_i / sqrt(D)); returns
    sum_j weight_j v_j (no max subtraction: for the small scores of the tests the
    exponentials are exact enough)."""
    d = len(q)
    scores = [math.fsum(a * b for a, b in zip(q, kj)) / math.sqrt(d) for kj in keys]
    ex = [math.exp(s) for s in scores]
    total = math.fsum(ex)
    return [math.fsum(ex[j] * values[j][m] for j in range(len(keys))) / total for m in range(len(values[0]))]
