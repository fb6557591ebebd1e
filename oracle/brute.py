"""Pure-Python brute force of the generalised attention of eq.(3), for tiny N.

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


def attention(q, k, v, causal=True):
    """q, k: lists of N lists of D floats; v: N lists of M floats.
    Returns N lists of M floats: sum_j sim(q_i,k_j) v_j / sum_j sim(q_i,k_j),
    with j <= i when causal (inclusive mask) and all j otherwise."""
    n = len(q)
    m_dim = len(v[0])
    out = []
    for i in range(n):
        last = i + 1 if causal else n
        weights = [sim(q[i], k[j]) for j in range(last)]
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
