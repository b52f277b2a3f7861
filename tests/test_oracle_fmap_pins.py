"""Pins of the oracle's feature-map variants (ELU + 1, ReLU, random Fourier
features of "Linear Attention > Kernel Feature Maps", sections 1-3) against
their definitions written out entry by entry, closed forms (the identity
projection gives the page's elementwise maps; sin^2 + cos^2 = 1), the Gaussian
kernel that random Fourier features estimate, with its closed-form variance,
and brute-force attention loops.
"""
import math

import numpy as np
import pytest

import oracle


def test_identity_projection_gives_the_elementwise_maps():
    x = np.array([[2.0, -1.0, 0.0, 0.5, -3.0]])
    eye = np.eye(5)
    np.testing.assert_allclose(oracle.feature_map(x, eye, "elu1")[0],
                               [3.0, math.exp(-1.0), 1.0, 1.5, math.exp(-3.0)], rtol=1e-15)
    np.testing.assert_allclose(oracle.feature_map(x, eye, "relu")[0], [2.0, 0.0, 0.0, 0.5, 0.0], rtol=0)


def test_elu1_is_continuous_and_positive():
    w = np.eye(1)
    for t in (1e-9, 1e-6):
        a = oracle.feature_map(np.array([[t]]), w, "elu1")[0, 0]
        b = oracle.feature_map(np.array([[-t]]), w, "elu1")[0, 0]
        assert abs(a - b) < 3 * t
    rng = np.random.default_rng(41)
    assert np.all(oracle.feature_map(rng.standard_normal((50, 4)) * 5, rng.standard_normal((8, 4)), "elu1") > 0)


def test_trig_layout_and_unit_norm():
    """Output 2i is sin(omega_i . x)/sqrt(m), 2i+1 the cosine; the squared norm
    of every feature vector is exactly 1."""
    rng = np.random.default_rng(42)
    x = rng.standard_normal((7, 3))
    w = rng.standard_normal((5, 3))
    phi = oracle.feature_map(x, w, "trig")
    assert phi.shape == (7, 10)
    for i in range(7):
        for f in range(5):
            p = sum(w[f, j] * x[i, j] for j in range(3))
            assert abs(phi[i, 2 * f] - math.sin(p) / math.sqrt(5)) < 1e-15
            assert abs(phi[i, 2 * f + 1] - math.cos(p) / math.sqrt(5)) < 1e-15
    np.testing.assert_allclose((phi ** 2).sum(1), 1.0, rtol=1e-14)


def test_trig_estimates_the_gaussian_kernel():
    """With omega ~ N(0, I): E[phi(q).phi(k)] = E[cos(omega.(q-k))] =
    exp(-|q-k|^2/2), and Var = (1 - exp(-|q-k|^2))^2 / (2m) for independent
    rows (from E[cos^2] = (1 + exp(-2|delta|^2))/2)."""
    rng = np.random.default_rng(43)
    d, m, trials = 4, 64, 20000
    q = rng.standard_normal(d) * 0.5
    k = rng.standard_normal(d) * 0.5
    est = np.empty(trials)
    for t in range(trials):
        w = rng.standard_normal((m, d))
        est[t] = oracle.feature_map(q[None], w, "trig")[0] @ oracle.feature_map(k[None], w, "trig")[0]
    d2 = float(np.sum((q - k) ** 2))
    mean = math.exp(-d2 / 2)
    var = (1 - math.exp(-d2)) ** 2 / (2 * m)
    assert abs(est.mean() - mean) < 4 * math.sqrt(var / trials)
    assert abs(est.var() / var - 1) < 0.05


def _brute(q, k, v, w, eps, causal, phi):
    L = q.shape[0]
    pq = [phi(q[i]) for i in range(L)]
    pk = [phi(k[j]) for j in range(L)]
    out = np.zeros((L, v.shape[1]))
    for i in range(L):
        den = eps
        for j in range(L):
            if causal and j > i:
                continue
            a = sum(pq[i][f] * pk[j][f] for f in range(len(pq[i])))
            den += a
            out[i] += a * v[j]
        out[i] /= den
    return out


def _phi_by_hand(w, kind):
    m, d = w.shape

    def proj(x, f):
        return sum(w[f][j] * x[j] for j in range(d))

    if kind == "elu1":
        return lambda x: [proj(x, f) + 1 if proj(x, f) > 0 else math.exp(proj(x, f)) for f in range(m)]
    if kind == "relu":
        return lambda x: [max(0.0, proj(x, f)) for f in range(m)]
    return lambda x: [g(proj(x, f)) / math.sqrt(m) for f in range(m) for g in (math.sin, math.cos)]


@pytest.mark.parametrize("kind", ["elu1", "relu", "trig"])
@pytest.mark.parametrize("causal", [False, True])
def test_attention_variants_brute_force(kind, causal):
    rng = np.random.default_rng(44)
    L, d, m = 7, 3, 5
    q = rng.standard_normal((L, d)) * 0.4
    k = rng.standard_normal((L, d)) * 0.4
    v = rng.standard_normal((L, 2))
    w = rng.standard_normal((m, d))
    eps = 0.05
    ref = _brute(q, k, v, w, eps, causal, _phi_by_hand(w, kind))
    np.testing.assert_allclose(oracle.attn_quadratic(q, k, v, w, eps, causal, kind=kind), ref, rtol=1e-11)
    fn = oracle.attn_causal if causal else oracle.attn_noncausal
    np.testing.assert_allclose(fn(q, k, v, w, eps, kind=kind), ref, rtol=1e-11)
    np.testing.assert_allclose(oracle.attn_rows(q, k, v, w, range(L), eps, causal, kind=kind), ref, rtol=1e-11)


def test_relu_query_with_no_active_feature_outputs_zero():
    """A query whose projections are all <= 0 has phi = 0: the numerator is 0
    and the denominator is eps, so its output row is exactly 0."""
    w = np.eye(2)
    q = np.array([[-1.0, -2.0], [1.0, 0.5]])
    k = np.array([[0.5, 1.0], [2.0, 0.1]])
    v = np.array([[1.0, 2.0], [3.0, 4.0]])
    out = oracle.attn_noncausal(q, k, v, w, 1e-6, kind="relu")
    assert np.all(out[0] == 0.0)
    assert np.all(out[1] != 0.0)
