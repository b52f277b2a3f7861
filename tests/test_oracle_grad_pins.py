"""Pins of the oracle's backward pass (gradients of sum(G * O) with respect to
Q, K and V) against what the mathematics fixes, independently of the
oracle's chain-rule code: central finite differences of the forward
definition (the L x L quadratic form, itself pinned in test_oracle_pins),
a closed form for W = 0, and the identity sum_j dv_j = sum_i g_i (1 - eps/den_i).
A dropped term, a wrong sign, a transposed state or a mask off by one in the
reverse accumulation fails at least one of them.
"""
import numpy as np
import pytest

import oracle


def _inputs(seed, L, d, m, scale=0.6):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((L, d)) * scale
    k = rng.standard_normal((L, d)) * scale
    v = rng.standard_normal((L, d))
    w = rng.standard_normal((m, d))
    g = rng.standard_normal((L, d))
    return q, k, v, w, g


def _fd_grads(q, k, v, w, g, eps, causal, h=1e-5):
    """Central differences of sum(G * O) with O the quadratic definition."""
    def loss(qq, kk, vv):
        return float(np.sum(g * oracle.attn_quadratic(qq, kk, vv, w, eps, causal)))

    out = []
    for which in range(3):
        args = [q.copy(), k.copy(), v.copy()]
        grad = np.empty_like(args[which])
        for idx in np.ndindex(grad.shape):
            x0 = args[which][idx]
            args[which][idx] = x0 + h
            lp = loss(*args)
            args[which][idx] = x0 - h
            lm = loss(*args)
            args[which][idx] = x0
            grad[idx] = (lp - lm) / (2 * h)
        out.append(grad)
    return out


def _grad_fn(causal):
    return oracle.attn_causal_grad if causal else oracle.attn_noncausal_grad


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("seed,L,d,m,eps", [(31, 7, 3, 5, 0.05), (32, 9, 4, 8, 1e-6), (33, 5, 6, 3, 0.3)])
def test_gradients_match_finite_differences(causal, seed, L, d, m, eps):
    q, k, v, w, g = _inputs(seed, L, d, m)
    got = _grad_fn(causal)(q, k, v, w, g, eps)
    ref = _fd_grads(q, k, v, w, g, eps, causal)
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        scale = np.abs(b).max()
        assert np.abs(a - b).max() <= 1e-7 * scale, name


def test_feature_vjp_matches_finite_differences():
    rng = np.random.default_rng(34)
    x = rng.standard_normal((3, 5)) * 0.5
    w = rng.standard_normal((7, 5))
    dphi = rng.standard_normal((3, 7))
    phi = oracle.favor_features(x, w)
    got = oracle.favor_features_vjp(x, w, phi, dphi)
    h = 1e-6
    ref = np.empty_like(x)
    for idx in np.ndindex(x.shape):
        xp, xm = x.copy(), x.copy()
        xp[idx] += h
        xm[idx] -= h
        ref[idx] = np.sum(dphi * (oracle.favor_features(xp, w) - oracle.favor_features(xm, w))) / (2 * h)
    np.testing.assert_allclose(got, ref, rtol=1e-7, atol=1e-9)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_projection_gradient_closed_form(causal):
    """W = 0: phi(x) = a(x)/sqrt(m) in every coordinate with a(x) = exp(-|x|^2/2),
    so a_ij = a_i b_j and o_i = a_i A_i / (a_i B_i + eps) with A_i = sum b_j v_j,
    B_i = sum b_j over the keys query i sees.  Differentiating by hand:
      dq_i = -(g_i . A_i) eps a_i q_i / (a_i B_i + eps)^2,
      dv_j = b_j sum_i a_i g_i / (a_i B_i + eps),
      dk_j = -b_j k_j sum_i a_i g_i . (v_j - o_i) / (a_i B_i + eps),
    the sums over the queries i that see key j."""
    rng = np.random.default_rng(35)
    L, d, m = 8, 4, 6
    q = rng.standard_normal((L, d))
    k = rng.standard_normal((L, d))
    v = rng.standard_normal((L, d))
    g = rng.standard_normal((L, d))
    w = np.zeros((m, d))
    eps = 0.2
    a = np.exp(-0.5 * (q * q).sum(1))
    b = np.exp(-0.5 * (k * k).sum(1))
    sees = np.tril(np.ones((L, L))) if causal else np.ones((L, L))      # sees[i, j]
    A = sees @ (b[:, None] * v)
    B = sees @ b
    den = a * B + eps
    o = a[:, None] * A / den[:, None]
    dq = -((g * A).sum(1) * eps * a / den ** 2)[:, None] * q
    coef = a[:, None] * g / den[:, None]                                 # [i, c]
    dv = b[:, None] * (sees.T @ coef)
    dk = np.empty_like(k)
    for j in range(L):
        s = sum(sees[i, j] * a[i] * (g[i] @ (v[j] - o[i])) / den[i] for i in range(L))
        dk[j] = -b[j] * k[j] * s
    got = _grad_fn(causal)(q, k, v, w, g, eps)
    for x, y in zip(got, (dq, dk, dv)):
        np.testing.assert_allclose(x, y, rtol=1e-11, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_value_gradient_sums_to_weighted_upstream(causal):
    """sum_j dv_j = sum_i g_i sum_j a_ij / den_i = sum_i g_i (1 - eps/den_i)."""
    rng = np.random.default_rng(36)
    L, d, m = 40, 8, 32
    q = rng.standard_normal((L, d)) * d ** -0.25
    k = rng.standard_normal((L, d)) * d ** -0.25
    v = rng.standard_normal((L, d))
    g = rng.standard_normal((L, d))
    w = rng.standard_normal((m, d))
    eps = 0.01
    fq = oracle.favor_features(q, w)
    fk = oracle.favor_features(k, w)
    a = fq @ fk.T
    if causal:
        a = np.tril(a)
    den = a.sum(1) + eps
    _, _, dv = _grad_fn(causal)(q, k, v, w, g, eps)
    np.testing.assert_allclose(dv.sum(0), (g * (1 - eps / den)[:, None]).sum(0), rtol=1e-11)


def test_causal_last_key_sees_only_last_query():
    """Key L-1 is seen by query L-1 alone, so its gradients depend on that row."""
    q, k, v, w, g = _inputs(37, 6, 4, 8)
    _, dk1, dv1 = oracle.attn_causal_grad(q, k, v, w, g, 0.05)
    g2 = g.copy()
    g2[:-1] = 0.0
    _, dk2, dv2 = oracle.attn_causal_grad(q, k, v, w, g2, 0.05)
    np.testing.assert_allclose(dv1[-1], dv2[-1], rtol=1e-12)
    np.testing.assert_allclose(dk1[-1], dk2[-1], rtol=1e-12)


def test_per_head_grad_uses_the_right_projection():
    rng = np.random.default_rng(38)
    B, H, L, d, m = 1, 2, 5, 4, 8
    q, k, v, g = (rng.standard_normal((B, H, L, d)) for _ in range(4))
    w = rng.standard_normal((H, m, d))
    dq, dk, dv = oracle.per_head_grad(oracle.attn_noncausal_grad, q, k, v, w, g, eps=0.1)
    for h in range(H):
        ref = oracle.attn_noncausal_grad(q[0, h], k[0, h], v[0, h], w[h], g[0, h], 0.1)
        for x, y in zip((dq, dk, dv), ref):
            np.testing.assert_allclose(x[0, h], y, rtol=1e-13)
