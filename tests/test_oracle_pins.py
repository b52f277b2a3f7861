"""Pins of the float64 oracle against what the pages and the mathematics fix.

Every check here is independent of the oracle's own code path: a printed worked
example, closed forms derived from the feature-map equation, Monte-Carlo
moments, and brute-force loops on tiny inputs.  Each is chosen so that a
plausible slip in the oracle (a dropped -|x|^2/2 or 1/sqrt(m), a sign, a wrong
mask index, eps in the wrong place, a transposed projection) fails at least one.
"""
import math
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _cosine_rows(a, b):
    return float(np.mean([a[i] @ b[i] / (np.linalg.norm(a[i]) * np.linalg.norm(b[i]))
                          for i in range(a.shape[0])]))


def _load_t1():
    rows = []
    with open(os.path.join(GOLDEN, "t1_quality.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                m, c, e = line.split()
                rows.append((int(m), float(c), float(e)))
    return rows


# ---------------------------------------------------------------------------
# 1. the printed worked example
# ---------------------------------------------------------------------------

def test_t1_table_reproduced_to_printed_digits():
    """Performer: Unbiased Softmax Approximation, Out[27]: every printed
    cosine (4 decimals) and MSE (6 decimals) is reproduced."""
    q, k, v = synth.t1_qkv()
    exact = oracle.softmax_attention(q, k, v, scale=1.0 / math.sqrt(32))
    for m, cos_printed, mse_printed in _load_t1():
        out = oracle.attn_noncausal(q, k, v, synth.t1_projection(m), eps=1e-6)
        assert round(_cosine_rows(exact, out), 4) == pytest.approx(cos_printed, abs=1e-12)
        assert round(float(np.mean((exact - out) ** 2)), 6) == pytest.approx(mse_printed, abs=1e-12)


def test_t1_unscaled_reference_does_not_reproduce():
    """The exact reference without a temperature gives visibly different
    numbers, which is why the 1/sqrt(d) reading is the one taken."""
    q, k, v = synth.t1_qkv()
    exact = oracle.softmax_attention(q, k, v, scale=1.0)
    out = oracle.attn_noncausal(q, k, v, synth.t1_projection(256))
    assert _cosine_rows(exact, out) < 0.95


# ---------------------------------------------------------------------------
# 2. the feature map: positivity, unbiasedness, variance
# ---------------------------------------------------------------------------

def test_features_strictly_positive():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((200, 16)) * 2.0
    w = rng.standard_normal((64, 16))
    phi = oracle.favor_features(x, w)
    assert phi.shape == (200, 64)
    assert np.all(phi > 0)


def test_features_closed_form_single_entry():
    """One entry written out with math.exp: exp(omega.x - |x|^2/2)/sqrt(m)."""
    x = np.array([0.3, -1.2, 0.5])
    w = np.array([[1.0, 0.0, 2.0], [-0.5, 0.25, 0.0]])
    phi = oracle.favor_features(x[None], w)[0]
    for i in range(2):
        dot = sum(w[i][j] * x[j] for j in range(3))
        sq = sum(t * t for t in x)
        assert phi[i] == pytest.approx(math.exp(dot - sq / 2) / math.sqrt(2), rel=1e-14)


def _mc_products(q, k, m, trials, rng, orthogonal=False):
    d = q.shape[0]
    vals = np.empty(trials)
    for t in range(trials):
        if orthogonal:
            w = synth.orthogonal_projection(rng, 1, m, d)[0]
        else:
            w = rng.standard_normal((m, d))
        vals[t] = oracle.favor_features(q[None], w)[0] @ oracle.favor_features(k[None], w)[0]
    return vals


def _closed_variance(q, k, m):
    """Var[phi(q).phi(k)] for m iid N(0, I) rows, from the lognormal moments of
    exp(omega.(q+k)): (1/m) * exp(2 q.k) * (exp(|q+k|^2) - 1)."""
    s = q + k
    return math.exp(2 * q @ k) * (math.exp(s @ s) - 1.0) / m


def test_unbiased_estimate_of_softmax_kernel():
    """E[phi(q).phi(k)] = exp(q.k) (P1 goal equation, P3 section 4)."""
    rng = np.random.default_rng(11)
    d, m, trials = 4, 64, 20000
    q = rng.standard_normal(d) * 0.5
    k = rng.standard_normal(d) * 0.5
    vals = _mc_products(q, k, m, trials, rng)
    target = math.exp(q @ k)
    se = math.sqrt(_closed_variance(q, k, m) / trials)
    assert abs(vals.mean() - target) < 5 * se
    assert abs(vals.mean() - target) / target < 0.01


def test_variance_matches_closed_form():
    rng = np.random.default_rng(12)
    d, m, trials = 4, 256, 20000
    q = rng.standard_normal(d) * 0.5
    k = rng.standard_normal(d) * 0.5
    vals = _mc_products(q, k, m, trials, rng)
    assert vals.var() == pytest.approx(_closed_variance(q, k, m), rel=0.05)


def test_variance_falls_as_one_over_m():
    """Doubling m halves the variance (P1, closing paragraph): m * Var is flat."""
    rng = np.random.default_rng(11)      # |q+k|^2 ~ 1: moderate lognormal tail
    d = 4
    q = rng.standard_normal(d) * 0.5
    k = rng.standard_normal(d) * 0.5
    scaled = []
    for m in (16, 64, 256):
        vals = _mc_products(q, k, m, 8000, rng)
        scaled.append(m * vals.var())
    ref = _closed_variance(q, k, 1)
    for s in scaled:
        assert s == pytest.approx(ref, rel=0.08)


def test_orthogonal_rows_unbiased_and_lower_variance():
    """Orthogonal rows keep the estimate unbiased and lower its variance (P2
    key points on orthogonality)."""
    rng = np.random.default_rng(14)
    d = m = 16
    q = rng.standard_normal(d) * 0.3
    k = rng.standard_normal(d) * 0.3
    iid = _mc_products(q, k, m, 6000, rng)
    orth = _mc_products(q, k, m, 6000, rng, orthogonal=True)
    target = math.exp(q @ k)
    se = math.sqrt(_closed_variance(q, k, m) / 6000)
    assert abs(orth.mean() - target) < 5 * se
    assert orth.var() < 0.95 * iid.var()


# ---------------------------------------------------------------------------
# 3. attention: brute force, reassociation, causal prefix sum
# ---------------------------------------------------------------------------

def _brute(q, k, v, w, eps, causal):
    """Pure-Python loops: every kernel estimate a_ij written out entry by entry."""
    L, d = q.shape
    m = w.shape[0]

    def phi(x):
        sq = sum(t * t for t in x)
        return [math.exp(sum(w[f][j] * x[j] for j in range(d)) - sq / 2) / math.sqrt(m)
                for f in range(m)]

    pq = [phi(q[i]) for i in range(L)]
    pk = [phi(k[j]) for j in range(L)]
    out = np.zeros((L, v.shape[1]))
    for i in range(L):
        den = eps
        for j in range(L):
            if causal and j > i:
                continue
            a = sum(pq[i][f] * pk[j][f] for f in range(m))
            den += a
            for c in range(v.shape[1]):
                out[i, c] += a * v[j][c]
        out[i] /= den
    return out


@pytest.mark.parametrize("causal", [False, True])
def test_brute_force_tiny(causal):
    rng = np.random.default_rng(21)
    L, d, m, dv = 6, 3, 5, 2
    q = rng.standard_normal((L, d)) * 0.7
    k = rng.standard_normal((L, d)) * 0.7
    v = rng.standard_normal((L, dv))
    w = rng.standard_normal((m, d))
    eps = 0.05
    ref = _brute(q, k, v, w, eps, causal)
    np.testing.assert_allclose(oracle.attn_quadratic(q, k, v, w, eps, causal), ref, rtol=1e-12)
    np.testing.assert_allclose(oracle.attn_rows(q, k, v, w, range(L), eps, causal), ref, rtol=1e-12)
    if causal:
        np.testing.assert_allclose(oracle.attn_causal(q, k, v, w, eps), ref, rtol=1e-12)
    else:
        np.testing.assert_allclose(oracle.attn_noncausal(q, k, v, w, eps), ref, rtol=1e-12)


def test_reassociation_equals_quadratic():
    """(AB)C = A(BC): the m x d state order equals the L x L order (P2 换顺序)."""
    rng = np.random.default_rng(22)
    L, d, m = 64, 16, 128
    q = rng.standard_normal((L, d)) * d ** -0.25
    k = rng.standard_normal((L, d)) * d ** -0.25
    v = rng.standard_normal((L, d))
    w = synth.orthogonal_projection(rng, 1, m, d)[0]
    np.testing.assert_allclose(oracle.attn_noncausal(q, k, v, w), oracle.attn_quadratic(q, k, v, w),
                               rtol=1e-11, atol=1e-13)


def test_causal_prefix_sum_equals_masked_quadratic():
    """Running S_i (P2 案例 2) equals the j <= i masked L x L form."""
    rng = np.random.default_rng(23)
    L, d, m = 64, 16, 128
    q = rng.standard_normal((L, d)) * d ** -0.25
    k = rng.standard_normal((L, d)) * d ** -0.25
    v = rng.standard_normal((L, d))
    w = synth.orthogonal_projection(rng, 1, m, d)[0]
    ref = oracle.attn_quadratic(q, k, v, w, causal=True)
    np.testing.assert_allclose(oracle.attn_causal(q, k, v, w), ref, rtol=1e-11, atol=1e-13)
    rows = [0, 1, 17, 63]
    np.testing.assert_allclose(oracle.attn_rows(q, k, v, w, rows, causal=True), ref[rows], rtol=1e-11)


def test_causal_mask_is_inclusive_and_last_row_is_noncausal():
    rng = np.random.default_rng(24)
    L, d, m = 9, 4, 8
    q = rng.standard_normal((L, d))
    k = rng.standard_normal((L, d))
    v = rng.standard_normal((L, d))
    w = rng.standard_normal((m, d))
    eps = 0.1
    c = oracle.attn_causal(q, k, v, w, eps)
    n = oracle.attn_noncausal(q, k, v, w, eps)
    np.testing.assert_allclose(c[-1], n[-1], rtol=1e-12)
    a00 = oracle.favor_features(q[:1], w)[0] @ oracle.favor_features(k[:1], w)[0]
    np.testing.assert_allclose(c[0], v[0] * a00 / (a00 + eps), rtol=1e-12)


def test_zero_projection_closed_form():
    """W = 0 makes phi(x) = exp(-|x|^2/2)/sqrt(m) in every coordinate, so the
    output is a fixed weighted mean with weights exp(-|k_j|^2/2)."""
    rng = np.random.default_rng(25)
    L, d, m = 10, 5, 7
    q = rng.standard_normal((L, d))
    k = rng.standard_normal((L, d))
    v = rng.standard_normal((L, 3))
    w = np.zeros((m, d))
    eps = 0.01
    gq = np.exp(-0.5 * (q * q).sum(1))
    gk = np.exp(-0.5 * (k * k).sum(1))
    # phi(q).phi(k) = m * gq*gk/m = gq*gk
    num = gq[:, None] * (gk @ v)[None, :]
    den = gq * gk.sum() + eps
    np.testing.assert_allclose(oracle.attn_noncausal(q, k, v, w, eps), num / den[:, None], rtol=1e-12)
    cum_v = np.cumsum(gk[:, None] * v, axis=0)
    cum_g = np.cumsum(gk)
    ref_c = gq[:, None] * cum_v / (gq * cum_g + eps)[:, None]
    np.testing.assert_allclose(oracle.attn_causal(q, k, v, w, eps), ref_c, rtol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_constant_values_expose_eps_placement(causal):
    """V = 1 gives O = den/(den + eps) in every column: eps sits in the
    denominator only (P1 In[25])."""
    rng = np.random.default_rng(26)
    L, d, m = 12, 4, 16
    q = rng.standard_normal((L, d))
    k = rng.standard_normal((L, d))
    w = rng.standard_normal((m, d))
    eps = 0.5
    fq = oracle.favor_features(q, w)
    fk = oracle.favor_features(k, w)
    a = fq @ fk.T
    if causal:
        a = np.tril(a)
    den = a.sum(1)
    fn = oracle.attn_causal if causal else oracle.attn_noncausal
    out = fn(q, k, np.ones((L, 2)), w, eps)
    np.testing.assert_allclose(out, np.repeat((den / (den + eps))[:, None], 2, 1), rtol=1e-12)


def test_single_token():
    rng = np.random.default_rng(27)
    q = rng.standard_normal((1, 8))
    k = rng.standard_normal((1, 8))
    v = rng.standard_normal((1, 8))
    w = rng.standard_normal((32, 8))
    a = oracle.favor_features(q, w)[0] @ oracle.favor_features(k, w)[0]
    for out in (oracle.attn_noncausal(q, k, v, w), oracle.attn_causal(q, k, v, w)):
        np.testing.assert_allclose(out[0], v[0] * a / (a + 1e-6), rtol=1e-12)


def test_key_value_permutation_invariance_noncausal():
    rng = np.random.default_rng(28)
    L, d, m = 20, 6, 12
    q = rng.standard_normal((L, d))
    k = rng.standard_normal((L, d))
    v = rng.standard_normal((L, d))
    w = rng.standard_normal((m, d))
    p = rng.permutation(L)
    np.testing.assert_allclose(oracle.attn_noncausal(q, k[p], v[p], w), oracle.attn_noncausal(q, k, v, w),
                               rtol=1e-12)


def test_projection_is_used_row_wise():
    """Swapping two rows of W (features) leaves attention unchanged, but
    replacing W by a matrix with the same entries transposed does not: pins
    the (m, d) orientation of W."""
    rng = np.random.default_rng(29)
    L, d = 8, 6
    q = rng.standard_normal((L, d))
    k = rng.standard_normal((L, d))
    v = rng.standard_normal((L, d))
    w = rng.standard_normal((d, d))
    p = rng.permutation(d)
    base = oracle.attn_noncausal(q, k, v, w)
    np.testing.assert_allclose(oracle.attn_noncausal(q, k, v, w[p]), base, rtol=1e-12)
    assert not np.allclose(oracle.attn_noncausal(q, k, v, w.T), base, rtol=1e-3)


# ---------------------------------------------------------------------------
# 4. the page code's large-m limit (why the printed table plateaus)
# ---------------------------------------------------------------------------

def test_page_projection_limit_is_not_softmax():
    """With rows drawn as N(0, I/d) (the page code's randn/sqrt(d)), the
    expectation of phi(q).phi(k) is exp(q.k/d - (1-1/d)(|q|^2+|k|^2)/2); after
    row normalisation the |q|^2 term cancels.  At large m the oracle's output
    approaches attention under that kernel, not softmax: this is why the
    printed cosine does not approach 1 as m grows."""
    q, k, v = (x.astype(np.float64) for x in synth.t1_qkv())
    d = 32
    m = 32768
    w = np.random.default_rng(30).standard_normal((m, d)) / math.sqrt(d)
    out = oracle.attn_noncausal(q, k, v, w)
    s = q @ k.T / d - (1 - 1 / d) * 0.5 * (k * k).sum(1)[None, :]
    p = np.exp(s - s.max(1, keepdims=True))
    limit = (p / p.sum(1, keepdims=True)) @ v
    gap_limit = np.abs(out - limit).max()
    gap_softmax = np.abs(out - oracle.softmax_attention(q, k, v, 1 / math.sqrt(d))).max()
    assert gap_limit < 3e-3
    assert gap_softmax > 20 * gap_limit


# ---------------------------------------------------------------------------
# 5. the exact softmax reference
# ---------------------------------------------------------------------------

def test_softmax_reference_invariants():
    rng = np.random.default_rng(31)
    L, d = 7, 4
    q = rng.standard_normal((L, d))
    k = rng.standard_normal((L, d))
    eye = np.eye(L)
    wts = oracle.softmax_attention(q, k, eye, scale=0.7)     # rows are the weights
    np.testing.assert_allclose(wts.sum(1), 1.0, rtol=1e-14)
    s = 0.7 * q @ k.T
    # ratio of weights equals exp of score difference
    np.testing.assert_allclose(wts[:, 1] / wts[:, 0], np.exp(s[:, 1] - s[:, 0]), rtol=1e-12)
    v = rng.standard_normal((L, 3))
    np.testing.assert_allclose(oracle.softmax_attention(q, k, v, scale=0.0), np.repeat(v.mean(0)[None], L, 0),
                               rtol=1e-13)


def test_causal_softmax_brute_force_and_invariants():
    """Masked softmax written out entry by entry; row 0 is v_0; the last row
    is the unmasked one; with scale 0 row i is the mean of v_0..v_i."""
    rng = np.random.default_rng(32)
    L, d = 6, 3
    q = rng.standard_normal((L, d))
    k = rng.standard_normal((L, d))
    v = rng.standard_normal((L, 2))
    got = oracle.softmax_attention(q, k, v, scale=0.5, causal=True)
    for i in range(L):
        e = [math.exp(0.5 * sum(q[i][c] * k[j][c] for c in range(d))) for j in range(i + 1)]
        ref = sum(e[j] * v[j] for j in range(i + 1)) / sum(e)
        np.testing.assert_allclose(got[i], ref, rtol=1e-13)
    np.testing.assert_allclose(got[0], v[0], rtol=1e-15)
    np.testing.assert_allclose(got[-1], oracle.softmax_attention(q, k, v, scale=0.5)[-1], rtol=1e-13)
    mean = oracle.softmax_attention(q, k, v, scale=0.0, causal=True)
    np.testing.assert_allclose(mean, np.cumsum(v, 0) / np.arange(1, L + 1)[:, None], rtol=1e-13)


def test_per_head_uses_the_right_projection():
    rng = np.random.default_rng(32)
    B, H, L, d, m = 2, 3, 5, 4, 8
    q = rng.standard_normal((B, H, L, d))
    k = rng.standard_normal((B, H, L, d))
    v = rng.standard_normal((B, H, L, d))
    w = rng.standard_normal((H, m, d))
    out = oracle.per_head(oracle.attn_noncausal, q, k, v, w)
    np.testing.assert_allclose(out[1, 2], oracle.attn_noncausal(q[1, 2], k[1, 2], v[1, 2], w[2]), rtol=1e-14)
    shared = oracle.per_head(oracle.attn_noncausal, q, k, v, w[:1])
    np.testing.assert_allclose(shared[1, 2], oracle.attn_noncausal(q[1, 2], k[1, 2], v[1, 2], w[0]), rtol=1e-14)
