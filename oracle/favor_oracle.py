"""Float64 CPU oracle for FAVOR+ attention -- TEST INFRASTRUCTURE ONLY.

Only the tests, the package's smoke entry and the benchmark's CPU-baseline leg
may import this module.  The product path (the HIP library and its Python
binding) never calls it and shares no code with it.

Everything here is plain NumPy in float64, written from the three source pages:

* "Linear Attention > Performer: Unbiased Softmax Approximation" (P1): the
  feature-map equation, the code cell In[25] (feature map and reassociated
  attention) and the experiment of In[26] / Out[27].
* "Performer -- 用随机特征把 softmax attention 拉成线性复杂度" (P2, study notes on
  performer-2020): section 核心要点 (key points: kernel view, reordering,
  linearised denominator), the 换顺序 diagram and 案例 2 (causal prefix sum).
* "Linear Attention > Kernel Feature Maps" (P3): the softmax-kernel equation
  and section 4, positive random features; sections 1-3 (ELU + 1, ReLU,
  random Fourier features) for the feature-map variants.

Conventions: X is (L, d) per head, the projection W is (m, d) with rows
omega_i, and every function takes the values actually handed to the device,
upcast to float64.  No stabiliser, no 1/sqrt(d) temperature and no rescaling
of eps are applied: the caller pre-scales Q and K if it wants a temperature.

Readings of points the pages leave open:
* causal denominator = phi(q_i) . sum_{j<=i} phi(k_j) + eps, by analogy with
  the non-causal denominator (P2 key points; P1 In[25]);
* the causal sum includes the diagonal j = i (P2 案例 2 says j <= i);
* eps is added after the dot product and never to the numerator (P1 In[25]);
* the 1/sqrt(m) factor is kept (P1 feature-map equation, P3 section 4).

Pins: tests/test_oracle_pins.py checks every function here against the worked
example's printed table, closed forms, Monte-Carlo moments and brute force.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "favor_features", "feature_map", "FEATURE_MAPS", "attn_quadratic", "attn_noncausal", "attn_causal",
    "attn_rows", "softmax_attention", "per_head", "head_projection",
    "favor_features_vjp", "attn_noncausal_grad", "attn_causal_grad", "per_head_grad",
]


def favor_features(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Positive random features, phi(x) = exp(-|x|^2/2) / sqrt(m) *
    [exp(omega_1 . x), ..., exp(omega_m . x)].

    Written in the general form of P3 section 4 (and P1's feature-map
    equation), phi(x) = h(x)/sqrt(m) (f(omega_1 . x), ..., f(omega_m . x))
    with h(x) = exp(-|x|^2/2) and f = exp, evaluated in the log domain so
    that h and f never overflow separately: log phi_i = log h(x) +
    omega_i . x - log(m)/2.  x: (..., d), w: (m, d).  Returns (..., m) float64.
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    log_h = -0.5 * np.einsum("...d,...d->...", x, x)            # log h(x)
    log_f = np.einsum("...d,md->...m", x, w)                    # log f(omega_i . x) = omega_i . x
    return np.exp(log_h[..., None] + log_f - 0.5 * np.log(w.shape[0]))


FEATURE_MAPS = ("positive", "elu1", "relu", "trig")


def feature_map(x: np.ndarray, w: np.ndarray, kind: str = "positive") -> np.ndarray:
    """The feature maps of P3 (sections 1-4), each applied to the projection
    p = x W^T (rows omega_i of W; with W the identity, m = d, the first two
    act on x itself as the page writes them):

    * "positive": FAVOR+ positive random features (favor_features);
    * "elu1": ELU(p) + 1, i.e. p + 1 where p > 0 and exp(p) where p <= 0;
    * "relu": max(0, p);
    * "trig": random Fourier features, 2m outputs
      (1/sqrt(m)) [sin(omega_1.x), cos(omega_1.x), ..., sin(omega_m.x), cos(omega_m.x)].

    x: (..., d), w: (m, d).  Returns (..., m) or, for "trig", (..., 2m) float64.
    """
    if kind == "positive":
        return favor_features(x, w)
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    p = x @ w.T
    if kind == "elu1":
        return np.where(p > 0, p + 1.0, np.exp(np.minimum(p, 0.0)))
    if kind == "relu":
        return np.maximum(p, 0.0)
    if kind == "trig":
        out = np.empty(p.shape[:-1] + (2 * p.shape[-1],))
        out[..., 0::2] = np.sin(p)
        out[..., 1::2] = np.cos(p)
        return out / np.sqrt(w.shape[0])
    raise ValueError(f"unknown feature map {kind!r}")


def attn_quadratic(q, k, v, w, eps: float = 1e-6, causal: bool = False, kind: str = "positive") -> np.ndarray:
    """The definition: A = phi(Q) phi(K)^T (an L x L matrix of kernel
    estimates), optionally masked to keys j <= query i, then
    O = (A V) / (A 1 + eps) row by row.

    This is the left-to-right product order of the 换顺序 diagram in P2 (the
    order FAVOR+ avoids), with the normaliser of P2's key points; `kind`
    selects the feature map (feature_map).
    """
    fq = feature_map(q, w, kind)
    fk = feature_map(k, w, kind)
    a = fq @ fk.T
    if causal:
        a = np.tril(a)
    num = a @ np.asarray(v, dtype=np.float64)
    den = a.sum(axis=1) + eps
    return num / den[:, None]


def attn_noncausal(q, k, v, w, eps: float = 1e-6, kind: str = "positive") -> np.ndarray:
    """Reassociated non-causal attention, the right-hand side of P2's 换顺序
    diagram: phi(K)^T is contracted once with the values augmented by a
    column of ones, [V | 1], giving the m x (d+1) block [M | z] (the state
    M = phi(K)^T V and the key sum z = phi(K)^T 1 of P2's key points); then
    phi(Q) [M | z] holds the numerators in its first d columns and the
    normaliser phi(Q) z in its last, and O = numerator / (normaliser + eps)."""
    fq = feature_map(q, w, kind)
    fk = feature_map(k, w, kind)
    v = np.asarray(v, dtype=np.float64)
    v_aug = np.concatenate([v, np.ones((v.shape[0], 1))], axis=1)      # [V | 1]
    r = fq @ (fk.T @ v_aug)                                           # phi(Q) [M | z]
    return r[:, :-1] / (r[:, -1:] + eps)


def attn_causal(q, k, v, w, eps: float = 1e-6, kind: str = "positive") -> np.ndarray:
    """Causal attention by the running prefix sum of P2 案例 2: walking the
    tokens in order, S_i = S_{i-1} + phi(k_i) v_i^T (an m x d matrix) and
    z_i = z_{i-1} + phi(k_i); the output is
    o_i = phi(q_i)^T S_i / (phi(q_i)^T z_i + eps).

    One Python step per token; O(L m d) time and O(m d) state.
    """
    fq = feature_map(q, w, kind)
    fk = feature_map(k, w, kind)
    v = np.asarray(v, dtype=np.float64)
    L, d = v.shape
    m = fq.shape[1]
    state = np.zeros((m, d))
    key_sum = np.zeros(m)
    out = np.empty((L, d))
    for i in range(L):
        state += np.outer(fk[i], v[i])
        key_sum += fk[i]
        out[i] = (fq[i] @ state) / (fq[i] @ key_sum + eps)
    return out


def attn_rows(q, k, v, w, rows, eps: float = 1e-6, causal: bool = False, kind: str = "positive") -> np.ndarray:
    """Selected output rows by the definition: for each query i,
    a_j = phi(q_i) . phi(k_j) over the keys it sees (all keys, or j <= i when
    causal), o_i = sum_j a_j v_j / (sum_j a_j + eps).

    Used for sampled-row checks at sizes where the full output is too big.
    """
    rows = np.asarray(rows, dtype=np.int64)
    fq = feature_map(np.asarray(q)[rows], w, kind)
    fk = feature_map(k, w, kind)
    v = np.asarray(v, dtype=np.float64)
    out = np.empty((len(rows), v.shape[1]))
    for r, i in enumerate(rows):
        seen = slice(0, i + 1) if causal else slice(None)
        a = fk[seen] @ fq[r]
        out[r] = (a @ v[seen]) / (a.sum() + eps)
    return out


def softmax_attention(q, k, v, scale: float = 1.0, causal: bool = False) -> np.ndarray:
    """Exact attention softmax(scale * Q K^T) V, the quantity the random
    features estimate (P3's softmax-kernel equation; P2 key points write the
    weights with a 1/sqrt(d) temperature), optionally masked to keys j <= i
    (the mask P2 案例 2 describes).  The row maximum is subtracted before
    exponentiating, which leaves the softmax unchanged."""
    s = scale * (np.asarray(q, dtype=np.float64) @ np.asarray(k, dtype=np.float64).T)
    if causal:
        s = np.where(np.tril(np.ones(s.shape, dtype=bool)), s, -np.inf)
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=1, keepdims=True)
    return p @ np.asarray(v, dtype=np.float64)


# ---------------------------------------------------------------------------
# Backward pass.  The pages give no formulas for it; they only note (P2,
# section 踩过的坑 / pitfalls) that the causal prefix sum must be accumulated
# in reverse for the gradient.  What is computed is the gradient of the
# forward definition above with respect to Q, K and V for an upstream
# gradient G = dLoss/dO (W is a fixed random projection and gets none),
# written out with the chain rule through the reassociated form.
# ---------------------------------------------------------------------------
def favor_features_vjp(x, w, phi, dphi) -> np.ndarray:
    """dLoss/dx given dLoss/dphi for phi = favor_features(x, w).

    d phi_f / d x = phi_f (omega_f - x)  (differentiating the feature-map
    equation of P1), hence dx = (dphi * phi) W - sum_f(dphi_f phi_f) x."""
    x = np.asarray(x, dtype=np.float64)
    g = np.asarray(dphi, dtype=np.float64) * phi
    return g @ np.asarray(w, dtype=np.float64) - g.sum(axis=-1, keepdims=True) * x


def attn_noncausal_grad(q, k, v, w, g, eps: float = 1e-6):
    """Gradients (dQ, dK, dV) of sum(G * O) for non-causal attention.

    With M = phi(K)^T V, z = phi(K)^T 1, den_i = phi(q_i).z + eps and
    o_i = phi(q_i) M / den_i:
      dnum_i = g_i / den_i,  dden_i = -(g_i . o_i) / den_i,
      dphi(q_i) = M dnum_i + z dden_i,
      dM = phi(Q)^T dnum,  dz = phi(Q)^T dden,
      dV = phi(K) dM,  dphi(k_j) = dM v_j + dz,
    then each feature gradient goes through favor_features_vjp."""
    fq = favor_features(q, w)
    fk = favor_features(k, w)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    state = fk.T @ v
    key_sum = fk.sum(axis=0)
    den = fq @ key_sum + eps
    o = (fq @ state) / den[:, None]
    dnum = g / den[:, None]
    dden = -(g * o).sum(axis=1) / den
    dfq = dnum @ state.T + dden[:, None] * key_sum[None, :]
    dstate = fq.T @ dnum
    dkey_sum = fq.T @ dden
    dv = fk @ dstate
    dfk = v @ dstate.T + dkey_sum[None, :]
    return favor_features_vjp(q, w, fq, dfq), favor_features_vjp(k, w, fk, dfk), dv


def attn_causal_grad(q, k, v, w, g, eps: float = 1e-6):
    """Gradients (dQ, dK, dV) of sum(G * O) for causal attention.

    Forward walk (as attn_causal): S_i, z_i, den_i, o_i, and with them
    dnum_i = g_i / den_i, dden_i = -(g_i . o_i) / den_i and
    dphi(q_i) = S_i dnum_i + z_i dden_i.
    Reverse walk (the reverse accumulation of P2's pitfalls): the suffix sums
    R_j = sum_{i>=j} phi(q_i) dnum_i^T and r_j = sum_{i>=j} phi(q_i) dden_i
    give dv_j = R_j^T phi(k_j) and dphi(k_j) = R_j v_j + r_j.
    One Python step per token in each walk."""
    fq = favor_features(q, w)
    fk = favor_features(k, w)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    L, d = v.shape
    m = fq.shape[1]
    state = np.zeros((m, d))
    key_sum = np.zeros(m)
    dnum = np.empty((L, d))
    dden = np.empty(L)
    dfq = np.empty((L, m))
    for i in range(L):
        state += np.outer(fk[i], v[i])
        key_sum += fk[i]
        den = fq[i] @ key_sum + eps
        o = (fq[i] @ state) / den
        dnum[i] = g[i] / den
        dden[i] = -(g[i] @ o) / den
        dfq[i] = state @ dnum[i] + key_sum * dden[i]
    rstate = np.zeros((m, d))
    rsum = np.zeros(m)
    dv = np.empty((L, d))
    dfk = np.empty((L, m))
    for j in range(L - 1, -1, -1):
        rstate += np.outer(fq[j], dnum[j])
        rsum += fq[j] * dden[j]
        dv[j] = rstate.T @ fk[j]
        dfk[j] = rstate @ v[j] + rsum
    return favor_features_vjp(q, w, fq, dfq), favor_features_vjp(k, w, fk, dfk), dv


def head_projection(w: np.ndarray, h: int) -> np.ndarray:
    """The projection of head h: W is (Hw, m, d) with Hw = 1 (shared by all
    heads) or Hw = H (one per head)."""
    return w[0] if w.shape[0] == 1 else w[h]


def per_head(fn, q, k, v, w, **kw) -> np.ndarray:
    """Apply a single-head function to every (b, h) of [B, H, L, d] inputs."""
    B, H, L, _ = q.shape
    out = np.empty(q.shape[:3] + (v.shape[-1],))
    for b in range(B):
        for h in range(H):
            out[b, h] = fn(q[b, h], k[b, h], v[b, h], head_projection(w, h), **kw)
    return out


def per_head_grad(fn, q, k, v, w, g, **kw):
    """Apply a single-head gradient function to every (b, h); returns
    (dQ, dK, dV) shaped like Q, K, V."""
    B, H, L, _ = q.shape
    dq, dk, dv = np.empty(q.shape), np.empty(k.shape), np.empty(v.shape)
    for b in range(B):
        for h in range(H):
            dq[b, h], dk[b, h], dv[b, h] = fn(q[b, h], k[b, h], v[b, h], head_projection(w, h), g[b, h], **kw)
    return dq, dk, dv
