"""Pins of the oracle's projection sampler (oracle/projection.py): the
Philox4x64-10 generator against NumPy's own Philox bit generator (a library
implementation of the same published generator; NumPy advances its counter
before each block), the Box-Muller normals against their defining transform
and their moments, and the structure of the drawn W (orthogonal blocks,
chi(d) lengths, marginal N(0, I) rows)."""
import math

import numpy as np
import pytest

import oracle


@pytest.mark.parametrize("ctr", [[0, 0, 0, 0], [7, 3, 2, 1], [2 ** 64 - 2, 5, 0, 9]])
@pytest.mark.parametrize("seed", [0, 12345, 2 ** 63 + 11])
def test_philox_matches_numpy(ctr, seed):
    bg = np.random.Philox()
    st = bg.state
    # set the state from exact uint64 arrays (the constructor's conversion
    # of large Python ints is lossy)
    st["state"] = {"counter": np.array(ctr, dtype=np.uint64), "key": np.array([seed, 0], dtype=np.uint64)}
    st["buffer_pos"] = 4
    bg.state = st
    raw = [int(x) for x in bg.random_raw(4)]
    nxt = list(ctr)
    nxt[0] = (nxt[0] + 1) % 2 ** 64
    if nxt[0] == 0:
        nxt[1] += 1
    assert oracle.philox4x64(nxt, [seed, 0]) == raw


def test_normals_follow_box_muller():
    w = oracle.philox4x64([0, 3, 1, 0], [99, 0])
    u = [((x >> 11) + 0.5) * 2.0 ** -53 for x in w]
    z = oracle.philox_normals(99, 1, 0, 3, 4)
    r0, r1 = math.sqrt(-2 * math.log(u[0])), math.sqrt(-2 * math.log(u[2]))
    np.testing.assert_allclose(z, [r0 * math.cos(2 * math.pi * u[1]), r0 * math.sin(2 * math.pi * u[1]),
                                   r1 * math.cos(2 * math.pi * u[3]), r1 * math.sin(2 * math.pi * u[3])], rtol=1e-15)


def test_normal_moments():
    z = np.concatenate([oracle.philox_normals(5, 0, 0, r, 64) for r in range(400)])
    assert abs(z.mean()) < 4 / math.sqrt(len(z))
    assert abs(z.var() - 1) < 0.03
    assert abs((z ** 4).mean() - 3) < 0.15


def test_orthogonal_draw_structure():
    d, m = 8, 20
    W = oracle.draw_projection(7, 2, m, d)
    for h in range(2):
        for b in range(0, m, d):
            blk = W[h, b:b + d]
            g = blk @ blk.T
            off = g - np.diag(np.diag(g))
            assert np.abs(off).max() < 1e-12 * np.abs(np.diag(g)).max()
        # row norms are the chi(d) lengths drawn from purpose 1
        lengths = [np.linalg.norm(oracle.philox_normals(7, h, 1, f, d)) for f in range(m)]
        np.testing.assert_allclose(np.linalg.norm(W[h], axis=1), lengths, rtol=1e-13)
    assert not np.allclose(W[0], W[1])


def test_draws_are_marginally_standard_normal():
    d, m = 16, 64
    W = np.concatenate([oracle.draw_projection(s, 1, m, d)[0] for s in range(40)])
    assert abs(W.mean()) < 0.03
    assert abs(W.var() - 1) < 0.05
    I = oracle.draw_projection(3, 1, 2 * d, d, orthogonal=False, scale=0.5)[0]
    np.testing.assert_allclose(I[0] / 0.5, oracle.philox_normals(3, 0, 0, 0, d), rtol=1e-15)


def test_qr_sign_fix_gives_positive_projections():
    """Row i of a block is column i of Q with R_ii > 0, so it has a positive
    inner product with column i of G after removing the earlier columns: in
    particular row 0 points along G's first column."""
    d = 6
    W = oracle.draw_projection(21, 1, d, d)[0]
    G = np.stack([oracle.philox_normals(21, 0, 0, i, d) for i in range(d)])
    u0 = W[0] / np.linalg.norm(W[0])
    np.testing.assert_allclose(u0, G[:, 0] / np.linalg.norm(G[:, 0]), rtol=1e-12, atol=1e-14)
