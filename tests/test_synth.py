"""Pins of the seeded input generators: orthogonal projection rows, their
chi(d) lengths, bf16 round-to-nearest-even and determinism."""
import numpy as np
import pytest

import synth


def test_orthogonal_blocks_are_orthogonal():
    """Rows inside each d-row block are mutually orthogonal (P2 key points:
    the sampled projection vectors are made mutually orthogonal)."""
    rng = np.random.default_rng(1)
    d, m = 16, 40                      # 3 blocks, the last one partial
    w = synth.orthogonal_projection(rng, 2, m, d)
    for h in range(2):
        for b0 in range(0, m, d):
            blk = w[h, b0:b0 + d]
            g = blk @ blk.T
            off = g - np.diag(np.diag(g))
            assert np.abs(off).max() < 1e-12 * np.abs(np.diag(g)).max()
        # rows of different blocks are generally not orthogonal
        cross = w[h, :d] @ w[h, d:2 * d].T
        assert np.abs(cross).max() > 1e-3


def test_orthogonality_survives_float32_storage():
    rng = np.random.default_rng(2)
    w = synth.orthogonal_projection(rng, 1, 64, 64)[0].astype(np.float32).astype(np.float64)
    g = w @ w.T
    off = g - np.diag(np.diag(g))
    assert np.abs(off).max() < 1e-5 * np.diag(g).max()


def test_row_lengths_are_chi_d():
    """Squared row lengths have mean d and variance 2d (chi-square with d
    degrees of freedom), so each row is marginally N(0, I_d)."""
    rng = np.random.default_rng(3)
    d = 8
    w = synth.orthogonal_projection(rng, 200, 64, d)
    sq = (w ** 2).sum(-1).ravel()
    n = sq.size
    assert abs(sq.mean() - d) < 5 * np.sqrt(2 * d / n)
    assert sq.var() == pytest.approx(2 * d, rel=0.08)


def test_rows_marginally_standard_normal():
    rng = np.random.default_rng(4)
    d = 8
    w = synth.orthogonal_projection(rng, 400, 16, d).reshape(-1, d)
    cov = w.T @ w / w.shape[0]
    np.testing.assert_allclose(cov, np.eye(d), atol=0.05)


def test_samplers_are_deterministic():
    a = synth.orthogonal_projection(np.random.default_rng(9), 2, 32, 8)
    b = synth.orthogonal_projection(np.random.default_rng(9), 2, 32, 8)
    np.testing.assert_array_equal(a, b)
    x = synth.make_inputs(synth.WORKLOADS["encoder"], B=1, H=1, L=8)
    y = synth.make_inputs(synth.WORKLOADS["encoder"], B=1, H=1, L=8)
    for key in ("q", "k", "v", "w"):
        np.testing.assert_array_equal(x[key], y[key])


@pytest.mark.parametrize("value,bits", [
    (1.0, 0x3F80),
    (-2.0, 0xC000),
    (1.0 + 2 ** -8, 0x3F80),           # tie, rounds to even (down)
    (1.0 + 3 * 2 ** -8, 0x3F82),       # tie, rounds to even (up)
    (1.0 + 2 ** -8 + 2 ** -20, 0x3F81),  # just above the tie
    (0.0, 0x0000),
    (-0.0, 0x8000),
])
def test_bf16_round_nearest_even(value, bits):
    assert int(synth.bf16_round(np.array([value], dtype=np.float32))[0]) == bits


def test_bf16_roundtrip_error_bound():
    rng = np.random.default_rng(5)
    x = rng.standard_normal(10000).astype(np.float32)
    y = synth.bf16_bits_to_f32(synth.bf16_round(x))
    rel = np.abs(y - x) / np.abs(x)
    assert rel.max() <= 2.0 ** -8 + 1e-12


def test_workload_shapes_and_value_recipe():
    wl = synth.WORKLOADS["wide"]
    x = synth.make_inputs(wl, B=1, H=2, L=512)
    assert x["q"].dtype == np.float32 and x["q"].shape == (1, 2, 512, 128)
    assert x["w"].shape == (2, 512, 128)
    # Q, K entries are 0.5 * N(0,1) * 128^-1/4
    assert x["q"].std() == pytest.approx(0.5 * 128 ** -0.25, rel=0.03)
    assert x["v"].std() == pytest.approx(1.0, rel=0.03)
    e = synth.make_inputs(synth.WORKLOADS["encoder"], B=1, H=1, L=256)
    assert e["q"].dtype == np.uint16
    assert e["q64"].std() == pytest.approx(64 ** -0.25, rel=0.05)
    t = synth.make_inputs(synth.WORKLOADS["t1"])
    assert t["q"].shape == (1, 1, 64, 32) and t["w"].shape == (1, 256, 32)
