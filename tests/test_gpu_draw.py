"""GPU parity of the device projection sampler (favor_draw_projection)
against the oracle's sampler (oracle/projection.py), which implements the
same Philox4x64-10 generator, Box-Muller normals and orthogonal blocks in
float64: the device values, rounded to float32, agree to a few float32 ulps
(the orthogonalisation rounds differently: Gram-Schmidt on the device,
Householder in the oracle)."""
import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("seed,Hw,m,d,orth,scale", [
    (1, 1, 32, 32, True, 1.0),
    (12345, 2, 100, 64, True, 1.0),          # m not a multiple of d
    (2 ** 63 + 11, 1, 256, 128, True, 1.0),
    (7, 3, 50, 16, True, 0.25),
    (99, 2, 70, 64, False, 1.0 / 8),         # independent rows, the page code's 1/sqrt(d)
    (5, 1, 1, 5, False, 1.0),
])
def test_draw_matches_oracle(gpu, seed, Hw, m, d, orth, scale):
    import torch
    print(f"[draw] seed={seed} Hw={Hw} m={m} d={d} orth={orth}", flush=True)
    W = gpu.draw_projection(seed, Hw, m, d, orthogonal=orth, scale=scale)
    torch.cuda.synchronize()
    ref = oracle.draw_projection(seed, Hw, m, d, orthogonal=orth, scale=scale)
    got = W.cpu().numpy().astype(np.float64)
    err = np.abs(got - ref).max() / np.abs(ref).max()
    assert err < 2e-6, err


def test_drawn_projection_drives_attention(gpu):
    """A W drawn on the device is an ordinary input: attention with it
    matches the oracle given the same W values."""
    import torch
    import synth
    from _util import TOL, row_rel_err, to_device, to_f64
    x = synth.random_case(4300, 1, 2, 300, 64, 32, "f32")
    W = gpu.draw_projection(4301, 2, 128, 64)
    q, k, v = (to_device(x[n], "f32") for n in ("q", "k", "v"))
    o = gpu.attn(q, k, v, W)
    torch.cuda.synchronize()
    w64 = W.cpu().numpy().astype(np.float64)
    assert np.abs(w64 - oracle.draw_projection(4301, 2, 128, 64)).max() < 1e-5
    ref = oracle.per_head(oracle.attn_noncausal, x["q64"], x["k64"], x["v64"], w64)
    assert row_rel_err(to_f64(o), ref) <= TOL["f32"]
