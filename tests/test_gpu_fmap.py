"""GPU parity of the feature-map variants ("Linear Attention > Kernel Feature
Maps", sections 1-3: ELU + 1, ReLU, random Fourier features) against the
float64 oracle, non-causal and causal, with the forward's per-row metric and
tolerances (1e-4 float32, 2e-2 bfloat16).

Inputs follow the encoder recipe; for the trig map Q and K are scaled by
0.15 instead of d^-1/4, so that the Gaussian kernel it estimates,
exp(-|q-k|^2/2), stays well above the estimator's noise and the denominators
stay away from zero (the pages warn that trig features make them unstable).
"""
import numpy as np
import pytest

import oracle
import synth
from _util import TOL, row_rel_err, to_device, to_f64

pytestmark = pytest.mark.gpu


def _case(seed, B, H, L, d, m, dtype, kind):
    return synth.random_case(seed, B, H, L, d, m, dtype, qk_scale=0.15 if kind == "trig" else None)


@pytest.mark.parametrize("kind", ["elu1", "relu", "trig"])
@pytest.mark.parametrize("dtype,d,m,L", [("f32", 32, 64, 70), ("f32", 64, 128, 129), ("bf16", 64, 256, 200),
                                         ("bf16", 128, 64, 33)])
def test_features_variants(gpu, kind, dtype, d, m, L):
    import torch
    x = _case(8000 + d + m, 1, 2, L, d, m, dtype, kind)
    print(f"[fmap] features {kind} {dtype} d={d} m={m} L={L}", flush=True)
    phi = to_f64(gpu.features(to_device(x["q"], dtype), torch.from_numpy(x["w"]).cuda(), fmap=kind))
    ref = np.stack([oracle.feature_map(x["q64"][0, h], x["w64"][h], kind) for h in range(2)])[None]
    assert phi.shape == ref.shape
    # absolute error against each row's largest feature (ReLU and trig
    # features cross or touch zero, so elementwise relative error is ill-posed)
    tol = 1e-4 if dtype == "f32" else 2e-2
    assert row_rel_err(phi, ref) <= tol


@pytest.mark.parametrize("kind", ["elu1", "relu", "trig"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype,d,m,B,H,L", [
    ("bf16", 64, 256, 1, 2, 1000),      # ragged tail, several spans
    ("bf16", 32, 128, 2, 1, 300),
    ("bf16", 128, 256, 1, 1, 257),
    ("f32", 64, 96, 1, 2, 130),
    ("f32", 32, 256, 1, 1, 200),
])
def test_attention_variants(gpu, kind, causal, dtype, d, m, B, H, L):
    import torch
    x = _case(9000 + d + m + L, B, H, L, d, m, dtype, kind)
    print(f"[fmap] attn {kind} causal={causal} {dtype} B={B} H={H} L={L} d={d} m={m}", flush=True)
    q, k, v = (to_device(x[n], dtype) for n in ("q", "k", "v"))
    o = gpu.attn(q, k, v, torch.from_numpy(x["w"]).cuda(), causal=causal, fmap=kind)
    torch.cuda.synchronize()
    fn = oracle.attn_causal if causal else oracle.attn_noncausal
    ref = oracle.per_head(fn, x["q64"], x["k64"], x["v64"], x["w64"], kind=kind)
    err = row_rel_err(to_f64(o), ref)
    print(f"[fmap]   err {err:.3g}", flush=True)
    assert err <= TOL[dtype]


def test_identity_projection_elu_matches_the_page_map(gpu):
    """With W = I (m = d) the ELU+1 map acts on q and k themselves, as the
    page writes it."""
    import torch
    x = synth.random_case(9500, 1, 1, 256, 32, 32, "f32")
    eye = np.eye(32, dtype=np.float32)[None]
    q, k, v = (to_device(x[n], "f32") for n in ("q", "k", "v"))
    o = gpu.attn(q, k, v, torch.from_numpy(eye).cuda(), fmap="elu1")
    torch.cuda.synchronize()
    ref = oracle.attn_noncausal(x["q64"][0, 0], x["k64"][0, 0], x["v64"][0, 0], np.eye(32), kind="elu1")
    assert row_rel_err(to_f64(o)[0, 0], ref) <= TOL["f32"]


def test_long_shape_variants_sampled(gpu):
    """The long workload's shape (B=1, H=8, L=65536, d=64, m=256, bf16) with
    each map, both paths; sampled rows of two heads against the oracle's
    per-row definition."""
    import torch
    wl = synth.WORKLOADS["long"]
    rng = np.random.default_rng(3)
    for kind in ("elu1", "relu", "trig"):
        x = synth.random_case(9600, 1, 2, wl.L, wl.d, wl.m, "bf16", qk_scale=0.15 if kind == "trig" else None)
        q, k, v = (to_device(x[n], "bf16") for n in ("q", "k", "v"))
        w = torch.from_numpy(x["w"]).cuda()
        for causal in (False, True):
            print(f"[fmap] long {kind} causal={causal}", flush=True)
            o = gpu.attn(q, k, v, w, causal=causal, fmap=kind)
            torch.cuda.synchronize()
            for h in range(2):
                rows = np.unique(np.concatenate([[0, 1, 1023, 1024, wl.L - 1], rng.choice(wl.L, 12, replace=False)]))
                ref = oracle.attn_rows(x["q64"][0, h], x["k64"][0, h], x["v64"][0, h], x["w64"][h], rows,
                                       causal=causal, kind=kind)
                got = o[0, h, torch.from_numpy(rows).cuda()].float().cpu().numpy().astype(np.float64)
                assert row_rel_err(got, ref) <= TOL["bf16"]
