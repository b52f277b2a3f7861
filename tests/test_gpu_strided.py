"""GPU parity of favor_attn_strided: token-major [B, L, H, d] layouts and
value widths d_v != d (the page's code cell allows d_v != d_k), against the
float64 oracle, which takes V of any width."""
import numpy as np
import pytest

import oracle
import synth
from _util import TOL, row_rel_err, to_device, to_f64

pytestmark = pytest.mark.gpu


def _token_major(t):
    """A [B, H, L, d] tensor re-laid out as [B, L, H, d] memory, returned as
    the [B, H, L, d] view of it."""
    return t.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype,d,dv,m,B,H,L,layout", [
    ("bf16", 64, 64, 256, 2, 3, 300, "token"),     # same width, token-major
    ("bf16", 64, 96, 256, 1, 2, 200, "head"),      # wider values, contiguous
    ("bf16", 64, 16, 128, 1, 2, 130, "token"),     # narrower values
    ("bf16", 32, 200, 64, 1, 1, 257, "token"),     # several chunks, ragged last one
    ("f32", 64, 96, 96, 1, 2, 100, "token"),
    ("f32", 128, 40, 128, 1, 1, 70, "head"),
])
def test_strided_parity(gpu, causal, dtype, d, dv, m, B, H, L, layout):
    import torch
    x = synth.random_case(7500 + d + dv + L, B, H, L, d, m, dtype)
    vx = synth.random_case(7600 + dv, B, H, L, dv, 32, dtype)     # values of width dv
    print(f"[strided] causal={causal} {dtype} d={d} dv={dv} m={m} L={L} {layout}", flush=True)
    q, k = (to_device(x[n], dtype) for n in ("q", "k"))
    v = to_device(vx["v"], dtype)
    out = torch.empty((B, L, H, dv), dtype=q.dtype, device=q.device).permute(0, 2, 1, 3)
    if layout == "token":
        q, k, v = _token_major(q), _token_major(k), _token_major(v)
    else:
        out = out.contiguous()
    w = torch.from_numpy(x["w"]).cuda()
    o = gpu.attn_strided(q, k, v, w, causal=causal, out=out)
    torch.cuda.synchronize()
    fn = oracle.attn_causal if causal else oracle.attn_noncausal
    ref = oracle.per_head(fn, x["q64"], x["k64"], vx["v64"], x["w64"])
    assert row_rel_err(to_f64(o), ref) <= TOL[dtype]


def test_strided_same_layout_matches_contiguous_call(gpu):
    """Contiguous tensors of equal widths take the direct path: identical
    results to favor_attn."""
    import torch
    x = synth.random_case(7700, 1, 2, 500, 64, 256, "bf16")
    q, k, v = (to_device(x[n], "bf16") for n in ("q", "k", "v"))
    w = torch.from_numpy(x["w"]).cuda()
    for causal in (False, True):
        assert torch.equal(gpu.attn_strided(q, k, v, w, causal=causal), gpu.attn(q, k, v, w, causal=causal))


def test_strided_feature_map(gpu):
    import torch
    x = synth.random_case(7800, 1, 2, 150, 64, 128, "f32")
    q, k, v = (_token_major(to_device(x[n], "f32")) for n in ("q", "k", "v"))
    w = torch.from_numpy(x["w"]).cuda()
    o = gpu.attn_strided(q, k, v, w, causal=True, fmap="elu1")
    torch.cuda.synchronize()
    ref = oracle.per_head(oracle.attn_causal, x["q64"], x["k64"], x["v64"], x["w64"], kind="elu1")
    assert row_rel_err(to_f64(o), ref) <= TOL["f32"]
