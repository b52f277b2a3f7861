"""GPU parity of the backward pass (gradients of sum(G * O) with respect to
Q, K, V) against the float64 oracle's gradients on the same seeded inputs,
W and upstream gradient G, with the tolerances of the forward (1e-4
float32, 2e-2 bfloat16) on the per-row metric of _util.grad_err: each row
relative to its own size, except that dQ rows smaller than 1/128 of their
head's largest row are measured against that floor (dQ is formed from a
per-feature difference that nearly cancels in some rows; see grad_err)."""
import numpy as np
import pytest

import oracle
import synth
from _util import TOL, grad_err, row_rel_err, to_device, to_f64

pytestmark = pytest.mark.gpu


def _case(seed, B, H, L, d, m, dtype, heads_w=None, eps=1e-6):
    import torch
    x = synth.random_case(seed, B, H, L, d, m, dtype, heads_w=heads_w)
    g, g64 = synth.upstream_gradient(seed + 1, (B, H, L, d), dtype)
    dev = [to_device(x[n], dtype) for n in ("q", "k", "v")] + [to_device(g, dtype)]
    w = torch.from_numpy(x["w"]).cuda()
    return x, g64, dev, w


def _check(gpu, seed, B, H, L, d, m, dtype, heads_w=None, eps=1e-6, causal=False):
    import torch
    x, g64, (q, k, v, g), w = _case(seed, B, H, L, d, m, dtype, heads_w)
    print(f"[bwd] causal={causal} {dtype} B={B} H={H} L={L} d={d} m={m} Hw={heads_w}", flush=True)
    dq, dk, dv = gpu.attn_backward(q, k, v, w, g, causal=causal, eps=eps)
    torch.cuda.synchronize()
    fn = oracle.attn_causal_grad if causal else oracle.attn_noncausal_grad
    ref = oracle.per_head_grad(fn, x["q64"], x["k64"], x["v64"], x["w64"], g64, eps=eps)
    errs = [grad_err(to_f64(t), r, floored=name == "dq") for name, t, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref)]
    strict = [row_rel_err(to_f64(t), r) for t, r in zip((dq, dk, dv), ref)]
    print(f"[bwd]   metric {errs}  strict per-row {strict}", flush=True)
    assert max(errs) <= TOL[dtype], dict(zip(("dq", "dk", "dv"), errs))
    return errs


@pytest.mark.parametrize("dtype,d,m,B,H,L", [
    ("bf16", 64, 256, 1, 2, 4096),      # the encoder head shape
    ("bf16", 64, 256, 2, 2, 1000),      # ragged tail
    ("bf16", 64, 32, 1, 2, 333),        # smallest m
    ("bf16", 64, 512, 1, 2, 777),       # several feature groups
    ("bf16", 32, 128, 1, 2, 260),
    ("bf16", 32, 256, 1, 2, 300),       # eight-wave reductions with 64-token tiles at d = 32
    ("bf16", 128, 512, 1, 2, 300),
    ("f32", 32, 256, 1, 2, 500),
    ("f32", 64, 96, 1, 2, 129),
    ("f32", 128, 512, 1, 1, 200),
])
def test_noncausal_backward_parity(gpu, dtype, d, m, B, H, L):
    _check(gpu, 5000 + d + m + L, B, H, L, d, m, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noncausal_backward_one_token(gpu, dtype):
    """L = 1: o = v a/(a + eps) depends on q and k only through eps/a, so
    their gradients are of relative size eps/a next to the terms they are
    computed from.  With eps comparable to a they are well resolved; with a
    tiny eps only dv (= g a/(a + eps)) is meaningful at any finite precision
    and is checked alone."""
    import torch
    _check(gpu, 5050, 1, 2, 1, 64, 256, dtype, eps=1.0)
    x, g64, (q, k, v, g), w = _case(5060, 1, 2, 1, 64, 256, dtype)
    _, _, dv = gpu.attn_backward(q, k, v, w, g)
    torch.cuda.synchronize()
    ref = oracle.per_head_grad(oracle.attn_noncausal_grad, x["q64"], x["k64"], x["v64"], x["w64"], g64)
    assert row_rel_err(to_f64(dv), ref[2]) <= TOL[dtype]


def test_noncausal_backward_shared_projection(gpu):
    _check(gpu, 5100, 2, 3, 300, 64, 256, "bf16", heads_w=1)


def test_noncausal_backward_large_eps(gpu):
    """A large eps makes the query side's eps term (s eps / D^2) visible."""
    _check(gpu, 5200, 1, 2, 200, 64, 128, "f32", eps=5.0)


def test_noncausal_backward_deterministic(gpu):
    import torch
    _, _, (q, k, v, g), w = _case(5300, 1, 4, 2048, 64, 256, "bf16")
    first = gpu.attn_backward(q, k, v, w, g)
    for _ in range(3):
        again = gpu.attn_backward(q, k, v, w, g)
        assert all(torch.equal(a, b) for a, b in zip(first, again))


def test_noncausal_backward_long_sampled(gpu):
    """The long workload's shape (B=1, H=8, L=65536, d=64, m=256, bf16) with
    a seeded upstream gradient; two heads are checked in full against the
    oracle (float64 over all 65536 tokens)."""
    import torch
    wl = synth.WORKLOADS["long"]
    x = synth.make_inputs(wl, with64=False)
    g, _ = synth.upstream_gradient(7004, (wl.B, wl.H, wl.L, wl.d), "bf16")
    q, k, v, gd = (to_device(a, "bf16") for a in (x["q"], x["k"], x["v"], g))
    dq, dk, dv = gpu.attn_backward(q, k, v, torch.from_numpy(x["w"]).cuda(), gd)
    torch.cuda.synchronize()
    for h in (0, wl.H - 1):
        q64, k64, v64, g64 = (synth.as_f64(a[0, h], "bf16") for a in (x["q"], x["k"], x["v"], g))
        ref = oracle.attn_noncausal_grad(q64, k64, v64, x["w64"][h], g64, wl.eps)
        errs = [grad_err(to_f64(t[0, h]), r, floored=name == "dq")
                for name, t, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref)]
        print(f"[bwd]   metric {errs}", flush=True)
        assert max(errs) <= TOL["bf16"]


# ---------------------------------------------------------------------------
# causal
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,d,m,B,H,L", [
    ("bf16", 64, 256, 1, 2, 32),        # one chunk
    ("bf16", 64, 256, 1, 2, 100),       # ragged last chunk
    ("bf16", 64, 256, 1, 2, 1000),      # several spans and chunks
    ("bf16", 64, 256, 2, 2, 4096),
    ("bf16", 64, 32, 2, 1, 300),        # smallest m
    ("bf16", 64, 512, 1, 1, 257),       # four feature groups
    ("bf16", 32, 128, 1, 2, 333),
    ("bf16", 32, 256, 1, 2, 1000),      # fused query walk and eight-wave reductions at d = 32
    ("bf16", 128, 256, 1, 1, 200),
    ("f32", 32, 256, 1, 1, 200),
    ("f32", 64, 96, 1, 2, 130),
    ("f32", 128, 128, 1, 1, 150),
])
def test_causal_backward_parity(gpu, dtype, d, m, B, H, L):
    _check(gpu, 6000 + d + m + L, B, H, L, d, m, dtype, causal=True)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype,d,m,L,heads_w", [
    ("bf16", 64, 100, 300, None),
    ("bf16", 32, 40, 130, None),
    ("bf16", 64, 200, 257, 1),          # one W for both heads
    ("f32", 64, 33, 129, None),
    ("f32", 128, 250, 100, None),
])
def test_backward_ragged_feature_count(gpu, causal, dtype, d, m, L, heads_w):
    """m not a multiple of 32: the padding features of the last 32-feature
    block are zero in every backward kernel (phi of rows past m), the padded
    W operands are zero there, and 1/sqrt(m) uses the true m."""
    _check(gpu, 7000 + d + m + L, 1, 2, L, d, m, dtype, heads_w=heads_w, causal=causal)


def test_causal_backward_shared_projection_and_large_eps(gpu):
    _check(gpu, 6100, 1, 3, 300, 64, 256, "bf16", heads_w=1, causal=True)
    _check(gpu, 6101, 1, 2, 200, 64, 128, "f32", eps=5.0, causal=True)


def test_causal_backward_one_token(gpu):
    """L = 1 equals the non-causal case; see test_noncausal_backward_one_token."""
    _check(gpu, 6150, 1, 2, 1, 64, 256, "f32", eps=1.0, causal=True)


def test_causal_backward_deterministic(gpu):
    import torch
    _, _, (q, k, v, g), w = _case(6200, 1, 4, 2048, 64, 256, "bf16")
    first = gpu.attn_backward(q, k, v, w, g, causal=True)
    for _ in range(3):
        again = gpu.attn_backward(q, k, v, w, g, causal=True)
        assert all(torch.equal(a, b) for a, b in zip(first, again))


def test_causal_backward_long_full_heads(gpu):
    """The long workload's shape (B=1, H=8, L=65536, d=64, m=256, bf16) in the
    benchmark's launch configuration; two heads are checked in full against
    the oracle's per-token recurrences."""
    import torch
    wl = synth.WORKLOADS["long"]
    x = synth.make_inputs(wl, with64=False)
    g, _ = synth.upstream_gradient(wl.seed_data + 6000, (wl.B, wl.H, wl.L, wl.d), "bf16")
    q, k, v, gd = (to_device(a, "bf16") for a in (x["q"], x["k"], x["v"], g))
    dq, dk, dv = gpu.attn_backward(q, k, v, torch.from_numpy(x["w"]).cuda(), gd, causal=True)
    torch.cuda.synchronize()
    for h in (0, wl.H - 1):
        print(f"[bwd] long causal head {h}", flush=True)
        q64, k64, v64, g64 = (synth.as_f64(a[0, h], "bf16") for a in (x["q"], x["k"], x["v"], g))
        ref = oracle.attn_causal_grad(q64, k64, v64, x["w64"][h], g64, wl.eps)
        errs = [grad_err(to_f64(t[0, h]), r, floored=name == "dq")
                for name, t, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref)]
        print(f"[bwd]   metric {errs}", flush=True)
        assert max(errs) <= TOL["bf16"]
