"""GPU parity: the HIP library against the float64 oracle on the same seeded
inputs and the same W.

Tolerances (stated for the method's float paths): per-row infinity-norm
relative error <= 1e-4 for float32 inputs and <= 2e-2 for bfloat16 inputs with
float32 accumulation.  Feature values are checked elementwise against a bound
derived from the bf16 rounding of W (see test_features_bf16_within_bound).
"""
import math
import os

import numpy as np
import pytest

import oracle
import synth
from _util import TOL, row_rel_err, to_device, to_f64

pytestmark = pytest.mark.gpu


def _run_attn(favor, x, dtype, causal, eps=1e-6):
    import torch
    q, k, v = (to_device(x[n], dtype) for n in ("q", "k", "v"))
    w = torch.from_numpy(x["w"]).cuda()
    o = favor.attn(q, k, v, w, causal=causal, eps=eps)
    torch.cuda.synchronize()
    return to_f64(o)


def _ref(x, causal, eps=1e-6, heads=None):
    fn = oracle.attn_causal if causal else oracle.attn_noncausal
    return oracle.per_head(fn, x["q64"], x["k64"], x["v64"], x["w64"], eps=eps)


# ---------------------------------------------------------------------------
# feature map
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("d,m,L", [(32, 256, 64), (64, 256, 200), (128, 512, 33), (64, 32, 1)])
def test_features_f32(gpu, d, m, L):
    import torch
    x = synth.random_case(100 + d + m, 1, 2, L, d, m, "f32")
    phi = gpu.features(to_device(x["q"], "f32"), torch.from_numpy(x["w"]).cuda())
    torch.cuda.synchronize()
    ref = np.stack([oracle.favor_features(x["q64"][0, h], x["w64"][h]) for h in range(2)])[None]
    rel = np.abs(to_f64(phi) - ref) / ref
    assert rel.max() < 1e-4


@pytest.mark.parametrize("d,m,L", [(32, 256, 64), (64, 256, 300), (128, 512, 65), (64, 96, 7)])
def test_features_bf16_within_bound(gpu, d, m, L):
    """bf16 inputs are converted exactly to the fp16 projection operands; W is
    scaled by log2(e) and rounded to fp16, so each exponent (base 2) moves by
    at most 2^-11 * log2(e) * sum_d |x_d w_fd| (one half-ulp per product term)
    plus float32 rounding; the relative error of phi is bounded by
    2^that - 1."""
    import torch
    x = synth.random_case(200 + d + m, 1, 2, L, d, m, "bf16")
    phi = to_f64(gpu.features(to_device(x["q"], "bf16"), torch.from_numpy(x["w"]).cuda()))
    for h in range(2):
        q = x["q64"][0, h]
        w = x["w64"][h]
        ref = oracle.favor_features(q, w)
        e2 = 2.0 ** -11 * math.log2(math.e) * (np.abs(q) @ np.abs(w).T) + 1e-5 * (1 + np.abs(q @ w.T))
        bound = np.exp2(e2) - 1 + 1e-6
        assert np.all(np.abs(phi[0, h] - ref) <= bound * ref)


# ---------------------------------------------------------------------------
# non-causal attention
# ---------------------------------------------------------------------------

def _t1_table():
    rows = []
    with open(os.path.join(os.path.dirname(__file__), "golden", "t1_quality.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                m, c, e = line.split()
                rows.append((int(m), float(c), float(e)))
    return rows


@pytest.mark.parametrize("m,cos_printed,mse_printed", _t1_table())
def test_noncausal_worked_example(gpu, m, cos_printed, mse_printed):
    """The worked example (Performer page, In[26] / Out[27]): n=64, d=32,
    float32, the page's seeded Q, K, V and projection randn(d, m)/sqrt(d)
    (passed as float32 W^T).  The GPU output matches the oracle per row, and
    its mean row cosine and mean squared error against exact softmax
    attention with scores scaled by 1/sqrt(d) reproduce the printed table
    (4 and 6 decimals)."""
    import torch
    q64, k64, v64 = synth.t1_qkv()
    w = synth.t1_projection(m).astype(np.float32)
    dev = torch.device("cuda", 0)
    q, k, v = (torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).reshape(1, 1, 64, 32).to(dev)
               for a in (q64, k64, v64))
    out = gpu.attn(q, k, v, torch.from_numpy(w).to(dev), causal=False, eps=1e-6)
    torch.cuda.synchronize()
    got = to_f64(out)[0, 0]
    ref = oracle.attn_noncausal(q64, k64, v64, w.astype(np.float64), eps=1e-6)
    assert row_rel_err(got, ref) <= TOL["f32"]
    exact = oracle.softmax_attention(q64, k64, v64, scale=1.0 / math.sqrt(32))
    cos = float(np.mean([exact[i] @ got[i] / (np.linalg.norm(exact[i]) * np.linalg.norm(got[i])) for i in range(64)]))
    mse = float(np.mean((exact - got) ** 2))
    assert round(cos, 4) == pytest.approx(cos_printed, abs=1e-12)
    assert round(mse, 6) == pytest.approx(mse_printed, abs=1e-12)


@pytest.mark.parametrize("dtype,d,m,B,H,L", [
    ("bf16", 64, 256, 1, 3, 4096),      # encoder shape, 3 heads
    ("bf16", 64, 256, 2, 2, 1000),      # ragged tail
    ("bf16", 64, 256, 1, 1, 1),         # one token
    ("bf16", 64, 32, 1, 2, 333),        # smallest m
    ("bf16", 64, 512, 1, 2, 777),       # two feature groups
    ("bf16", 32, 128, 1, 2, 260),
    ("bf16", 128, 512, 1, 2, 300),
    ("f32", 32, 256, 1, 2, 500),
    ("f32", 64, 96, 1, 2, 129),
    ("f32", 128, 512, 1, 1, 200),
])
def test_noncausal_parity(gpu, dtype, d, m, B, H, L):
    x = synth.random_case(1000 + d + m + L, B, H, L, d, m, dtype)
    out = _run_attn(gpu, x, dtype, causal=False)
    assert row_rel_err(out, _ref(x, False)) <= TOL[dtype]


def test_noncausal_shared_projection(gpu):
    x = synth.random_case(7, 2, 3, 300, 64, 256, "bf16", heads_w=1)
    out = _run_attn(gpu, x, "bf16", causal=False)
    assert row_rel_err(out, _ref(x, False)) <= TOL["bf16"]


@pytest.mark.parametrize("dtype,d,m,B,H,L,heads_w", [
    ("f32", 32, 256, 1, 1, 64, None),   # the worked example's shape
    ("f32", 32, 32, 1, 2, 17, None),
    ("f32", 64, 96, 2, 2, 33, None),    # second token block holds one token
    ("f32", 64, 250, 1, 3, 64, 1),      # ragged m, one W for every head
    ("bf16", 64, 256, 1, 4, 64, None),
    ("bf16", 32, 200, 3, 1, 31, None),
    ("bf16", 64, 40, 1, 2, 2, None),
    ("bf16", 32, 256, 2, 2, 64, 1),
])
def test_noncausal_short_heads(gpu, dtype, d, m, B, H, L, heads_w):
    """Heads of at most 64 tokens (m <= 256, d 32 or 64) take the one-launch
    kernel: every row against the oracle at the same tolerances."""
    x = synth.random_case(8100 + d + m + L, B, H, L, d, m, dtype, heads_w=heads_w)
    out = _run_attn(gpu, x, dtype, causal=False)
    assert row_rel_err(out, _ref(x, False)) <= TOL[dtype]


def test_noncausal_encoder_full_size_sampled(gpu):
    """The full encoder workload (B=8, H=12, L=4096, d=64, m=256, bf16) in the
    launch configuration the benchmark uses; every head is checked on 64
    sampled rows by the oracle's per-row definition."""
    wl = synth.WORKLOADS["encoder"]
    x = synth.make_inputs(wl)
    out = _run_attn(gpu, x, "bf16", causal=False)
    rng = np.random.default_rng(0)
    worst = 0.0
    for b in range(wl.B):
        for h in range(wl.H):
            rows = np.sort(rng.choice(wl.L, 64, replace=False))
            ref = oracle.attn_rows(x["q64"][b, h], x["k64"][b, h], x["v64"][b, h], x["w64"][h], rows)
            worst = max(worst, row_rel_err(out[b, h, rows], ref))
    assert worst <= TOL["bf16"]


def test_noncausal_long_full_size_sampled(gpu):
    """The non-causal half of the long workload (B=1, H=8, L=65536, d=64,
    m=256, bf16) in the benchmark's launch configuration; every head is
    checked on sampled rows, the first and last included."""
    import torch
    wl = synth.WORKLOADS["long"]
    x = synth.make_inputs(wl, with64=False)
    q, k, v = (to_device(x[n], "bf16") for n in ("q", "k", "v"))
    o = gpu.attn(q, k, v, torch.from_numpy(x["w"]).cuda(), causal=False)
    torch.cuda.synchronize()
    rng = np.random.default_rng(2)
    worst = 0.0
    for h in range(wl.H):
        rows = np.unique(np.concatenate([[0, 511, 512, wl.L - 1], rng.choice(wl.L, 28, replace=False)]))
        q64, k64, v64 = (synth.as_f64(x[n][0, h], "bf16") for n in ("q", "k", "v"))
        ref = oracle.attn_rows(q64, k64, v64, x["w64"][h], rows)
        got = o[0, h, torch.from_numpy(rows).cuda()].float().cpu().numpy().astype(np.float64)
        worst = max(worst, row_rel_err(got, ref))
    assert worst <= TOL["bf16"]


@pytest.mark.parametrize("causal", [False, True])
def test_total_size_beyond_32_bits(gpu, causal):
    """B*H*L*max(d, m) = 2^31 (B=1, H=64, L=131072, d=64, m=256, bf16; 1 GiB
    per tensor): heads are addressed with 64-bit offsets.  Each head is drawn
    from its own seed (the encoder recipe, one W per head); the first, a
    middle and the last head are checked on sampled rows by the oracle's
    per-row definition."""
    import torch
    B, H, L, d, m = 1, 64, 131072, 64, 256
    dev = torch.device("cuda", 0)
    q = torch.empty((B, H, L, d), dtype=torch.bfloat16, device=dev)
    k, v = torch.empty_like(q), torch.empty_like(q)
    w = torch.empty((H, m, d), dtype=torch.float32, device=dev)
    keep = {}
    for h in range(H):
        x = synth.random_case(77000 + h, 1, 1, L, d, m, "bf16")
        for name, t in (("q", q), ("k", k), ("v", v)):
            t[0, h].copy_(to_device(x[name][0, 0], "bf16"))
        w[h].copy_(torch.from_numpy(x["w"][0]))
        if h in (0, 31, 63):
            keep[h] = x
    o = gpu.attn(q, k, v, w, causal=causal)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    worst = 0.0
    for h, x in keep.items():
        rows = np.unique(np.concatenate([[0, 1, 4095, 4096, L // 2, L - 1], rng.choice(L, 10, replace=False)]))
        ref = oracle.attn_rows(x["q64"][0, 0], x["k64"][0, 0], x["v64"][0, 0], x["w64"][0], rows, causal=causal)
        got = o[0, h, torch.from_numpy(rows).cuda()].float().cpu().numpy().astype(np.float64)
        worst = max(worst, row_rel_err(got, ref))
    assert worst <= TOL["bf16"]


def test_noncausal_deterministic(gpu):
    import torch
    x = synth.random_case(9, 1, 4, 2048, 64, 256, "bf16")
    q, k, v = (to_device(x[n], "bf16") for n in ("q", "k", "v"))
    w = torch.from_numpy(x["w"]).cuda()
    first = gpu.attn(q, k, v, w)
    for _ in range(5):
        assert torch.equal(gpu.attn(q, k, v, w), first)


def test_noncausal_constant_values(gpu):
    """V = 1 gives O = den / (den + eps) in every column (eps in the
    denominator only); with a large eps this is visibly below 1."""
    import torch
    x = synth.random_case(11, 1, 2, 100, 64, 128, "f32")
    q, k = (to_device(x[n], "f32") for n in ("q", "k"))
    v = torch.ones_like(q)
    w = torch.from_numpy(x["w"]).cuda()
    eps = 1000.0
    out = to_f64(gpu.attn(q, k, v, w, eps=eps))
    ref = oracle.per_head(oracle.attn_noncausal, x["q64"], x["k64"], np.ones_like(x["v64"]), x["w64"], eps=eps)
    assert row_rel_err(out, ref) <= TOL["f32"]
    assert out.max() < 0.9


# ---------------------------------------------------------------------------
# causal attention
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,d,m,B,H,L", [
    ("bf16", 64, 256, 1, 2, 64),        # one chunk
    ("bf16", 64, 256, 1, 2, 100),       # ragged second chunk
    ("bf16", 64, 256, 1, 2, 1000),      # several spans and chunks
    ("bf16", 64, 256, 1, 1, 1),         # one token
    ("bf16", 64, 32, 2, 1, 300),        # smallest m
    ("bf16", 32, 128, 1, 2, 333),
    ("bf16", 128, 512, 1, 1, 257),      # several feature groups
    ("f32", 32, 256, 1, 1, 200),        # two feature groups
    ("f32", 64, 96, 1, 2, 130),
    ("f32", 128, 512, 1, 1, 300),       # wide-feature shape, four feature groups
    ("f32", 64, 256, 1, 2, 1000),       # several spans, two feature groups (two workgroups per CU build)
    ("f32", 32, 512, 1, 2, 700),        # several spans, four feature groups
    ("bf16", 32, 256, 1, 2, 1000),      # the m = 256 scan at d = 32, several spans
    ("f32", 128, 512, 1, 2, 1000),      # split-product scan: several spans, four feature groups
    ("f32", 128, 128, 2, 2, 777),       # split-product scan: one feature group, ragged last chunk
    ("f32", 128, 200, 1, 1, 333),       # split-product scan: ragged m, a feature block past m
    ("f32", 128, 256, 1, 1, 1),         # split-product scan: one token
])
def test_causal_parity(gpu, dtype, d, m, B, H, L):
    x = synth.random_case(3000 + d + m + L, B, H, L, d, m, dtype)
    out = _run_attn(gpu, x, dtype, causal=True)
    assert row_rel_err(out, _ref(x, True)) <= TOL[dtype]


@pytest.mark.parametrize("dtype,d,m", [("bf16", 64, 256), ("bf16", 32, 96), ("f32", 64, 128), ("bf16", 128, 256)])
def test_causal_shared_projection(gpu, dtype, d, m):
    """One W for every head (Hw = 1), several batches and heads, both scans."""
    x = synth.random_case(8 + d + m, 2, 3, 700, d, m, dtype, heads_w=1)
    out = _run_attn(gpu, x, dtype, causal=True)
    assert row_rel_err(out, _ref(x, True)) <= TOL[dtype]


@pytest.mark.parametrize("dtype,d,m", [("bf16", 64, 256), ("bf16", 32, 256), ("bf16", 64, 96), ("f32", 64, 128),
                                     ("f32", 128, 256)])
def test_causal_independent_of_span_count(gpu, dtype, d, m, monkeypatch):
    """The causal result does not depend on how the sequence is cut into
    spans (the cross-span prefix is exact): forced span counts of 1, 3, 7
    and 16 per head each match the oracle, and each other within rounding."""
    x = synth.random_case(4100 + d + m, 1, 2, 2000, d, m, dtype)
    ref = _ref(x, True)
    outs = []
    for spans in (1, 3, 7, 16):
        monkeypatch.setenv("FAVOR_SPANS", str(spans))
        out = _run_attn(gpu, x, dtype, causal=True)
        assert row_rel_err(out, ref) <= TOL[dtype], spans
        outs.append(out)
    monkeypatch.delenv("FAVOR_SPANS")
    for out in outs[1:]:
        assert row_rel_err(out, outs[0]) <= TOL[dtype]


@pytest.mark.parametrize("f32_mfma", ["0", "1"])
def test_float32_causal_both_product_forms(gpu, f32_mfma, monkeypatch):
    """Float32 FAVOR+ causal at d = 128 runs on split 16-bit products by
    default and on float32 products with FAVOR_F32_MFMA=1; both match the
    oracle at the float32 tolerance, on several spans and feature groups."""
    monkeypatch.setenv("FAVOR_F32_MFMA", f32_mfma)
    x = synth.random_case(4170, 1, 3, 1500, 128, 384, "f32")
    out = _run_attn(gpu, x, "f32", causal=True)
    monkeypatch.delenv("FAVOR_F32_MFMA")
    assert row_rel_err(out, _ref(x, True)) <= TOL["f32"]


@pytest.mark.parametrize("dtype,d,m", [("bf16", 64, 256), ("f32", 128, 256)])
def test_causal_many_spans(gpu, dtype, d, m, monkeypatch):
    """More than 16 spans per head take the two-level prefix scan (groups of
    spans summed, then the groups' offsets); 19 spans of 320 tokens."""
    x = synth.random_case(4150 + d, 1, 2, 6000, d, m, dtype)
    monkeypatch.setenv("FAVOR_SPANS", "20")
    out = _run_attn(gpu, x, dtype, causal=True)
    monkeypatch.delenv("FAVOR_SPANS")
    assert row_rel_err(out, _ref(x, True)) <= TOL[dtype]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype,d,m", [("bf16", 64, 256), ("bf16", 32, 256), ("bf16", 64, 96), ("bf16", 128, 256),
                                     ("f32", 128, 256)])
def test_entries_beyond_fp16_range(gpu, causal, dtype, d, m):
    """Query and key rows with one entry of 3e5, past fp16's 65504 (the
    projection's operand type for bf16): their FAVOR+ features
    exp(w.x - |x|^2/2)/sqrt(m) are 0 in float64 as well, so such a query row's
    output is exactly 0 and such a key adds nothing; every other row matches
    the oracle."""
    L = 300
    x = synth.random_case(4300 + d + m, 1, 2, L, d, m, dtype)
    rows_q, rows_k = [5, 77, L - 1], [10, 150]
    for name, rows in (("q", rows_q), ("k", rows_k)):
        arr = x[name + "64"].copy()
        arr[0, :, rows, 3] = 3e5
        x[name] = synth.bf16_round(arr.astype(np.float32)) if dtype == "bf16" else arr.astype(np.float32)
        x[name + "64"] = synth.as_f64(x[name], dtype)
    out = _run_attn(gpu, x, dtype, causal=causal)
    ref = _ref(x, causal)
    assert np.all(ref[0, :, rows_q] == 0)
    assert np.all(out[0, :, rows_q] == 0), out[0, :, rows_q]
    keep = np.setdiff1d(np.arange(L), rows_q)
    assert row_rel_err(out[:, :, keep], ref[:, :, keep]) <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noncausal_key_value_permutation_invariance(gpu, dtype):
    """Non-causal attention sums over keys: permuting the rows of K and V
    together leaves every output row unchanged up to rounding (the reduction
    splits see different keys; each result also matches the oracle)."""
    x = synth.random_case(4200, 1, 2, 3000, 64, 256, dtype)
    out = _run_attn(gpu, x, dtype, causal=False)
    perm = np.random.default_rng(9).permutation(3000)
    y = dict(x)
    for n in ("k", "v"):
        y[n] = np.ascontiguousarray(x[n][:, :, perm])
        y[n + "64"] = np.ascontiguousarray(x[n + "64"][:, :, perm])
    out_p = _run_attn(gpu, y, dtype, causal=False)
    assert row_rel_err(out_p, _ref(x, False)) <= TOL[dtype]
    assert row_rel_err(out_p, out) <= TOL[dtype]


def test_causal_deterministic(gpu):
    """The causal path adds in a fixed order (span scan, chunk walk, cross-wave
    sums): repeated calls give identical bits."""
    import torch
    x = synth.random_case(15, 1, 4, 3000, 64, 256, "bf16")
    q, k, v = (to_device(x[n], "bf16") for n in ("q", "k", "v"))
    w = torch.from_numpy(x["w"]).cuda()
    first = gpu.attn(q, k, v, w, causal=True)
    for _ in range(5):
        assert torch.equal(gpu.attn(q, k, v, w, causal=True), first)


def test_causal_last_row_matches_noncausal(gpu):
    x = synth.random_case(13, 1, 2, 777, 64, 256, "f32")
    c = _run_attn(gpu, x, "f32", causal=True)
    n = _run_attn(gpu, x, "f32", causal=False)
    assert row_rel_err(c[:, :, -1], n[:, :, -1]) <= TOL["f32"]


def test_causal_first_row_is_first_value(gpu):
    """Row 0 sees only key 0: o_0 = v_0 * a / (a + eps)."""
    x = synth.random_case(14, 1, 2, 128, 32, 64, "f32")
    out = _run_attn(gpu, x, "f32", causal=True)
    for h in range(2):
        a = oracle.favor_features(x["q64"][0, h, :1], x["w64"][h])[0] @ \
            oracle.favor_features(x["k64"][0, h, :1], x["w64"][h])[0]
        np.testing.assert_allclose(out[0, h, 0], x["v64"][0, h, 0] * a / (a + 1e-6), rtol=1e-4, atol=1e-6)


@pytest.mark.parametrize("name", ["causal_lm", "long"])
def test_causal_full_size_sampled(gpu, name):
    """Full causal workloads in the benchmark's launch configuration; every
    head is checked on sampled rows (first, last, span/chunk edges, random)
    by the oracle's per-row definition."""
    wl = synth.WORKLOADS[name]
    x = synth.make_inputs(wl, with64=False)
    import torch
    q, k, v = (to_device(x[n], "bf16") for n in ("q", "k", "v"))
    o = gpu.attn(q, k, v, torch.from_numpy(x["w"]).cuda(), causal=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    fixed = np.array([0, 1, 63, 64, 65, 1023, 1024, 2047, 2048, wl.L - 1])
    worst = 0.0
    heads = [(b, h) for b in range(wl.B) for h in range(wl.H)]
    for b, h in heads[:: max(1, len(heads) // 8)]:
        rows = np.unique(np.concatenate([fixed[fixed < wl.L], rng.choice(wl.L, 12, replace=False)]))
        q64, k64, v64 = (synth.as_f64(x[n][b, h], "bf16") for n in ("q", "k", "v"))
        ref = oracle.attn_rows(q64, k64, v64, x["w64"][h], rows, causal=True)
        got = o[b, h, torch.from_numpy(rows).cuda()].float().cpu().numpy().astype(np.float64)
        worst = max(worst, row_rel_err(got, ref))
    assert worst <= TOL["bf16"]


def test_causal_wide_full_size_sampled(gpu):
    """The float32 wide-state workload (B=2, H=32, L=32768, d=128, m=512,
    causal) at full size; eight heads spread over both batches are checked on
    sampled rows (first, chunk and span edges, last, random) to the float32
    tolerance."""
    import torch
    wl = synth.WORKLOADS["wide"]
    x = synth.make_inputs(wl, with64=False)
    q, k, v = (to_device(x[n], "f32") for n in ("q", "k", "v"))
    o = gpu.attn(q, k, v, torch.from_numpy(x["w"]).cuda(), causal=True)
    torch.cuda.synchronize()
    del q, k, v
    rng = np.random.default_rng(3)
    fixed = np.array([0, 1, 31, 32, 33, 255, 256, 1023, 1024, wl.L - 1])
    worst = 0.0
    heads = [(b, h) for b in range(wl.B) for h in range(wl.H)]
    for b, h in heads[:: len(heads) // 8]:
        rows = np.unique(np.concatenate([fixed, rng.choice(wl.L, 10, replace=False)]))
        q64, k64, v64 = (np.asarray(x[n][b, h], dtype=np.float64) for n in ("q", "k", "v"))
        ref = oracle.attn_rows(q64, k64, v64, x["w64"][h], rows, causal=True)
        got = o[b, h, torch.from_numpy(rows).cuda()].cpu().numpy().astype(np.float64)
        worst = max(worst, row_rel_err(got, ref))
    assert worst <= TOL["f32"]


# ---------------------------------------------------------------------------
# m not a multiple of 32 (padding features)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype,d,m,L", [("bf16", 64, 100, 300), ("bf16", 64, 1, 130), ("bf16", 32, 200, 257),
                                         ("f32", 64, 33, 129), ("f32", 128, 250, 100)])
def test_ragged_feature_count(gpu, causal, dtype, d, m, L):
    """m not a multiple of 32: the kernels pad to whole 32-feature blocks
    whose key-side features are exactly zero; the result equals the
    definition with the m given features (1/sqrt(m) with the true m)."""
    x = synth.random_case(4000 + d + m + L, 1, 2, L, d, m, dtype)
    print(f"[ragged] causal={causal} {dtype} d={d} m={m} L={L}", flush=True)
    out = _run_attn(gpu, x, dtype, causal=causal)
    assert row_rel_err(out, _ref(x, causal)) <= TOL[dtype]


@pytest.mark.parametrize("kind", ["positive", "trig", "relu"])
def test_ragged_features_and_maps(gpu, kind):
    import torch
    x = synth.random_case(4100, 1, 2, 200, 64, 72, "f32", qk_scale=0.15 if kind == "trig" else None)
    phi = gpu.features(to_device(x["q"], "f32"), torch.from_numpy(x["w"]).cuda(), fmap=kind)
    torch.cuda.synchronize()
    ref = np.stack([oracle.feature_map(x["q64"][0, h], x["w64"][h], kind) for h in range(2)])[None]
    assert phi.shape == ref.shape
    assert row_rel_err(to_f64(phi), ref) <= 1e-4
    for causal in (False, True):
        q, k, v = (to_device(x[n], "f32") for n in ("q", "k", "v"))
        o = gpu.attn(q, k, v, torch.from_numpy(x["w"]).cuda(), causal=causal, fmap=kind)
        torch.cuda.synchronize()
        fn = oracle.attn_causal if causal else oracle.attn_noncausal
        ref_o = oracle.per_head(fn, x["q64"], x["k64"], x["v64"], x["w64"], kind=kind)
        assert row_rel_err(to_f64(o), ref_o) <= TOL["f32"]


@pytest.mark.parametrize("kind", ["positive", "elu1", "relu", "trig"])
@pytest.mark.parametrize("d,m,L", [(64, 72, 300), (32, 40, 97)])
def test_ragged_maps_bf16(gpu, kind, d, m, L):
    """bf16, m not a multiple of 32, every feature map: the 32-token causal
    scan's padded-feature path (and for trig a feature pair whose sine and
    cosine blocks share a wave) against the definition with m features."""
    import torch
    x = synth.random_case(4200 + d + m, 1, 2, L, d, m, "bf16", qk_scale=0.15 if kind == "trig" else None)
    print(f"[ragged bf16] {kind} d={d} m={m} L={L}", flush=True)
    for causal in (False, True):
        q, k, v = (to_device(x[n], "bf16") for n in ("q", "k", "v"))
        o = gpu.attn(q, k, v, torch.from_numpy(x["w"]).cuda(), causal=causal, fmap=kind)
        torch.cuda.synchronize()
        fn = oracle.attn_causal if causal else oracle.attn_noncausal
        ref_o = oracle.per_head(fn, x["q64"], x["k64"], x["v64"], x["w64"], kind=kind)
        err = row_rel_err(to_f64(o), ref_o)
        print(f"[ragged bf16]   causal={causal} err {err:.3g}", flush=True)
        assert err <= TOL["bf16"]
