"""favor_attn_noalloc (the entry point for callers that cannot allocate):
called through the C ABI, its output equals favor_attn's with a caller
workspace bit for bit, on two calls in a row (the second with a smaller
input, so the shared static scratch holds the first call's contents), and a
shape whose workspace exceeds the scratch is refused without a launch."""
import numpy as np
import pytest

import synth
from _util import to_device

pytestmark = pytest.mark.gpu


def _case(seed, L, d=64, m=256, dtype="bf16", H=2):
    import torch
    x = synth.random_case(seed, 1, H, L, d, m, dtype)
    q, k, v = (to_device(x[n], dtype) for n in ("q", "k", "v"))
    return q, k, v, torch.from_numpy(x["w"]).cuda()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype,d,m", [("bf16", 64, 256), ("bf16", 32, 96), ("f32", 64, 128)])
def test_noalloc_matches_workspace_entry_point(gpu, causal, dtype, d, m):
    import torch
    for seed, L in ((51, 4000), (52, 777)):            # the second call is smaller
        q, k, v, w = _case(seed + d + m, L, d, m, dtype)
        out = torch.full_like(q, float("nan"))
        gpu.attn_noalloc(q, k, v, w, out, causal=causal)
        ref = gpu.attn(q, k, v, w, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), (seed, L)
        assert np.isfinite(out.float().cpu().numpy()).all()


def test_noalloc_refuses_shapes_beyond_the_scratch(gpu):
    """float32 causal d = 128, m = 512 at L = 65536, H = 8 needs ~290 MB of
    workspace (partial numerators of four feature groups), more than the
    64 MB scratch: status FAVOR_ERR_WORKSPACE and the output untouched."""
    import torch
    B, H, L, d, m = 1, 8, 65536, 128, 512
    assert gpu.workspace_bytes(B, H, L, d, m, True, torch.float32) > 64 << 20
    q = torch.zeros((B, H, L, d), dtype=torch.float32, device="cuda")
    w = torch.zeros((H, m, d), dtype=torch.float32, device="cuda")
    out = torch.full_like(q, 7.0)
    with pytest.raises(gpu.FavorError) as e:
        gpu.attn_noalloc(q, q, q, w, out, causal=True)
    assert e.value.code == 4
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
