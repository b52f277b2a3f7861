"""HIP graph capture of the attention calls.  A call enqueues kernels only
(no memset, no copy, no allocation when the caller passes the output and
the workspace, or uses the static-scratch entry point), so a captured call
replays the same launches: every replay must reproduce the eager output bit
for bit, with eager work on the same buffers and a synchronisation between
the replays."""
import pytest

import synth
from _util import to_device

pytestmark = pytest.mark.gpu


def _inputs(seed, L, d, m, dtype, H=2):
    import torch
    x = synth.random_case(seed, 1, H, L, d, m, dtype)
    q, k, v = (to_device(x[n], dtype) for n in ("q", "k", "v"))
    return q, k, v, torch.from_numpy(x["w"]).cuda()


def _replays_match(torch, g, out, ref, n=3):
    for i in range(n):
        out.fill_(float("nan"))            # eager work on the captured output between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {i}"


@pytest.mark.parametrize("dtype,d,m,L,causal", [
    ("bf16", 64, 256, 2048, False),
    ("bf16", 64, 256, 2048, True),          # reduction, span prefixes, pipelined scan
    ("bf16", 32, 96, 777, True),            # generic scan, ragged m and L
    ("f32", 32, 256, 64, False),            # the worked example's shape
    ("f32", 128, 256, 300, True),           # split-product float32 scan
])
def test_graph_replays_match_eager(gpu, dtype, d, m, L, causal):
    import torch
    q, k, v, w = _inputs(9100 + d + m + L, L, d, m, dtype)
    out = torch.empty_like(q)
    ws = torch.empty(gpu.workspace_bytes(1, 2, L, d, m, causal, gpu.BF16 if dtype == "bf16" else gpu.F32),
                     dtype=torch.uint8, device="cuda")
    gpu.attn(q, k, v, w, causal=causal, out=out, workspace=ws)
    torch.cuda.synchronize()
    ref = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gpu.attn(q, k, v, w, causal=causal, out=out, workspace=ws)
    _replays_match(torch, g, out, ref)


def test_graph_replays_both_paths_and_noalloc(gpu):
    """One graph holding a non-causal call, a causal call and a static-scratch
    call, as a serving step would capture them."""
    import torch
    q, k, v, w = _inputs(9200, 1500, 64, 256, "bf16")
    outs = [torch.empty_like(q) for _ in range(3)]
    wss = [torch.empty(gpu.workspace_bytes(1, 2, 1500, 64, 256, c, gpu.BF16), dtype=torch.uint8, device="cuda")
           for c in (False, True)]

    def step():
        gpu.attn(q, k, v, w, causal=False, out=outs[0], workspace=wss[0])
        gpu.attn(q, k, v, w, causal=True, out=outs[1], workspace=wss[1])
        gpu.attn_noalloc(q, k, v, w, outs[2], causal=True)

    step()
    torch.cuda.synchronize()
    refs = [o.clone() for o in outs]
    assert torch.equal(refs[1], refs[2])
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(3):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for j, (o, r) in enumerate(zip(outs, refs)):
            assert torch.equal(o, r), (i, j)
