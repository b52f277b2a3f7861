"""Calling conventions of the binding on the GPU: work goes to the caller's
current stream, and one workspace serves calls of different shapes."""
import numpy as np
import pytest

import synth
from _util import to_device

pytestmark = pytest.mark.gpu


def _case(seed, L, causal_dtype="bf16"):
    import torch
    x = synth.random_case(seed, 1, 2, L, 64, 256, causal_dtype)
    q, k, v = (to_device(x[n], causal_dtype) for n in ("q", "k", "v"))
    return q, k, v, torch.from_numpy(x["w"]).cuda()


@pytest.mark.parametrize("causal", [False, True])
def test_side_stream_gives_the_same_bits(gpu, causal):
    """A call made while a side stream is current runs on that stream and
    matches the call on the default stream exactly."""
    import torch
    q, k, v, w = _case(41, 1500)
    ref = gpu.attn(q, k, v, w, causal=causal)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        out = gpu.attn(q, k, v, w, causal=causal)
        done = torch.cuda.Event()
        done.record(side)
    torch.cuda.current_stream().wait_event(done)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


@pytest.mark.parametrize("causal", [False, True])
def test_workspace_reused_across_shapes(gpu, causal):
    """A workspace sized for a long call serves a shorter one after it (and
    the long one again), with results equal to calls with fresh workspaces."""
    import torch
    big = _case(42, 3000)
    small = _case(43, 333)
    need = max(gpu.workspace_bytes(1, 2, 3000, 64, 256, causal, gpu.BF16),
               gpu.workspace_bytes(1, 2, 333, 64, 256, causal, gpu.BF16))
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    outs = [gpu.attn(*c, causal=causal, workspace=ws) for c in (big, small, big)]
    refs = [gpu.attn(*c, causal=causal) for c in (big, small)]
    torch.cuda.synchronize()
    assert torch.equal(outs[0], refs[0]) and torch.equal(outs[2], refs[0])
    assert torch.equal(outs[1], refs[1])
    assert np.isfinite(outs[1].float().cpu().numpy()).all()


def _bad_arg_cases():
    import torch
    dev = torch.device("cuda", 0)
    q = torch.zeros(1, 2, 40, 64, dtype=torch.bfloat16, device=dev)
    w = torch.zeros(2, 32, 64, device=dev)
    return dev, q, w


@pytest.mark.parametrize("bad", ["out_shape", "out_dtype", "out_host", "out_noncontig", "ws_host", "ws_dtype",
                                 "w_host"])
@pytest.mark.parametrize("causal", [False, True])
def test_attn_rejects_bad_caller_buffers(gpu, bad, causal):
    """Caller-supplied out, workspace and W are checked before any launch:
    a wrong-sized or host buffer raises instead of being written through."""
    import torch
    dev, q, w = _bad_arg_cases()
    kw = {}
    if bad == "out_shape":
        kw["out"] = torch.empty(1, 2, 39, 64, dtype=q.dtype, device=dev)
    elif bad == "out_dtype":
        kw["out"] = torch.empty_like(q, dtype=torch.float32)
    elif bad == "out_host":
        kw["out"] = torch.empty(q.shape, dtype=q.dtype)
    elif bad == "out_noncontig":
        kw["out"] = torch.empty(1, 2, 64, 40, dtype=q.dtype, device=dev).transpose(2, 3)
    elif bad == "ws_host":
        kw["workspace"] = torch.empty(1 << 20, dtype=torch.uint8)
    elif bad == "ws_dtype":
        kw["workspace"] = torch.empty(1 << 18, dtype=torch.float32, device=dev)
    else:
        w = w.cpu()
    with pytest.raises((ValueError, TypeError)):
        gpu.attn(q, q, q, w, causal=causal, **kw)


@pytest.mark.parametrize("bad", ["out_shape", "out_host"])
def test_softmax_and_strided_reject_bad_outputs(gpu, bad):
    import torch
    dev, q, w = _bad_arg_cases()
    out = torch.empty(1, 2, 39, 64, dtype=q.dtype, device=dev) if bad == "out_shape" else torch.empty(q.shape, dtype=q.dtype)
    with pytest.raises((ValueError, TypeError)):
        gpu.softmax_attn(q, q, q, out=out)
    with pytest.raises((ValueError, TypeError)):
        gpu.attn_strided(q, q, q, w, out=out)


def test_backward_rejects_host_workspace(gpu):
    import torch
    dev, q, w = _bad_arg_cases()
    with pytest.raises(ValueError):
        gpu.attn_backward(q, q, q, w, q, workspace=torch.empty(1 << 20, dtype=torch.uint8))
