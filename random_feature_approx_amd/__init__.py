"""Python binding of the gfx950 FAVOR+ library (libfavor.so).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/favor.h.  PyTorch provides device
memory and the current stream.  There is no CPU fallback: if the library is
missing, or the tensors are not on a HIP device, calls raise.

Functions
    features(x, w, fmap="positive")         phi(x) as float32 [B, H, L, m] (2m for "trig")
    attn(q, k, v, w, causal=False, eps=1e-6, fmap="positive")
                                            attention, output like q; fmap is one of
                                            FMAPS (FAVOR+ "positive", "elu1", "relu", "trig")
    attn_noncausal(...), attn_causal(...)    the two paths explicitly
    workspace_bytes(B, H, L, d, m, causal, dtype)
    attn_backward(q, k, v, w, g, causal=False, eps=1e-6)
                                            gradients (dq, dk, dv) of sum(g * O)
    bwd_workspace_bytes(B, H, L, d, m, causal, dtype)

Shapes: q, k, v are [B, H, L, d] (bfloat16 or float32, same dtype, contiguous);
w is float32 [m, d] (shared by all heads) or [H, m, d] (one per head).
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["load", "library_path", "features", "attn", "attn_noalloc", "attn_noncausal", "attn_causal", "FMAPS", "softmax_attn", "attn_strided", "draw_projection",
           "workspace_bytes", "attn_backward", "bwd_workspace_bytes", "FavorError", "STATUS", "KERNELS",
           "timing_start", "timing_stop"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIBNAME = "libfavor.so"
_lib = None

FMAPS = {"positive": 0, "elu1": 1, "relu": 2, "trig": 3}
STATUS = {0: "ok", 1: "null pointer argument", 2: "invalid shape", 3: "unsupported d, m or dtype",
          4: "workspace missing or too small", 5: "HIP runtime error", 6: "internal error"}
F32, BF16 = 0, 1
KERNELS = {"k_features": 0, "k_reduce": 1, "k_combine": 2, "k_apply": 3, "k_span_scan": 4, "k_causal": 5,
           "k_bprep": 6, "k_bred": 7, "k_bcombine": 8, "k_bside_q": 9, "k_bside_k": 10, "k_softmax": 11,
           "k_draw": 12}


class FavorError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} failed: {STATUS.get(code, 'unknown status')} (status {code})")
        self.code = code


def library_path() -> str:
    return os.path.join(_HERE, _LIBNAME)


def load():
    """Load libfavor.so (built by ``build.py``); raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m random_feature_approx_amd.build` "
                           "(there is no CPU fallback)")
    lib = ctypes.CDLL(path)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.favor_abi_version.restype = i
    lib.favor_abi_version.argtypes = []
    lib.favor_status_string.restype = ctypes.c_char_p
    lib.favor_status_string.argtypes = [i]
    lib.favor_workspace_bytes.restype = sz
    lib.favor_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    lib.favor_features.restype = i
    lib.favor_features.argtypes = [vp, vp, i, vp, i, i, i, i, i, i, vp]
    attn_args = [vp, vp, vp, vp, i, vp, i, i, i, i, i, f, i, vp, sz, vp]
    for name in ("favor_attn_noncausal", "favor_attn_causal"):
        getattr(lib, name).restype = i
        getattr(lib, name).argtypes = attn_args
    lib.favor_attn.restype = i
    lib.favor_attn.argtypes = [vp, vp, vp, vp, i, vp, i, i, i, i, i, f, i, i, vp, sz, vp]
    lib.favor_attn_noalloc.restype = i
    lib.favor_attn_noalloc.argtypes = [vp, vp, vp, vp, i, vp, i, i, i, i, i, f, i, i, vp]
    lib.favor_workspace_bytes_fmap.restype = sz
    lib.favor_workspace_bytes_fmap.argtypes = [i, i, i, i, i, i, i, i]
    lib.favor_features_fmap.restype = i
    lib.favor_features_fmap.argtypes = [vp, vp, i, vp, i, i, i, i, i, i, i, vp]
    lib.favor_attn_fmap.restype = i
    lib.favor_attn_fmap.argtypes = [vp, vp, vp, vp, i, vp, i, i, i, i, i, f, i, i, i, vp, sz, vp]
    ll3 = ctypes.POINTER(ctypes.c_longlong)
    lib.favor_workspace_bytes_strided.restype = sz
    lib.favor_workspace_bytes_strided.argtypes = [i, i, i, i, i, i, i, i, i]
    lib.favor_attn_strided.restype = i
    lib.favor_attn_strided.argtypes = [vp, ll3, vp, ll3, vp, ll3, vp, i, vp, ll3, i, i, i, i, i, i, f, i, i, i,
                                       vp, sz, vp]
    lib.favor_draw_projection.restype = i
    lib.favor_draw_projection.argtypes = [ctypes.c_ulonglong, i, i, i, i, f, vp, vp]
    lib.favor_softmax_attn.restype = i
    lib.favor_softmax_attn.argtypes = [vp, vp, vp, vp, i, i, i, i, f, i, i, vp]
    lib.favor_bwd_workspace_bytes.restype = sz
    lib.favor_bwd_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    for name in ("favor_attn_noncausal_bwd", "favor_attn_causal_bwd"):
        getattr(lib, name).restype = i
        getattr(lib, name).argtypes = [vp, vp, vp, vp, i, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, sz, vp]
    lib.favor_timing_start.restype = i
    lib.favor_timing_start.argtypes = [i, i]
    lib.favor_timing_stop.restype = i
    lib.favor_timing_stop.argtypes = [i, ctypes.POINTER(ctypes.c_double), i, ctypes.POINTER(i)]
    lib.favor_kernel_name.restype = ctypes.c_char_p
    lib.favor_kernel_name.argtypes = [i]
    if lib.favor_abi_version() != 1:
        raise RuntimeError("libfavor.so has an unexpected ABI version")
    _lib = lib
    return lib


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}: use bfloat16 or float32")


def _check_device(*ts):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("FAVOR+ tensors must live on a HIP device (no CPU path)")
        if not t.is_contiguous():
            raise ValueError("FAVOR+ tensors must be contiguous")


def _check_out(out, shape, dtype, device):
    """A caller-supplied output must match exactly: the kernels write every
    element of the expected shape through its pointer."""
    if not out.is_cuda or out.device != device:
        raise ValueError(f"out must live on {device}")
    if tuple(out.shape) != tuple(shape):
        raise ValueError(f"out must have shape {tuple(shape)}, got {tuple(out.shape)}")
    if out.dtype != dtype:
        raise TypeError(f"out must have dtype {dtype}, got {out.dtype}")
    if not out.is_contiguous():
        raise ValueError("out must be contiguous")


def _check_workspace(ws, device):
    torch = _torch()
    if not ws.is_cuda or ws.device != device:
        raise ValueError(f"workspace must live on {device}")
    if ws.dtype != torch.uint8 or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor")


def _proj(w, H, m_d):
    """Return (w, Hw) with w float32 [Hw, m, d] contiguous on the device."""
    torch = _torch()
    if w.dtype != torch.float32:
        raise TypeError("the projection W must be float32")
    if w.dim() == 2:
        w = w.unsqueeze(0)
    if w.dim() != 3 or tuple(w.shape[1:]) != m_d or w.shape[0] not in (1, H):
        raise ValueError(f"W must be [m, d] or [H, m, d], got {tuple(w.shape)}")
    if not w.is_cuda:
        raise ValueError("the projection W must live on a HIP device (no CPU path)")
    return w.contiguous(), int(w.shape[0])


def _stream():
    return ctypes.c_void_p(_torch().cuda.current_stream().cuda_stream)


def _fmap_code(fmap) -> int:
    if fmap not in FMAPS:
        raise ValueError(f"unknown feature map {fmap!r}; use one of {sorted(FMAPS)}")
    return FMAPS[fmap]


def workspace_bytes(B: int, H: int, L: int, d: int, m: int, causal: bool, dtype, fmap: str = "positive") -> int:
    code = dtype if isinstance(dtype, int) else _dtype_code(_torch().empty(0, dtype=dtype))
    return int(load().favor_workspace_bytes_fmap(B, H, L, d, m, int(bool(causal)), _fmap_code(fmap), code))


def features(x, w, fmap: str = "positive"):
    """phi(x) as float32 [B, H, L, m] (FAVOR+: exp(W x - |x|^2/2)/sqrt(m));
    [B, H, L, 2m] for the trig map, sines and cosines interleaved."""
    lib = load()
    torch = _torch()
    if x.dim() != 4:
        raise ValueError("x must be [B, H, L, d]")
    B, H, L, d = x.shape
    w, hw = _proj(w, H, (w.shape[-2], d))
    m = int(w.shape[1])
    _check_device(x, w)
    if w.device != x.device:
        raise ValueError("x and W must live on one device")
    code = _fmap_code(fmap)
    phi = torch.empty((B, H, L, 2 * m if fmap == "trig" else m), dtype=torch.float32, device=x.device)
    st = lib.favor_features_fmap(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(w.data_ptr()), hw,
                                 ctypes.c_void_p(phi.data_ptr()), B, H, L, d, m, code, _dtype_code(x), _stream())
    if st != 0:
        raise FavorError("favor_features_fmap", st)
    return phi


def attn(q, k, v, w, causal: bool = False, eps: float = 1e-6, out=None, workspace=None, fmap: str = "positive"):
    """Linear attention with the given feature map (FAVOR+ by default);
    returns O with the shape and dtype of q."""
    lib = load()
    torch = _torch()
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one [B, H, L, d] shape")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    B, H, L, d = q.shape
    w, hw = _proj(w, H, (w.shape[-2], d))
    m = int(w.shape[1])
    _check_device(q, k, v, w)
    if k.device != q.device or v.device != q.device or w.device != q.device:
        raise ValueError("q, k, v and W must live on one device")
    code = _dtype_code(q)
    if out is None:
        o = torch.empty_like(q)
    else:
        _check_out(out, q.shape, q.dtype, q.device)
        o = out
    fcode = _fmap_code(fmap)
    need = int(lib.favor_workspace_bytes_fmap(B, H, L, d, m, int(bool(causal)), fcode, code))
    if need == 0:
        raise FavorError("favor_workspace_bytes_fmap", 2)
    if workspace is not None:
        _check_workspace(workspace, q.device)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ptrs = (ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
            ctypes.c_void_p(w.data_ptr()), hw, ctypes.c_void_p(o.data_ptr()), B, H, L, d, m, float(eps))
    tail = (ctypes.c_void_p(workspace.data_ptr()), workspace.numel(), _stream())
    if fcode == 0:
        name = "favor_attn_causal" if causal else "favor_attn_noncausal"
        st = getattr(lib, name)(*ptrs, code, *tail)
    else:
        name = "favor_attn_fmap"
        st = lib.favor_attn_fmap(*ptrs, int(bool(causal)), fcode, code, *tail)
    if st != 0:
        raise FavorError(name, st)
    return o


def attn_noalloc(q, k, v, w, out, causal: bool = False, eps: float = 1e-6):
    """favor_attn_noalloc: attention into the caller's `out` with the
    library's static device scratch as workspace (no allocation by the call;
    calls on one device must not overlap).  Raises FavorError (status 4) when
    the shape needs more workspace than the scratch holds."""
    lib = load()
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one [B, H, L, d] shape")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    B, H, L, d = q.shape
    w, hw = _proj(w, H, (w.shape[-2], d))
    m = int(w.shape[1])
    _check_device(q, k, v, w)
    if k.device != q.device or v.device != q.device or w.device != q.device:
        raise ValueError("q, k, v and W must live on one device")
    _check_out(out, q.shape, q.dtype, q.device)
    st = lib.favor_attn_noalloc(ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
                                ctypes.c_void_p(v.data_ptr()), ctypes.c_void_p(w.data_ptr()), hw,
                                ctypes.c_void_p(out.data_ptr()), B, H, L, d, m, float(eps), int(bool(causal)),
                                _dtype_code(q), _stream())
    if st != 0:
        raise FavorError("favor_attn_noalloc", st)
    return out


def attn_noncausal(q, k, v, w, eps: float = 1e-6, **kw):
    return attn(q, k, v, w, causal=False, eps=eps, **kw)


def attn_causal(q, k, v, w, eps: float = 1e-6, **kw):
    return attn(q, k, v, w, causal=True, eps=eps, **kw)


def attn_strided(q, k, v, w, causal: bool = False, eps: float = 1e-6, out=None, fmap: str = "positive"):
    """Attention for tensors of any layout whose last dimension is contiguous
    (views such as a [B, L, H, d] tensor permuted to [B, H, L, d]) and for a
    value width dv that may differ from d: q, k are [B, H, L, d] views, v is
    [B, H, L, dv]; returns (or fills `out`, a [B, H, L, dv] view) O."""
    lib = load()
    torch = _torch()
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:3] != q.shape[:3]:
        raise ValueError("q, k must share a [B, H, L, d] shape and v must be [B, H, L, dv]")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    for t in (q, k, v):
        if not t.is_cuda or t.stride(3) != 1 or t.device != q.device:
            raise ValueError("tensors must live on one HIP device with a contiguous last dimension")
    B, H, L, d = q.shape
    dv = int(v.shape[3])
    w, hw = _proj(w, H, (w.shape[-2], d))
    if w.device != q.device:
        raise ValueError("W must live on the device of q")
    m = int(w.shape[1])
    code, fcode = _dtype_code(q), _fmap_code(fmap)
    o = torch.empty((B, H, L, dv), dtype=q.dtype, device=q.device) if out is None else out
    if not o.is_cuda or o.device != q.device:
        raise ValueError(f"out must live on {q.device}")
    if o.shape != (B, H, L, dv) or o.stride(3) != 1 or o.dtype != q.dtype:
        raise ValueError("out must be a [B, H, L, dv] view of the input dtype with a contiguous last dimension")
    if any(st < 0 for st in o.stride()):
        raise ValueError("out must have non-negative strides")
    need = int(lib.favor_workspace_bytes_strided(B, H, L, d, dv, m, int(bool(causal)), fcode, code))
    if need == 0:
        raise FavorError("favor_workspace_bytes_strided", 2)
    ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    st3 = lambda t: (ctypes.c_longlong * 3)(t.stride(0), t.stride(1), t.stride(2))  # noqa: E731
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    st = lib.favor_attn_strided(ptr(q), st3(q), ptr(k), st3(k), ptr(v), st3(v), ptr(w), hw, ptr(o), st3(o),
                                B, H, L, d, dv, m, float(eps), int(bool(causal)), fcode, code, ptr(ws), need,
                                _stream())
    if st != 0:
        raise FavorError("favor_attn_strided", st)
    return o


def draw_projection(seed: int, heads: int, m: int, d: int, orthogonal: bool = True, scale: float = 1.0,
                    device=None):
    """W [heads, m, d] float32 drawn on the device from `seed` (Philox4x64-10
    normals; orthogonal blocks with chi(d) row lengths, or independent rows)."""
    lib = load()
    torch = _torch()
    W = torch.empty((heads, m, d), dtype=torch.float32, device=device or "cuda")
    st = lib.favor_draw_projection(int(seed) & ((1 << 64) - 1), heads, m, d, int(bool(orthogonal)), float(scale),
                                   ctypes.c_void_p(W.data_ptr()), _stream())
    if st != 0:
        raise FavorError("favor_draw_projection", st)
    return W


def softmax_attn(q, k, v, scale=None, causal: bool = False, out=None):
    """Exact softmax(scale * q k^T) v (scale defaults to 1/sqrt(d)),
    optionally causal; the quadratic reference that FAVOR+ approximates."""
    lib = load()
    torch = _torch()
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one [B, H, L, d] shape")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    B, H, L, d = q.shape
    _check_device(q, k, v)
    if k.device != q.device or v.device != q.device:
        raise ValueError("q, k, v must live on one device")
    if out is None:
        o = torch.empty_like(q)
    else:
        _check_out(out, q.shape, q.dtype, q.device)
        o = out
    sc = float(d) ** -0.5 if scale is None else float(scale)
    st = lib.favor_softmax_attn(ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
                                ctypes.c_void_p(v.data_ptr()), ctypes.c_void_p(o.data_ptr()), B, H, L, d, sc,
                                int(bool(causal)), _dtype_code(q), _stream())
    if st != 0:
        raise FavorError("favor_softmax_attn", st)
    return o


def bwd_workspace_bytes(B: int, H: int, L: int, d: int, m: int, causal: bool, dtype) -> int:
    code = dtype if isinstance(dtype, int) else _dtype_code(_torch().empty(0, dtype=dtype))
    return int(load().favor_bwd_workspace_bytes(B, H, L, d, m, int(bool(causal)), code))


def attn_backward(q, k, v, w, g, causal: bool = False, eps: float = 1e-6, workspace=None):
    """Gradients (dq, dk, dv) of sum(g * attn(q, k, v, w, causal, eps)),
    each with the shape and dtype of q.  W gets no gradient."""
    lib = load()
    torch = _torch()
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape or g.shape != q.shape:
        raise ValueError("q, k, v, g must share one [B, H, L, d] shape")
    if k.dtype != q.dtype or v.dtype != q.dtype or g.dtype != q.dtype:
        raise TypeError("q, k, v, g must share one dtype")
    B, H, L, d = q.shape
    w, hw = _proj(w, H, (w.shape[-2], d))
    m = int(w.shape[1])
    _check_device(q, k, v, g, w)
    if any(t.device != q.device for t in (k, v, g, w)):
        raise ValueError("q, k, v, g and W must live on one device")
    code = _dtype_code(q)
    need = int(lib.favor_bwd_workspace_bytes(B, H, L, d, m, int(bool(causal)), code))
    if need == 0:
        raise FavorError("favor_bwd_workspace_bytes", 2)
    if workspace is not None:
        _check_workspace(workspace, q.device)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    name = "favor_attn_causal_bwd" if causal else "favor_attn_noncausal_bwd"
    st = getattr(lib, name)(ptr(q), ptr(k), ptr(v), ptr(w), hw, ptr(g), ptr(dq), ptr(dk), ptr(dv),
                            B, H, L, d, m, float(eps), code, ptr(workspace), workspace.numel(), _stream())
    if st != 0:
        raise FavorError(name, st)
    return dq, dk, dv


def timing_start(kernel: str, capacity: int) -> None:
    """Time the next `capacity` launches of a kernel with HIP events recorded
    by the library on the launch's own stream."""
    st = load().favor_timing_start(KERNELS[kernel], int(capacity))
    if st != 0:
        raise FavorError("favor_timing_start", st)


def timing_stop(kernel: str, capacity: int = 4096):
    """Per-launch durations (ms) recorded since timing_start, in launch order."""
    buf = (ctypes.c_double * capacity)()
    n = ctypes.c_int(0)
    st = load().favor_timing_stop(KERNELS[kernel], buf, capacity, ctypes.byref(n))
    if st != 0:
        raise FavorError("favor_timing_stop", st)
    return [buf[i] for i in range(min(n.value, capacity))]
