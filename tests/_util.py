"""Helpers shared by the GPU tests: device transfer of seeded inputs and the
per-row error metric."""
import numpy as np


def to_device(x: np.ndarray, dtype: str):
    """numpy device-format array (uint16 bf16 bits or float32) -> torch on cuda."""
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.cuda()


def to_f64(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def row_rel_err(out: np.ndarray, ref: np.ndarray) -> float:
    """max over rows of max_c |out - ref| / max_c |ref| (per-row infinity-norm
    relative error; elementwise relative error is ill-posed because outputs
    cross zero)."""
    num = np.abs(out - ref).max(axis=-1)
    den = np.abs(ref).max(axis=-1)
    return float((num / den).max())


def grad_err(out: np.ndarray, ref: np.ndarray, floored: bool = False, floor_frac: float = 2.0 ** -7) -> float:
    """Per-row infinity-norm error of a gradient relative to the row's own
    infinity norm, or (floored=True, used for dQ) relative to max(own norm,
    floor_frac times the largest row of its head).  dq_i is formed from the
    per-feature difference y - z s_i/D_i, which nearly cancels in some rows
    (the first causal query's dq is proportional to eps: its one key gives
    o_0 = v_0 a/(a + eps)); in such a row the error scales with the terms,
    not with the result, at any float precision.  dK and dV are held to
    their own size row by row.  Leading axes other than the last two are
    heads."""
    num = np.abs(out - ref).max(axis=-1)
    row = np.abs(ref).max(axis=-1)
    den = np.maximum(row, floor_frac * row.max(axis=-1, keepdims=True)) if floored else row
    return float((num / den).max())


TOL = {"f32": 1e-4, "bf16": 2e-2}
