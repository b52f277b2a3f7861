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


TOL = {"f32": 1e-4, "bf16": 2e-2}
