"""Seeded synthetic inputs for FAVOR+ attention.

This module is shared by the float64 oracle (``oracle/``), the tests and the
benchmark, and by nothing else.  It holds random-number generation and dtype
plumbing only: no step of the attention method's arithmetic lives here.  The
random projection ``W`` is drawn here because the method consumes it as an input
(the library takes ``W`` as an argument and never samples it).

Workloads (all values seeded; see ``WORKLOADS``):

* ``t1``       -- the worked example of "Linear Attention > Performer: Unbiased
                  Softmax Approximation" (experiment cell In[26] and the
                  projection sampled inside In[25]): n=64, d=32, legacy
                  ``RandomState`` streams, seed 42 for Q, K, V and seed 0 for the
                  projection.
* ``encoder``  -- B=8, H=12, L=4096, d=64, m=256, bf16, non-causal.
* ``causal_lm``-- B=4, H=16, L=16384, d=64, m=256, bf16, causal.
* ``long``     -- B=1, H=8, L=65536, d=64, m=256, bf16, both paths.
* ``wide``     -- B=2, H=32, L=32768, d=128, m=512, fp32, causal.

bf16 values are produced with round-to-nearest-even from float32 and are
returned both as raw uint16 bit patterns (what the device receives) and as
their exact float32 values (what the oracle receives, upcast to float64).
"""
from __future__ import annotations

import dataclasses

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "bf16_round", "bf16_bits_to_f32",
    "t1_qkv", "t1_projection", "iid_projection", "orthogonal_projection",
    "make_inputs", "random_case", "as_f64", "upstream_gradient",
]


# --------------------------------------------------------------------------
# dtype plumbing
# --------------------------------------------------------------------------

def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the uint16 bit patterns.  NaN is not expected in synthetic data.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact float32 value of bfloat16 bit patterns."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# --------------------------------------------------------------------------
# the worked example's streams (legacy Mersenne-Twister RandomState)
# --------------------------------------------------------------------------

def t1_qkv(n: int = 64, d: int = 32):
    """Q, K, V of the worked example: seed 42, Q and K are 0.3 * N(0,1) and V
    is N(0,1), drawn in the order Q, K, V, each rounded to float32 before the
    0.3 scale (which is applied in float32)."""
    rs = np.random.RandomState(42)
    q = rs.randn(n, d).astype(np.float32) * np.float32(0.3)
    k = rs.randn(n, d).astype(np.float32) * np.float32(0.3)
    v = rs.randn(n, d).astype(np.float32)
    return q, k, v


def t1_projection(m: int, d: int = 32) -> np.ndarray:
    """Projection of the worked example: seed 0, a (d, m) standard-normal
    matrix divided by sqrt(d), float64.  Returned transposed, as the rows
    omega_i, with shape (m, d)."""
    rs = np.random.RandomState(0)
    r = rs.randn(d, m) / np.sqrt(d)
    return np.ascontiguousarray(r.T)


# --------------------------------------------------------------------------
# projection samplers
# --------------------------------------------------------------------------

def iid_projection(rng: np.random.Generator, heads: int, m: int, d: int,
                   scale: float = 1.0) -> np.ndarray:
    """Rows omega_i ~ N(0, scale^2 I_d), independent.  Shape (heads, m, d),
    float64."""
    return rng.standard_normal((heads, m, d)) * scale


def orthogonal_projection(rng: np.random.Generator, heads: int, m: int, d: int) -> np.ndarray:
    """Orthogonal random features, one matrix per head, shape (heads, m, d),
    float64.

    Each head stacks ceil(m/d) blocks of d mutually orthogonal unit rows; a
    block is the orthogonal factor of the QR decomposition of a d x d standard
    Gaussian matrix with the column signs fixed by the signs of diag(R), which
    makes it Haar distributed.  Every row is then given an independent
    chi(d) length (the norm of a fresh N(0, I_d) draw), so each row is
    marginally N(0, I_d) while rows inside one block stay orthogonal.
    """
    nblk = -(-m // d)
    out = np.empty((heads, m, d))
    for h in range(heads):
        rows = []
        for _ in range(nblk):
            g = rng.standard_normal((d, d))
            qm, rm = np.linalg.qr(g)
            qm = qm * np.sign(np.diag(rm))[None, :]
            rows.append(qm.T)          # rows of Q^T are orthonormal
        blk = np.concatenate(rows, axis=0)[:m]
        lengths = np.linalg.norm(rng.standard_normal((m, d)), axis=1)
        out[h] = blk * lengths[:, None]
    return out


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    L: int
    d: int
    m: int
    dtype: str            # "bf16" or "f32"
    paths: tuple          # subset of ("noncausal", "causal")
    qk_std: float         # std of Q, K entries before the d^-1/4 scale
    qk_prescale: bool     # multiply Q, K by d^-1/4
    eps: float
    seed_data: int
    seed_w: int
    chunk: int = 64

    @property
    def tokens(self) -> int:
        return self.B * self.H * self.L


WORKLOADS = {
    "t1": Workload("t1", 1, 1, 64, 32, 256, "f32", ("noncausal",), 0.3, False, 1e-6, 42, 0),
    "encoder": Workload("encoder", 8, 12, 4096, 64, 256, "bf16", ("noncausal",), 1.0, True, 1e-6, 1002, 2002),
    "causal_lm": Workload("causal_lm", 4, 16, 16384, 64, 256, "bf16", ("causal",), 1.0, True, 1e-6, 1003, 2003),
    "long": Workload("long", 1, 8, 65536, 64, 256, "bf16", ("noncausal", "causal"), 1.0, True, 1e-6, 1004, 2004),
    "wide": Workload("wide", 2, 32, 32768, 128, 512, "f32", ("causal",), 0.5, True, 1e-6, 1005, 2005),
}


def _draw(rng, shape, std):
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def make_inputs(wl: Workload, B: int | None = None, H: int | None = None, L: int | None = None,
                heads_w: int | None = None, with64: bool = True):
    """Seeded inputs of a workload, optionally cut down to B x H x L.

    A cut is drawn at its own shape from the workload's seeds, so each cut is
    its own seeded case (it is not a slice of the full-size tensors).

    Returns a dict with
      q, k, v  -- device-format arrays: uint16 bf16 bits or float32, (B,H,L,d)
      q64, k64, v64 -- their exact values as float64 (omitted when
                       ``with64`` is false; ``as_f64`` converts on demand)
      w        -- float32 projection (Hw, m, d), Hw = H (one per head) unless
                  ``heads_w`` says otherwise
      w64      -- its exact values as float64
    """
    B = wl.B if B is None else B
    H = wl.H if H is None else H
    L = wl.L if L is None else L
    Hw = H if heads_w is None else heads_w
    d, m = wl.d, wl.m
    if wl.name == "t1":
        if (B, H) != (1, 1):
            raise ValueError("the worked example is a single head")
        q, k, v = (x.reshape(1, 1, L, d) for x in t1_qkv(L, d))
        w = t1_projection(m, d).astype(np.float32)[None]
    else:
        rng = np.random.default_rng(wl.seed_data)
        shape = (B, H, L, d)
        scale = wl.qk_std * (d ** -0.25 if wl.qk_prescale else 1.0)
        q = _draw(rng, shape, scale)
        k = _draw(rng, shape, scale)
        v = _draw(rng, shape, 1.0)
        w = orthogonal_projection(np.random.default_rng(wl.seed_w), Hw, m, d).astype(np.float32)
    out = {"w": np.ascontiguousarray(w), "w64": w.astype(np.float64), "dtype": wl.dtype}
    for name, x in (("q", q), ("k", k), ("v", v)):
        if wl.dtype == "bf16":
            out[name] = bf16_round(x)
        else:
            out[name] = np.ascontiguousarray(x, dtype=np.float32)
        if with64:
            out[name + "64"] = as_f64(out[name], wl.dtype)
    return out


def as_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of a device-format array (bf16 bits or float32)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def random_case(seed: int, B: int, H: int, L: int, d: int, m: int, dtype: str,
                qk_scale: float | None = None, heads_w: int | None = None):
    """A small seeded case with the encoder workload's value recipe at an
    arbitrary shape (used for ragged and edge-case parity tests)."""
    rng = np.random.default_rng(seed)
    scale = d ** -0.25 if qk_scale is None else qk_scale
    shape = (B, H, L, d)
    q = _draw(rng, shape, scale)
    k = _draw(rng, shape, scale)
    v = _draw(rng, shape, 1.0)
    Hw = H if heads_w is None else heads_w
    w = orthogonal_projection(rng, Hw, m, d).astype(np.float32)
    out = {"w": np.ascontiguousarray(w), "w64": w.astype(np.float64), "dtype": dtype}
    for name, x in (("q", q), ("k", k), ("v", v)):
        out[name] = bf16_round(x) if dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)
        out[name + "64"] = as_f64(out[name], dtype)
    return out



def upstream_gradient(seed: int, shape, dtype: str):
    """A seeded upstream gradient dLoss/dO for the backward pass: N(0, 1)
    entries in device format (bf16 bits or float32) and their exact float64
    values."""
    g = _draw(np.random.default_rng(seed), tuple(shape), 1.0)
    dev = bf16_round(g) if dtype == "bf16" else np.ascontiguousarray(g, dtype=np.float32)
    return dev, as_f64(dev, dtype)
