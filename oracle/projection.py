"""Float64 oracle of the on-device projection sampler -- TEST INFRASTRUCTURE
ONLY (tests, the package's smoke entry and the benchmark's CPU leg may use
it; the HIP library never does).

The page's code cell (P1 In[25]) draws a fresh random projection on every
call; the orthogonal variant of P2's key points stacks blocks of mutually
orthogonal rows.  The library can draw W on the device from a seed
(favor_draw_projection); this module draws the same W from the same
definition:

* random numbers: Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
  numbers: as easy as 1, 2, 3", SC 2011), keyed by (seed, 0); the block at
  counter (c, row, head, purpose) gives four 64-bit words;
* normals: each word w gives u = (floor(w / 2^11) + 1/2) 2^-53 in (0, 1); the
  pairs (u0, u1), (u2, u3) go through the Box-Muller transform
  z = sqrt(-2 ln u_a) (cos 2 pi u_b, sin 2 pi u_b); so normal j of (row, head,
  purpose) is component j mod 4 of block (j div 4, row, head, purpose);
* orthogonal rows (purpose 0 fills the d x d block matrices G_b row by row,
  row index b d + i): Q of the QR decomposition of G_b with a positive
  diagonal R (the Haar sign fix), its columns taken as rows b d .. b d + d - 1;
  each row scaled by an independent chi(d) length, the norm of d fresh
  normals (purpose 1, row = feature index); the first m rows are kept;
* independent rows: W[h][f][j] = normal j of (row f, head h, purpose 0);
* every row is finally multiplied by `scale` (1 for N(0, I) rows, 1/sqrt(d)
  for the page code's sampler).
"""
from __future__ import annotations

import math

import numpy as np

__all__ = ["philox4x64", "philox_normals", "draw_projection"]

_M0, _M1 = 0xD2E7470EE14C6C93, 0xCA5A826395121157      # multipliers
_W0, _W1 = 0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B      # key increments (Weyl)
_MASK = (1 << 64) - 1


def philox4x64(ctr, key, rounds: int = 10):
    """Philox4x64 with `rounds` rounds: each round multiplies words 0 and 2 of
    the counter by the two multipliers, takes the high and low 64 bits, and
    mixes the high halves with words 1 and 3 and the key; the key is
    advanced by the Weyl constants between rounds.  Returns four ints."""
    c = [int(x) & _MASK for x in ctr]
    k = [int(x) & _MASK for x in key]
    for _ in range(rounds):
        p0 = _M0 * c[0]
        p1 = _M1 * c[2]
        hi0, lo0 = p0 >> 64, p0 & _MASK
        hi1, lo1 = p1 >> 64, p1 & _MASK
        c = [hi1 ^ c[1] ^ k[0], lo1, hi0 ^ c[3] ^ k[1], lo0]
        k = [(k[0] + _W0) & _MASK, (k[1] + _W1) & _MASK]
    return c


def philox_normals(seed: int, head: int, purpose: int, row: int, n: int) -> np.ndarray:
    """The first n standard normals of (row, head, purpose), float64."""
    out = np.empty(4 * ((n + 3) // 4))
    for c in range(len(out) // 4):
        w = philox4x64([c, row, head, purpose], [seed, 0])
        u = [((x >> 11) + 0.5) * 2.0 ** -53 for x in w]
        for a, b, at in ((0, 1, 0), (2, 3, 2)):
            r = math.sqrt(-2.0 * math.log(u[a]))
            out[4 * c + at] = r * math.cos(2.0 * math.pi * u[b])
            out[4 * c + at + 1] = r * math.sin(2.0 * math.pi * u[b])
    return out[:n]


def draw_projection(seed: int, heads: int, m: int, d: int, orthogonal: bool = True,
                    scale: float = 1.0) -> np.ndarray:
    """W of shape (heads, m, d), float64, by the definition above."""
    W = np.empty((heads, m, d))
    for h in range(heads):
        if not orthogonal:
            for f in range(m):
                W[h, f] = philox_normals(seed, h, 0, f, d)
            continue
        rows = []
        for b in range((m + d - 1) // d):
            G = np.stack([philox_normals(seed, h, 0, b * d + i, d) for i in range(d)])
            q, r = np.linalg.qr(G)
            q = q * np.sign(np.diag(r))[None, :]
            rows.append(q.T)
        blk = np.concatenate(rows, axis=0)[:m]
        lengths = np.array([np.linalg.norm(philox_normals(seed, h, 1, f, d)) for f in range(m)])
        W[h] = blk * lengths[:, None]
    return W * scale
