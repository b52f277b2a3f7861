"""Exact softmax attention against FAVOR+ on one MI355X: where is the crossover
in L, and how close is FAVOR+ to softmax at the workload shapes.

    python crossover.py [--tokens 2097152] [--d 64] [--m 256]

The study notes ("Performer -- 用随机特征把 softmax attention 拉成线性复杂度",
case 1 and the pitfalls) say FAVOR+ is slower than softmax attention below
L of about 512 (or 1K) and recommend r = 256 features at d = 64.  For each L
the sweep keeps B*H*L fixed (H = 8, B = tokens / (8 L)), so the times compare
the same number of tokens; every call is timed with HIP events around K calls
after a warm-up.  Quality: at each workload shape, FAVOR+ output against the
library's exact softmax (scale 1 on the pre-scaled Q, K of the workloads),
mean cosine similarity of the rows and relative Frobenius error (no page
number exists at these shapes; this is a report, not a parity claim).

Writes profiles/crossover.txt (the table and the command) and prints it.
"""
from __future__ import annotations

import argparse
import os
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)


def timed(torch, fn, K=10, warm=3):
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(K):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / K


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--tokens", type=int, default=1 << 21)
    ap.add_argument("--d", type=int, default=64)
    ap.add_argument("--m", type=int, default=256)
    ap.add_argument("--out", default=os.path.join(ROOT, "profiles", "crossover.txt"))
    args = ap.parse_args()
    import numpy as np
    import torch
    import random_feature_approx_amd as favor
    import synth
    favor.load()
    dev = torch.device("cuda", 0)
    d, m, H = args.d, args.m, 8
    lines = [f"Exact softmax attention vs FAVOR+ (bf16, d={d}, m={m}, H={H}, B*H*L = {args.tokens} tokens per call)",
             "", f"{'L':>7s} {'B':>5s} {'softmax nc ms':>14s} {'favor nc ms':>12s} {'softmax c ms':>13s} "
                 f"{'favor c ms':>11s} {'nc ratio':>9s} {'c ratio':>8s}"]
    cross = {"nc": None, "c": None}
    rng = np.random.default_rng(11)
    for L in [128, 256, 512, 1024, 2048, 4096, 8192, 16384, 32768, 65536]:
        B = max(1, args.tokens // (H * L))
        shape = (B, H, L, d)
        q = (torch.randn(shape, device=dev) * d ** -0.25).to(torch.bfloat16)
        k = (torch.randn(shape, device=dev) * d ** -0.25).to(torch.bfloat16)
        v = torch.randn(shape, device=dev).to(torch.bfloat16)
        w = torch.from_numpy(synth.orthogonal_projection(rng, H, m, d).astype(np.float32)).to(dev)
        o = torch.empty_like(q)
        ws = {c: torch.empty(favor.workspace_bytes(B, H, L, d, m, c, favor.BF16), dtype=torch.uint8, device=dev)
              for c in (False, True)}
        t = {}
        for c in (False, True):
            t[("s", c)] = timed(torch, lambda: favor.softmax_attn(q, k, v, scale=1.0, causal=c, out=o))
            t[("f", c)] = timed(torch, lambda: favor.attn(q, k, v, w, causal=c, out=o, workspace=ws[c]))
        rn, rc = t[("s", False)] / t[("f", False)], t[("s", True)] / t[("f", True)]
        if cross["nc"] is None and rn > 1:
            cross["nc"] = L
        if cross["c"] is None and rc > 1:
            cross["c"] = L
        lines.append(f"{L:7d} {B:5d} {t[('s', False)]:14.4f} {t[('f', False)]:12.4f} {t[('s', True)]:13.4f} "
                     f"{t[('f', True)]:11.4f} {rn:9.2f} {rc:8.2f}")
        print(lines[-1], flush=True)
        del q, k, v, o, ws
    lines += ["", "ratio = softmax time / FAVOR+ time (> 1: FAVOR+ faster)",
              f"first L where FAVOR+ is faster: non-causal {cross['nc']}, causal {cross['c']}", ""]
    # quality against exact softmax at the workload shapes
    lines.append("FAVOR+ against exact softmax (scale 1 on the workloads' d^-1/4-scaled Q, K), bf16:")
    lines.append(f"{'workload':12s} {'path':10s} {'mean row cosine':>16s} {'rel. Frobenius err':>19s}")
    for name in ("encoder", "causal_lm", "long"):
        wl = synth.WORKLOADS[name]
        x = synth.make_inputs(wl, with64=False)
        to = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)  # noqa: E731
        q, k, v = (to(x[n]) for n in ("q", "k", "v"))
        w = torch.from_numpy(x["w"]).to(dev)
        for causal in (False, True):
            fo = favor.attn(q, k, v, w, causal=causal).float()
            so = favor.softmax_attn(q, k, v, scale=1.0, causal=causal).float()
            cos = torch.nn.functional.cosine_similarity(fo.reshape(-1, wl.d), so.reshape(-1, wl.d), dim=1).mean()
            rel = (fo - so).norm() / so.norm()
            lines.append(f"{name:12s} {'causal' if causal else 'noncausal':10s} {cos.item():16.4f} {rel.item():19.4f}")
            print(lines[-1], flush=True)
        del q, k, v, w
        torch.cuda.empty_cache()
    lines += ["", "made by: python3 crossover.py --tokens {} --d {} --m {}".format(args.tokens, d, m)]
    os.makedirs(os.path.dirname(args.out), exist_ok=True)
    with open(args.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))
    return 0


if __name__ == "__main__":
    sys.exit(main())
