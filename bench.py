#!/usr/bin/env python3
"""FAVOR+ forward throughput on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload long]

A step is one pass of the whole hot path over one batch of seeded synthetic
input already resident in HBM: for the default workload ("long": B=1, H=8,
L=65536, d=64, m=256, bf16) the non-causal forward and the causal forward of
the same Q, K, V.  `value` is B*H*L / step time, i.e. tokens per second
through both forward variants.  Prints one JSON line on stdout; progress goes
to stderr.

The JSON line also carries
  * "roofline": the dominant kernel's algorithmic bytes (or flops) per launch
    divided by its average launch duration, timed live with HIP events that
    the library records on the launch stream during the timed steps;
  * "cpu_baseline": the float64 NumPy oracle timed on the host cores on a
    bounded sample of the same workload (a reported baseline, not a target);
  * "paths" and "kernels": per-path and per-kernel timings;
  * "backward": the backward pass (gradients of sum(G * O) for a seeded
    upstream gradient G) of each path that has one, timed the same way after
    the forward measurement; it is reported beside `value`, never in it;
  * "feature_maps": the same forward step with each other feature map of
    the Kernel Feature Maps page (ELU + 1, ReLU, random Fourier features),
    also beside `value`.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FAVOR+ fwd tokens/sec (B·H·L/s) causal & non-causal; % of MFMA/HBM roofline"
PEAK_HBM_GBS = 8000.0                      # MI355X HBM3E, GB/s
PEAK_MFMA_TFLOPS = {"bf16": 2500.0, "f32": 157.3}   # dense matrix-core peaks
KERNEL_SOURCES = ["favor_device.hpp", "favor_tiles.hpp", "favor_nc.hip", "favor_causal.hip",
                  "favor_causal3.hip", "favor_x3.hip"]   # forward kernels
SPLIT_ARITHMETIC = ("float32 storage, sums and states; each product as three 16-bit matrix-core products "
                    "(hi*hi + hi*lo + lo*hi of fp16 halves for the projection, bf16 halves elsewhere), "
                    "float32 accumulation")
BWD_KERNELS = ["k_bprep", "k_bred", "k_bcombine", "k_bside_q", "k_bside_k"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")


def causal_chunk(wl) -> int:
    """Tokens per chunk of the causal scan: both scans carry the state every
    32 tokens (their registers hold a 32-token chunk)."""
    return 32


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "random_feature_approx_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic(kernel: str, path: str, wl) -> dict:
    """Algorithmic work of one launch: bytes the method must move and flops it
    must do for the tokens that launch processes (per token: the non-causal
    K side and Q side each move 2*d*s bytes and do 4*m*d flops; the causal
    scan moves Q, K, V, O (4*d*s) and does 8*m*d)."""
    T = wl.tokens
    s = 2 if wl.dtype == "bf16" else 4
    d, m = wl.d, wl.m
    if kernel == "k_causal":
        return {"bytes": 4 * d * s * T, "flops": 8 * m * d * T}
    if kernel in ("k_reduce", "k_apply"):
        return {"bytes": 2 * d * s * T, "flops": 4 * m * d * T}
    if kernel in ("k_combine", "k_span_scan"):
        return {"bytes": 0, "flops": 0}
    # backward (the features of each side are computed by two kernels each;
    # per launch of the reduction: read X and Y (2ds), projection and
    # phi^T Y (4md); non-causal query side: read Q, G, write dQ (3ds),
    # projection, y = M g and W^T (phi * dphi) (6md); key side: read K, V,
    # write dK, dV (4ds), projection, dM^T phi, dM v and W^T (phi * dphi)
    # (8md).  Causal: the query side also reads K, V for the state (5ds,
    # plus the state update 2md: 8md); the key side also reads Q, G (6ds,
    # plus the projection of Q and the update 4md: 12md).  The timed "launch"
    # of a side is every kernel launch of that side in one call.)
    if kernel == "k_bred":
        return {"bytes": 2 * d * s * T, "flops": 4 * m * d * T}
    if kernel == "k_bside_q":
        if path == "causal":
            return {"bytes": 5 * d * s * T, "flops": 8 * m * d * T}
        return {"bytes": 3 * d * s * T, "flops": 6 * m * d * T}
    if kernel == "k_bside_k":
        if path == "causal":
            return {"bytes": 6 * d * s * T, "flops": 12 * m * d * T}
        return {"bytes": 4 * d * s * T, "flops": 8 * m * d * T}
    return {"bytes": 0, "flops": 0}


def split_products(wl, path: str, kernel: str) -> bool:
    """True for the kernels the library runs on split 16-bit products: the
    causal scan and its span sums for float32 FAVOR+ at d = 128, unless
    FAVOR_F32_MFMA=1 selects float32 products."""
    forced = int(os.environ.get("FAVOR_F32_MFMA", "0") or 0) > 0
    return (wl.dtype == "f32" and wl.d == 128 and path == "causal" and kernel in ("k_causal", "k_reduce")
            and not forced)


def roofline_entry(kernel: str, path: str, wl, avg_ms: float, traffic) -> dict:
    a = algorithmic(kernel, path, wl)
    t = avg_ms * 1e-3
    split = split_products(wl, path, kernel)
    # split products: the matrix cores execute three bf16/fp16 products per
    # float32 one, against the bf16 dense peak
    peak_mfma = PEAK_MFMA_TFLOPS["bf16" if split else wl.dtype]
    executed = 3 * a["flops"] if split else a["flops"]
    intensity = executed / a["bytes"] if a["bytes"] else float("inf")
    ridge = peak_mfma * 1e12 / (PEAK_HBM_GBS * 1e9)
    if intensity <= ridge:
        achieved = a["bytes"] / t / 1e9
        entry = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                 "frac": round(achieved / PEAK_HBM_GBS, 4)}
    else:
        achieved = executed / t / 1e12
        entry = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak_mfma, "unit": "TFLOP/s",
                 "frac": round(achieved / peak_mfma, 4)}
    if split:
        entry["arithmetic"] = "split: 3 bf16/fp16 products per float32 product"
        entry["executed_flops_per_launch"] = executed
        entry["f32_equivalent_tflops"] = round(a["flops"] / t / 1e12, 2)
        entry["f32_equivalent_frac"] = round(a["flops"] / t / 1e12 / PEAK_MFMA_TFLOPS["f32"], 4)
    entry["traffic"] = traffic
    entry["kernel"] = kernel
    entry["path"] = path
    entry["avg_launch_ms"] = round(avg_ms, 5)
    entry["alg_bytes_per_launch"] = a["bytes"]
    entry["alg_flops_per_launch"] = a["flops"]
    entry["mfma_frac_alg"] = round(executed / t / 1e12 / peak_mfma, 4)
    entry["hbm_frac_alg"] = round(a["bytes"] / t / 1e9 / PEAK_HBM_GBS, 4)
    return entry


def stored_traffic(kernel: str, path: str, workload: str):
    """HBM bytes per launch measured with rocprofv3 counters (scaled by a
    plain copy kernel), valid only while the kernel sources are unchanged."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != kernel_source_hash():
        return None
    e = rec.get("kernels", {}).get(f"{workload}/{path}/{kernel}")
    return None if e is None else e.get("bytes_per_launch")


def cpu_baseline(wl, x, seconds: float) -> dict:
    """Time the float64 oracle on whole heads of the workload until about
    `seconds` per path have elapsed; report tokens/s for a full step (every
    path over the same tokens)."""
    import numpy as np
    import oracle
    import synth
    try:
        import threadpoolctl
        threads = max([p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()] or [1])
    except Exception:
        threads = 1
    heads = [(b, h) for b in range(wl.B) for h in range(wl.H)]
    per_token_s = {}
    sample = []
    for path in wl.paths:
        fn = oracle.attn_causal if path == "causal" else oracle.attn_noncausal
        done, elapsed = 0, 0.0
        for b, h in heads:
            q, k, v = (synth.as_f64(x[n][b, h], wl.dtype) for n in ("q", "k", "v"))
            w = x["w"][h if x["w"].shape[0] > 1 else 0].astype(np.float64)
            t0 = time.perf_counter()
            fn(q, k, v, w, eps=wl.eps)
            elapsed += time.perf_counter() - t0
            done += 1
            if elapsed >= seconds:
                break
        per_token_s[path] = elapsed / (done * wl.L)
        sample.append(f"{path}: {done} of {len(heads)} heads ({done * wl.L} tokens, {elapsed:.1f} s)")
        log(f"cpu oracle {path}: {done} heads in {elapsed:.1f} s")
    value = 1.0 / sum(per_token_s.values())
    return {"value": round(value, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "float64 NumPy oracle on whole heads of the same workload; " + "; ".join(sample)}


def backward_leg(favor, torch, wl, q, k, v, w, to_dev, K: int, warmup: int) -> dict:
    """Time the backward pass of every path that has one: K untimed warmup
    calls, K calls bracketed by two events, then K more with the library's
    per-launch kernel events (outside the timed region)."""
    import synth
    g_np, _ = synth.upstream_gradient(wl.seed_data + 6000, (wl.B, wl.H, wl.L, wl.d), wl.dtype)
    g = to_dev(g_np)
    out = {}
    for path in wl.paths:
        causal = path == "causal"
        code = favor.BF16 if wl.dtype == "bf16" else favor.F32
        ws = torch.empty(favor.bwd_workspace_bytes(wl.B, wl.H, wl.L, wl.d, wl.m, causal, code),
                         dtype=torch.uint8, device=q.device)

        def run():
            return favor.attn_backward(q, k, v, w, g, causal=causal, eps=wl.eps, workspace=ws)

        for _ in range(warmup):
            run()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(K):
            run()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / K
        log(f"backward {path}: {ms:.4f} ms per call")
        for kname in BWD_KERNELS:
            favor.timing_start(kname, 2 * K + 4)
        for _ in range(K):
            run()
        torch.cuda.synchronize()
        kern = {}
        for kname in BWD_KERNELS:
            durs = favor.timing_stop(kname, 2 * K + 4)
            if not durs:
                continue
            n_per = len(durs) // K if len(durs) >= K else 1
            avg = sum(durs) / len(durs)
            entry = {"avg_ms": round(avg, 5), "launches_per_call": n_per}
            if algorithmic(kname, path, wl)["bytes"]:
                r = roofline_entry(kname, path, wl, avg, None)
                entry.update(hbm_frac_alg=r["hbm_frac_alg"], mfma_frac_alg=r["mfma_frac_alg"])
            kern[kname] = entry
        dom = max((kn for kn in kern if algorithmic(kn, path, wl)["bytes"]), key=lambda kn: kern[kn]["avg_ms"])
        out[path] = {"ms": round(ms, 5), "tokens_per_s": round(wl.tokens / (ms * 1e-3), 1), "kernels": kern,
                     "roofline": roofline_entry(dom, path, wl, kern[dom]["avg_ms"], None)}
    return out


def fmap_leg(favor, torch, wl, q, k, v, w, outs, K: int, warmup: int) -> dict:
    """Time the forward step (every path) with each non-FAVOR+ feature map."""
    out = {}
    code = favor.BF16 if wl.dtype == "bf16" else favor.F32
    for kind in ("elu1", "relu", "trig"):
        wss = {p: torch.empty(favor.workspace_bytes(wl.B, wl.H, wl.L, wl.d, wl.m, p == "causal", code, fmap=kind),
                              dtype=torch.uint8, device=q.device) for p in wl.paths}

        def step():
            for p in wl.paths:
                favor.attn(q, k, v, w, causal=(p == "causal"), eps=wl.eps, out=outs[p], workspace=wss[p], fmap=kind)

        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(K):
            step()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / K
        log(f"feature map {kind}: {ms:.4f} ms per step")
        out[kind] = {"ms_per_step": round(ms, 5), "tokens_per_s": round(wl.tokens / (ms * 1e-3), 1),
                     "features": 2 * wl.m if kind == "trig" else wl.m}
    return out


def measure(favor, torch, np, synth, wl, K: int, warmup: int, settle_ms: float, with_traffic: bool,
            graph: bool = False) -> dict:
    """One workload: settle the clock, W warmup steps, K timed steps (no
    other events on the stream), then K more steps with per-path events and
    the library's per-launch kernel events for the per-path and per-kernel
    figures and the dominant kernel's roofline."""
    log(f"workload {wl.name}: B={wl.B} H={wl.H} L={wl.L} d={wl.d} m={wl.m} {wl.dtype} paths={wl.paths}")
    x = synth.make_inputs(wl, with64=False)
    dev = torch.device("cuda", 0)

    def to_dev(a):
        if wl.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    q, k, v = (to_dev(x[n]) for n in ("q", "k", "v"))
    w = torch.from_numpy(x["w"]).to(dev)
    outs = {p: torch.empty_like(q) for p in wl.paths}
    wss = {}
    for p in wl.paths:
        nbytes = favor.workspace_bytes(wl.B, wl.H, wl.L, wl.d, wl.m, p == "causal",
                                       favor.BF16 if wl.dtype == "bf16" else favor.F32)
        wss[p] = torch.empty(nbytes, dtype=torch.uint8, device=dev)

    def run(path):
        favor.attn(q, k, v, w, causal=(path == "causal"), eps=wl.eps, out=outs[path], workspace=wss[path])

    if settle_ms > 0:
        t_end = time.perf_counter() + settle_ms * 1e-3
        while time.perf_counter() < t_end:
            for p in wl.paths:
                run(p)
            torch.cuda.synchronize()
    for _ in range(warmup):
        for p in wl.paths:
            run(p)
    torch.cuda.synchronize()
    log(f"clock settle {settle_ms:.0f} ms, warmup {warmup} steps done")

    # the timed steps carry no per-kernel or per-path events: events between
    # launches add idle time to the stream
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(K):
        for p in wl.paths:
            run(p)
    stop.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(stop) / K
    log(f"timed {K} steps: {ms_step:.4f} ms/step")

    # a second pass of K steps, outside the timed region, gives per-path times
    # and per-launch kernel durations (HIP events the library records on the
    # launch stream)
    kernels = list(favor.KERNELS)
    for kname in kernels:
        favor.timing_start(kname, 2 * K + 4)
    ev = {p: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
          for p in wl.paths}
    torch.cuda.synchronize()
    for i in range(K):
        for p in wl.paths:
            ev[p][i][0].record()
            run(p)
            ev[p][i][1].record()
    torch.cuda.synchronize()

    path_ms = {p: sum(a.elapsed_time(b) for a, b in ev[p]) / K for p in wl.paths}
    # per-kernel launch durations; a kernel used by both paths alternates in
    # launch order (non-causal first within a step)
    per_kernel = {}
    for kname in kernels:
        durs = favor.timing_stop(kname, 2 * K + 4)
        if not durs:
            continue
        users = [p for p in wl.paths if kname in ("k_reduce",) or
                 (kname in ("k_combine", "k_apply") and p == "noncausal") or
                 (kname in ("k_span_scan", "k_causal") and p == "causal")]
        for j, p in enumerate(users):
            mine = durs[j::len(users)]
            per_kernel[f"{p}/{kname}"] = {"avg_ms": sum(mine) / len(mine), "launches": len(mine)}
    dom_key = max(per_kernel, key=lambda k: per_kernel[k]["avg_ms"])
    dom_path, dom_kernel = dom_key.split("/")
    traffic = stored_traffic(dom_kernel, dom_path, wl.name) if with_traffic else None
    roof = roofline_entry(dom_kernel, dom_path, wl, per_kernel[dom_key]["avg_ms"], traffic)
    kern_report = {}
    for key, val in per_kernel.items():
        p, kn = key.split("/")
        r = roofline_entry(kn, p, wl, val["avg_ms"], None) if algorithmic(kn, p, wl)["bytes"] else {}
        kern_report[key] = {"avg_ms": round(val["avg_ms"], 5), "launches": val["launches"],
                            "hbm_frac_alg": r.get("hbm_frac_alg"), "mfma_frac_alg": r.get("mfma_frac_alg")}
    paths_report = {p: {"ms": round(path_ms[p], 5), "tokens_per_s": round(wl.tokens / (path_ms[p] * 1e-3), 1)}
                    for p in wl.paths}
    res = {"ms_per_step": round(ms_step, 5), "roofline": roof, "kernels": kern_report, "paths": paths_report,
           "_inputs": (x, q, k, v, w, outs, to_dev)}
    if graph:
        # the step captured once as a HIP graph and replayed (no per-call
        # host work); every replay writes the eager outputs bit for bit (the
        # calls enqueue kernels only)
        ref = {p: outs[p].clone() for p in wl.paths}
        g = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for p in wl.paths:
                run(p)
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        start.record()
        for _ in range(K):
            g.replay()
        stop.record()
        torch.cuda.synchronize()
        res["graph_ms_per_step"] = round(start.elapsed_time(stop) / K, 5)
        res["graph_replays_match_eager"] = all(torch.equal(outs[p], ref[p]) for p in wl.paths)
        log(f"graph replay: {res['graph_ms_per_step']:.4f} ms/step, outputs equal to eager: "
            f"{res['graph_replays_match_eager']}")
    return res


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the default warmup (about 20 ms of back-to-back steps) outlasts the
    # shader clock's settling after a burst of work begins: a few ms in, the
    # clock falls from about 2.0 to about 1.5 GHz and climbs back over the
    # next ~10 ms, so a short warmup puts that dip into the timed steps
    ap.add_argument("--warmup", type=int, default=60)
    ap.add_argument("--workload", default="long", choices=["t1", "encoder", "causal_lm", "long", "wide"])
    ap.add_argument("--cpu-seconds", type=float, default=8.0, help="oracle time budget per path (0 = skip)")
    ap.add_argument("--paths", default="", help="comma-separated subset of the workload's paths to run "
                                                "(default: all; used to attribute profiler counters to a path)")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward-pass measurement")
    ap.add_argument("--no-fmaps", action="store_true", help="skip the feature-map variant measurement")
    ap.add_argument("--no-configs", action="store_true", help="skip the other workload configurations")
    ap.add_argument("--config-steps", type=int, default=20, help="timed steps per other configuration")
    ap.add_argument("--config-warmup", type=int, default=5, help="warmup steps per other configuration")
    ap.add_argument("--settle-ms", type=float, default=100.0,
                    help="back-to-back steps run for this long before the warmup steps of each workload, "
                         "so that the shader clock has left its dip at the start of a burst (0 = none)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB mebibytes 5 times (the reference "
                         "kernel for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE) and exit")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 5}))
        return 0
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}): heads are independent, so several "
              "GPUs would each run this library on their own heads; nothing here runs on more than one",
              file=sys.stderr)
        return 2
    if int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py is a single-process benchmark; do not launch it with several ranks", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    import random_feature_approx_amd as favor
    import synth

    favor.load()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    wl = synth.WORKLOADS[args.workload]
    if args.paths:
        keep = [p for p in args.paths.split(",") if p]
        bad = [p for p in keep if p not in wl.paths]
        if bad:
            print(f"workload {wl.name} has no path {bad}", file=sys.stderr)
            return 2
        wl = dataclasses.replace(wl, paths=tuple(keep))
    res = measure(favor, torch, np, synth, wl, args.steps, args.warmup, args.settle_ms, with_traffic=True)
    x, q, k, v, w, outs, to_dev = res.pop("_inputs")
    ms_step = res["ms_per_step"]
    roof = res["roofline"]
    kern_report = res["kernels"]
    path_ms = {p: res["paths"][p]["ms"] for p in wl.paths}
    K = args.steps

    bwd = None if args.no_backward else backward_leg(favor, torch, wl, q, k, v, w, to_dev, K, args.warmup)
    fmaps = None if args.no_fmaps else fmap_leg(favor, torch, wl, q, k, v, w, outs, K, args.warmup)

    tokens = wl.tokens
    value = tokens / (ms_step * 1e-3)
    paths_report = res["paths"]
    configs = None
    if not args.no_configs:
        configs = {}
        for name in ("t1", "encoder", "causal_lm", "wide"):
            if name == wl.name:
                continue
            other = synth.WORKLOADS[name]
            r = measure(favor, torch, np, synth, other, args.config_steps, args.config_warmup, args.settle_ms,
                        with_traffic=True, graph=(name == "t1"))
            r.pop("_inputs")
            configs[name] = {"workload": f"{other.name}: B={other.B} H={other.H} L={other.L} d={other.d} "
                                         f"m={other.m} {other.dtype}, {' + '.join(other.paths)}",
                             "ms_per_step": r["ms_per_step"],
                             "tokens_per_s": round(other.tokens / (r["ms_per_step"] * 1e-3), 1),
                             "dtype": other.dtype,
                             "steps": args.config_steps, "paths": r["paths"], "roofline": r["roofline"],
                             "kernels": r["kernels"]}
            if any(split_products(other, p, "k_causal") for p in other.paths):
                configs[name]["arithmetic"] = SPLIT_ARITHMETIC
            if name == "t1":
                # latency of one call; beside it the same step captured once
                # as a HIP graph and replayed (on this stack a replay of so
                # small a graph is not faster than the eager launches)
                configs[name]["latency_ms"] = r["ms_per_step"]
                configs[name]["graph_ms_per_step"] = r["graph_ms_per_step"]
                configs[name]["graph_replays_match_eager"] = r["graph_replays_match_eager"]
            torch.cuda.empty_cache()
    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(wl, x, args.cpu_seconds)

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded N(0,1) inputs, Q and K scaled as the workload states; orthogonal random W)",
        "config": {"workload": f"{wl.name}: B={wl.B} H={wl.H} L={wl.L} d={wl.d} m={wl.m} {wl.dtype}, "
                               f"{' + '.join(wl.paths)} per step",
                   "B": wl.B, "H": wl.H, "L": wl.L, "d": wl.d, "m": wl.m, "paths": list(wl.paths),
                   "chunk": causal_chunk(wl), "eps": wl.eps},
        "roofline": roof,
        "cpu_baseline": cpu,
        "clock_settle_ms": args.settle_ms,
        "paths": paths_report,
        "configs": configs,
        "kernels": kern_report,
        "backward": bwd,
        "feature_maps": fmaps,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
