"""Measure HBM traffic per kernel launch with rocprofv3 counters for bench.py.

    python traffic.py [--workload long] [--out DIR]   (DIR defaults to counter_runs/)
    python traffic.py --workload long --resummarise STAMP   (re-read the runs of STAMP)

Every counter is collected in a rocprofv3 run of its own (FETCH_SIZE, then
WRITE_SIZE), once per path of the workload (bench.py --paths P, so that a
kernel used by both paths is attributed to the right one), and once more on
bench.py --copy-calibration, a plain device-to-device copy of a known size.
The copy's counter reading gives the scale factor from counter units to
bytes for each counter (bytes copied / counter reading); the kernels'
per-dispatch readings are multiplied by it.

Writes profiles/hbm_traffic.json (read by bench.py, valid while the kernel
sources hash the same) and profiles/hbm_traffic_<workload>.txt (the summary
with the commands that produced it), and copies both into the --out folder.  Needs a GPU; the script itself does
not touch it, each rocprofv3 run is a child process.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import shutil
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import bench  # noqa: E402  (kernel_source_hash, workload table)
import synth  # noqa: E402

COPY_MIB = 1024
COUNTERS = ("FETCH_SIZE", "WRITE_SIZE")


def short_name(kernel_name: str) -> str:
    for k in ("k_reduce", "k_combine", "k_apply", "k_span_scan", "k_causal", "k_features"):
        if k in kernel_name:
            return k
    return kernel_name


def run_pass(counter: str, out_dir: str, prog: list, run: bool = True) -> tuple:
    """One rocprofv3 counter run (or, with run=False, the rows an earlier run
    left in out_dir); returns its counter rows and the command, with the
    repository's own path written as $REPO."""
    cmd = ["timeout", "-s", "KILL", "120", "rocprofv3", "--pmc", counter, "--output-format", "csv",
           "-d", out_dir, "-o", "run", "--", sys.executable, *prog]
    shown = " ".join(["python3" if c == sys.executable else c.replace(ROOT, "$REPO") for c in cmd[4:]])
    if run:
        print("[traffic] " + " ".join(cmd), flush=True)
        env = dict(os.environ, TMPDIR="/tmp")
        r = subprocess.run(cmd, cwd="/tmp", env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        if r.returncode != 0:
            print(r.stdout[-3000:], flush=True)
            raise SystemExit(f"rocprofv3 pass failed ({r.returncode}): {' '.join(cmd)}")
    rows = []
    for f in glob.glob(os.path.join(out_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            rows += [row for row in csv.DictReader(fh) if row.get("Counter_Name") == counter]
    if not rows:
        raise SystemExit(f"no {counter} rows under {out_dir}")
    return rows, shown


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--workload", default="long", choices=list(synth.WORKLOADS))
    ap.add_argument("--out", default=os.path.join(ROOT, "counter_runs"),
                    help="folder for the raw rocprofv3 runs and a copy of the summaries")
    ap.add_argument("--resummarise", metavar="STAMP", default=None,
                    help="rebuild the summary from the runs an earlier call left under --out")
    args = ap.parse_args()
    wl = synth.WORKLOADS[args.workload]
    bench_py = os.path.join(ROOT, "bench.py")
    args.out = os.path.abspath(args.out)      # rocprofv3 runs from /tmp
    stamp = args.resummarise or time.strftime("%Y%m%d-%H%M%S")
    run = args.resummarise is None

    # scale factors from the plain copy (bytes read = bytes written = COPY_MIB MiB)
    scale, commands = {}, []
    for c in COUNTERS:
        rows, cmd = run_pass(c, os.path.join(args.out, f"copy_{c}_{stamp}"),
                             [bench_py, "--copy-calibration", str(COPY_MIB)], run)
        commands.append(cmd)
        vals = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]]
        if not vals:
            raise SystemExit("copy kernel not found in the calibration run")
        reading = sorted(vals)[len(vals) // 2]
        scale[c] = (COPY_MIB << 20) / reading

    per = {}
    for path in wl.paths:
        for c in COUNTERS:
            rows, cmd = run_pass(c, os.path.join(args.out, f"{wl.name}_{path}_{c}_{stamp}"),
                                 [bench_py, "--workload", wl.name, "--paths", path, "--steps", "3", "--warmup", "1", "--no-backward", "--no-fmaps",
                                  "--no-configs", "--settle-ms", "0", "--cpu-seconds", "0"], run)
            commands.append(cmd)
            acc = {}
            for r in rows:
                k = short_name(r["Kernel_Name"])
                if not k.startswith("k_"):
                    continue
                acc.setdefault(k, []).append(float(r["Counter_Value"]) * scale[c])
            for k, v in acc.items():
                per.setdefault(f"{wl.name}/{path}/{k}", {})[c] = sum(v) / len(v)

    rec = {"source_hash": bench.kernel_source_hash(), "workload": wl.name, "scale": scale,
           "copy_bytes": COPY_MIB << 20, "kernels": {}}
    for key, d in sorted(per.items()):
        fetch, write = d.get("FETCH_SIZE", 0.0), d.get("WRITE_SIZE", 0.0)
        rec["kernels"][key] = {"fetch_bytes": round(fetch), "write_bytes": round(write),
                               "bytes_per_launch": round(fetch + write)}
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    old = {}
    try:
        with open(bench.TRAFFIC_FILE) as f:
            old = json.load(f)
    except (OSError, ValueError):
        pass
    if old.get("source_hash") == rec["source_hash"]:       # keep other workloads of the same sources
        old_k = {k: v for k, v in old.get("kernels", {}).items() if not k.startswith(wl.name + "/")}
        rec["kernels"] = {**old_k, **rec["kernels"]}
    with open(bench.TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)

    lines = [f"HBM traffic per launch, workload {wl.name} (rocprofv3 FETCH_SIZE / WRITE_SIZE, one counter per run)",
             f"kernel sources hash {rec['source_hash']}",
             "scale (bytes per counter unit, from a {} MiB device copy): FETCH_SIZE x{:.4g}, WRITE_SIZE x{:.4g}".format(
                 COPY_MIB, scale["FETCH_SIZE"], scale["WRITE_SIZE"]),
             "", f"{'path/kernel':32s} {'fetch MB':>10s} {'write MB':>10s} {'total MB':>10s}"]
    for key, v in sorted(rec["kernels"].items()):
        if not key.startswith(wl.name + "/"):
            continue
        lines.append(f"{key[len(wl.name) + 1:]:32s} {v['fetch_bytes'] / 1e6:10.2f} {v['write_bytes'] / 1e6:10.2f} "
                     f"{v['bytes_per_launch'] / 1e6:10.2f}")
    out_arg = "" if os.path.abspath(args.out) == os.path.join(ROOT, "counter_runs") else \
        " --out " + os.path.relpath(os.path.abspath(args.out), ROOT)
    lines += ["", "made by: python3 traffic.py --workload {}{} ($REPO = the repository root), which runs,".format(
        wl.name, out_arg),
              "from /tmp with TMPDIR=/tmp:"] + ["  " + c for c in commands]
    txt = os.path.join(ROOT, "profiles", f"hbm_traffic_{wl.name}.txt")
    with open(txt, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines), flush=True)
    os.makedirs(args.out, exist_ok=True)
    for src in (bench.TRAFFIC_FILE, txt):
        shutil.copy(src, os.path.join(args.out, os.path.basename(src)))
    return 0


if __name__ == "__main__":
    sys.exit(main())
