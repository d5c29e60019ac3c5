#!/usr/bin/env python3
"""HBM traffic of the step's dominant kernels, from rocprofv3 counters.

`python bench_traffic.py collect OUTDIR` runs, on a GPU host:
  1. `rocprofv3 --pmc FETCH_SIZE` and then `--pmc WRITE_SIZE` (separate runs)
     over two bench.py steps of the 124M workload;
  2. the same two counters over a plain device-to-device copy of 1 GiB, whose
     bytes are known, to scale the counters' KiB readings to bytes.
`python bench_traffic.py summarize OUTDIR DEST` turns the CSVs into DEST
(JSON text): per timing label, the calibrated fetch and write bytes per launch,
the command lines, the calibration factors, and a SHA-256 of the kernel sources
so that bench.py reports the figures only while the kernels are unchanged.
`python bench_traffic.py copy` is the calibration program itself.
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import re
import subprocess
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "decoder_only_transformer_04_amd", "csrc")
COPY_BYTES = 1 << 30
BENCH_ARGS = ["--steps", "2", "--warmup", "1", "--no-breakdown", "--no-cpu-baseline"]

# timing label -> (kernel-name pattern, which dispatches of a step): "all" of
# them, or "longest" (the one longest dispatch per step, for a template and grid
# that another label shares with shorter launches)
LABELS = {
    "gemm.dgrad.fc2": (r"gemm_bf16_kernel<128, 128, 32, true, false, 4,", "all"),
    "gemm.dgrad.head": (r"gemm_bf16_kernel<192, 192, 64, true, false, 3, 2, 2, 2, 2, false, true>", "longest"),
    "gemm.fwd.head": (r"gemm_bf16_kernel<256, 256, 64, true, true, 0,", "all"),
    "gemm.fwd.fc2": (r"gemm_bf16_kernel<192, 192, 64, true, true, 2,", "all"),
    "gemm.fwd.fc": (r"gemm_bf16_kernel<128, 128, 64, true, true, 1, 2, 4, 2,", "all"),
    "gemm.wgrad.head": (r"gemm_bf16_kernel<256, 256, 64, false, false, 3,", "longest"),
    "attn.fwd": (r"attn_fwd_d64", "all"),
    "attn.bwd.dq": (r"attn_bwd_dq_d64", "all"),
    "attn.bwd.dkdv": (r"attn_bwd_dkdv_d64", "all"),
    "ce": (r"ce_reg_kernel", "all"),
    "adamw": (r"adamw_kernel", "all"),
    "ln.bwd": (r"ln_bwd_v4", "all"),
}


def source_hash() -> str:
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(CSRC, "*"))):
        if f.endswith((".hip", ".h", ".cpp")):
            h.update(os.path.basename(f).encode())
            with open(f, "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()


def copy_main():
    import torch
    n = COPY_BYTES // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    y.copy_(x)
    torch.cuda.synchronize()
    print("copied", COPY_BYTES, "bytes", flush=True)


def run(cmd, log):
    print("+", " ".join(cmd), flush=True)
    env = dict(os.environ, TMPDIR="/tmp")
    with open(log, "w") as fh:
        r = subprocess.run(cmd, stdout=fh, stderr=subprocess.STDOUT, timeout=300, cwd="/tmp", env=env)
    if r.returncode != 0:
        sys.exit(f"command failed ({r.returncode}), see {log}")


def collect(out):
    os.makedirs(out, exist_ok=True)
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        for what, prog in (("bench", [sys.executable, os.path.join(ROOT, "bench.py")] + BENCH_ARGS),
                           ("copy", [sys.executable, os.path.abspath(__file__), "copy"])):
            d = os.path.join(out, f"{what}_{counter.lower()}")
            run(["rocprofv3", "--pmc", counter, "-d", d, "-o", "run", "--output-format", "csv", "--"] + prog,
                d + ".log")


def read_counter(d):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    rows = []
    for f in files:
        rows += list(csv.DictReader(open(f)))
    return rows


def summarize(out, dest):
    res = {"source_sha256": source_hash(), "bench_command": "python3 bench.py " + " ".join(BENCH_ARGS),
           "copy_bytes": COPY_BYTES, "labels": {}}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        key = counter.lower()
        copy_rows = [r for r in read_counter(os.path.join(out, f"copy_{key}")) if r["Counter_Name"] == counter]
        # the copy kernel is the dispatch with the largest reading
        kib = max(float(r["Counter_Value"]) for r in copy_rows)
        factor = COPY_BYTES / (kib * 1024.0)
        res[f"{key}_calibration"] = {"copy_kib": kib, "bytes_per_kib_reading": factor * 1024.0}
        rows = [r for r in read_counter(os.path.join(out, f"bench_{key}")) if r["Counter_Name"] == counter]
        for label, (pat, sel) in LABELS.items():
            hits = [r for r in rows if re.search(pat, r["Kernel_Name"])]
            if not hits:
                continue
            if sel == "longest":
                hits.sort(key=lambda r: int(r["End_Timestamp"]) - int(r["Start_Timestamp"]), reverse=True)
                hits = hits[:3]  # one per step (3 steps: warm-up + 2)
            vals = [float(r["Counter_Value"]) * 1024.0 * factor for r in hits]
            ent = res["labels"].setdefault(label, {"kernel": hits[0]["Kernel_Name"][:160]})
            ent[f"{key}_bytes_per_launch"] = sum(vals) / len(vals)
            ent["launches_sampled"] = len(vals)
    with open(dest, "w") as fh:
        json.dump(res, fh, indent=1)
    print(json.dumps(res, indent=1))


if __name__ == "__main__":
    if len(sys.argv) >= 2 and sys.argv[1] == "copy":
        copy_main()
    elif len(sys.argv) >= 3 and sys.argv[1] == "collect":
        collect(sys.argv[2])
    elif len(sys.argv) >= 4 and sys.argv[1] == "summarize":
        summarize(sys.argv[2], sys.argv[3])
    else:
        sys.exit(__doc__)
