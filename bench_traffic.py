"""HBM traffic of the dominant kernel (the SwiGLU up/gate GEMM at 1024 px).

Two steps:

1. ``python bench_traffic.py run`` -- launched under rocprofv3 with one
   counter per run, e.g.

       rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT/fetch -o p -- python3 bench_traffic.py run
       rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT/write -o p -- python3 bench_traffic.py run

   It runs, in this order, a plain elementwise copy with conversion (128 Mi
   float32 read = 512 MiB, 128 Mi bf16 written = 256 MiB, ordinary vector
   loads and stores) and the W13 GEMM with the SwiGLU epilogue in the
   configuration the block uses (dit_gemm_plan: 256 x 256 tiles with the
   last round split along K, plus the fixup pass) on the 1024 px shapes
   (h2 [9216, 4096], W13 [22016, 4096], U [9216, 11008], bf16), a few times
   each.

2. ``python bench_traffic.py summarize OUT/fetch OUT/write`` -- reads the
   two counter CSVs, scales each counter by what it reads for the copy
   (FETCH_SIZE and WRITE_SIZE are in KiB; the copy moves a known byte
   count), and writes profiles/traffic_gemm_w13_1024px.json (+ .md) with
   the per-launch HBM bytes and a hash of gemm.hip's code (comments and
   whitespace removed), so bench.py reports the figure only while the
   kernel code is unchanged.

``python bench_traffic.py stats <run_kernel_stats.csv> <out.md> <title> <command>``
renders a rocprofv3 ``--stats`` kernel summary CSV as the markdown table kept
under profiles/.
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import re
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

COPY_N = 128 << 20  # elements of the calibration copy
COPY_READ, COPY_WRITE = 4 * COPY_N, 2 * COPY_N
T, D, F = 9216, 4096, 11008


def run() -> None:
    import torch

    import diffusion_transformer_image_amd as dit
    torch.cuda.set_device(0)
    src = torch.empty(COPY_N, dtype=torch.float32, device="cuda")
    dst = torch.empty(COPY_N, dtype=torch.bfloat16, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    a = (torch.randn(T, D, generator=g, device="cuda")).to(torch.bfloat16)
    w = (torch.randn(2 * F, D, generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    u = torch.empty(T, F, dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    plan = dit.gemm_plan(T, F, D, swiglu=True)  # what dit_block_fwd runs for this shape
    ws = torch.empty(max(plan["part_bytes"] // 4, 1), dtype=torch.float32, device="cuda")
    for _ in range(3):
        if plan["sk_tiles"]:
            dit.gemm_splitk(a, w, u, plan["sk_tiles"], plan["segs"], ws, swiglu=True)
        else:
            dit.gemm_variant(plan["variant"], a, w, u, swiglu=True)
    torch.cuda.synchronize()
    print("done", flush=True)


def _counter(d: str, name: str):
    f = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not f:
        raise SystemExit(f"no counter CSV under {d}")
    copy, gemm, fix = [], [], []
    for r in csv.DictReader(open(f[0])):
        if r["Counter_Name"] != name:
            continue
        v = float(r["Counter_Value"]) * 1024.0  # KiB -> bytes
        k = r["Kernel_Name"]
        if "gemm_sk_fixup" in k:
            fix.append(v)
        elif "gemm_kernel" in k:
            gemm.append(v)
        elif "copy" in k.lower() and "distribution" not in k:
            copy.append(v)
    if not copy or not gemm:
        raise SystemExit(f"{name}: copy={len(copy)} gemm={len(gemm)} dispatches found")
    # one launch of the product = the tile kernel plus its fixup pass, if any
    return sum(copy) / len(copy), (sum(gemm) + sum(fix)) / len(gemm), f[0]


def code_hash(path: str) -> str:
    """sha256 prefix of a C++/HIP source with its comments and whitespace
    removed (string literals kept): the traffic record stays valid across
    comment-only edits and lapses when the code changes."""
    text = open(path, encoding="utf-8").read()
    tok = re.compile(r'"(?:\\.|[^"\\\n])*"|//[^\n]*|/\*.*?\*/', re.S)
    code = tok.sub(lambda m: m.group(0) if m.group(0).startswith('"') else " ", text)
    code = " ".join(code.split())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def summarize(fetch_dir: str, write_dir: str) -> None:
    cf, gf, _ = _counter(fetch_dir, "FETCH_SIZE")
    cw, gw, _ = _counter(write_dir, "WRITE_SIZE")
    kf, kw = cf / COPY_READ, cw / COPY_WRITE  # counter bytes per real byte
    fetch, write = gf / kf, gw / kw
    algorithmic = 2 * (T * D + 2 * F * D + T * F)
    sha = code_hash(os.path.join(ROOT, "diffusion_transformer_image_amd", "csrc", "gemm.hip"))
    rec = {"kernel": "gemm_kernel + gemm_sk_fixup (h2 * W13^T with the SwiGLU epilogue, split tail as in "
                     "the block), 1024 px shapes",
           "bytes_per_launch": fetch + write, "fetch_bytes": fetch, "write_bytes": write,
           "algorithmic_bytes": algorithmic, "ratio_to_algorithmic": (fetch + write) / algorithmic,
           "copy_calibration": {"read_bytes": COPY_READ, "write_bytes": COPY_WRITE,
                                "fetch_counter_per_byte": kf, "write_counter_per_byte": kw},
           "source_sha256_16": sha}
    out = os.path.join(ROOT, "profiles", "traffic_gemm_w13_1024px")
    json.dump(rec, open(out + ".json", "w"), indent=1)
    md = [f"# HBM traffic of the W13 GEMM (SwiGLU epilogue), 1024 px shapes\n\n",
          "Commands (R = repository root on the GPU box):\n\n```\n",
          "cd /tmp && export TMPDIR=/tmp\n",
          "rocprofv3 --pmc FETCH_SIZE --output-format csv -d $R/gpurun_out/traffic/fetch -o p -- python3 $R/bench_traffic.py run\n",
          "rocprofv3 --pmc WRITE_SIZE --output-format csv -d $R/gpurun_out/traffic/write -o p -- python3 $R/bench_traffic.py run\n",
          "python3 bench_traffic.py summarize gpurun_out/traffic/fetch gpurun_out/traffic/write\n```\n\n",
          f"| Quantity | Bytes per launch |\n|---|---|\n",
          f"| FETCH (calibrated) | {fetch:.4g} |\n| WRITE (calibrated) | {write:.4g} |\n",
          f"| total | {fetch + write:.4g} |\n| algorithmic (h2 + W13 + U) | {algorithmic:.4g} |\n\n",
          f"Copy calibration (float32 -> bf16 elementwise copy, {COPY_READ >> 20} MiB read, "
          f"{COPY_WRITE >> 20} MiB written): FETCH_SIZE reads {kf:.3f} and WRITE_SIZE {kw:.3f} "
          f"counter-bytes per byte.  gemm.hip code hash {sha} (comments and whitespace removed).\n"]
    open(out + ".md", "w").write("".join(md))
    print(json.dumps(rec, indent=1))


def stats(src: str, dst: str, title: str, command: str) -> None:
    rows = list(csv.DictReader(open(src)))
    out = [f"# {title}\n\n", "Command (R = repository root on the GPU box):\n\n```\n", command, "\n```\n\n",
           "| Kernel | Calls | Total (us) | Average (us) | Min (us) | Max (us) | % |\n"
           "|---|---|---|---|---|---|---|\n"]
    for r in rows:
        name = r["Name"]
        short = name if len(name) < 90 else name[:87] + "..."
        us = lambda k: float(r[k]) / 1e3
        out.append(f"| `{short}` | {r['Calls']} | {us('TotalDurationNs'):.1f} | {us('AverageNs'):.1f} | "
                   f"{us('MinNs'):.1f} | {us('MaxNs'):.1f} | {float(r['Percentage']):.2f} |\n")
    open(dst, "w").write("".join(out))


if __name__ == "__main__":
    if sys.argv[1:2] == ["run"]:
        run()
    elif sys.argv[1:2] == ["summarize"]:
        summarize(sys.argv[2], sys.argv[3])
    elif sys.argv[1:2] == ["stats"]:
        stats(*sys.argv[2:6])
    else:
        raise SystemExit(__doc__)
