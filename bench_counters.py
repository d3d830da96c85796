"""Hardware-counter evidence for the block's kernels (rocprofv3 --pmc).

Three steps, each a command of its own:

1. ``python3 bench_counters.py run`` -- the workload, launched once per
   counter pass under rocprofv3 (the program directly after ``--``):

       rocprofv3 --pmc <one pass of counters> --output-format csv -d OUT/<pass> -o p -- python3 bench_counters.py run

   It runs, in this order: a calibration copy (128 Mi float32 read = 512
   MiB, 128 Mi bf16 written = 256 MiB, plain vector loads and stores), the
   row-wise e4m3 quantisation of the four weight matrices (set-up, not
   reported), two steps of the 1024 px block (timestep modulation + one
   block, B = 2, L = 4608), two steps of the same block at B = 1 (the
   per-block shapes of the 60-block stack), then two steps of the 8-bit
   block at B = 2.  Seeded synthetic inputs, bf16.

2. ``python3 bench_counters.py summarize OUT`` -- reads every pass under
   OUT (one sub-directory per pass, named as in PASSES), labels each
   dispatch by its place in the step (the four projections are the first
   to fourth GEMM launch of a step; a split tail's fixup pass is added to
   its GEMM), averages the two steps of each workload, and writes
   profiles/counters_block_1024px.md and .json.

3. ``python3 bench_counters.py commands`` prints the rocprofv3 command of
   every pass.

``python3 bench_counters.py stats <run_kernel_stats.csv> <out.md> <title> <command>``
renders a rocprofv3 ``--stats`` kernel summary CSV as the markdown table kept
under profiles/.

Derived quantities (per kernel and workload):
  * clock = GRBM_GUI_ACTIVE / 8 (the counter sums the 8 XCDs) over the
    dispatch's duration;
  * MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 x 256 CUs x
    4 SIMDs): the fraction of SIMD cycles whose matrix unit is busy (the
    counter advances 16 cycles per 16x16x32 bf16 MFMA, so this equals the
    kernel's FLOPs over the peak at the clock it ran);
  * FLOPs / clock peak = the kernel's algorithmic FLOPs per GPU clock
    (GRBM_GUI_ACTIVE, the kernel's duration in clocks: a counter pass runs
    one dispatch at a time) and CU, against the 4096 dense bf16 FLOPs per
    clock and CU behind the 2.5 PFLOP/s peak -- the MFMA fraction at
    whatever clock the chip ran;
  * waits = SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES (share of a wave's life
    spent waiting on s_waitcnt / barriers), LDS waits likewise;
  * per-wave instruction counts (VALU, of them transcendental, MFMA, LDS);
  * LDS bank conflicts per LDS instruction cycle;
  * DRAM-side bytes: TCC_EA0_RDREQ_DRAM_sum and TCC_EA0_WRREQ_DRAM_sum
    (requests the L2 sends towards memory, which includes hits in the
    memory-side last-level cache) scaled by what the same counters read
    per byte of the calibration copy; FETCH_SIZE / WRITE_SIZE the same way.
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

COPY_N = 128 << 20
COPY_READ, COPY_WRITE = 4 * COPY_N, 2 * COPY_N
CUS, SIMDS, XCDS = 256, 4, 8
FLOP_PER_CLK_CU = 4096  # dense bf16 MFMA, the figure behind the 2.5 PFLOP/s peak at 2.4 GHz

PASSES = {
    "mfma": ["GRBM_GUI_ACTIVE", "SQ_WAVES", "SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES",
             "SQ_INSTS_VALU", "SQ_WAIT_INST_ANY", "SQ_INSTS_LDS", "SQ_INSTS_MFMA"],
    "lds": ["GRBM_GUI_ACTIVE", "SQ_WAVES", "SQ_LDS_BANK_CONFLICT", "SQ_ACTIVE_INST_LDS", "SQ_WAIT_INST_LDS",
            "SQ_INSTS_VALU_TRANS_F32", "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_INSTS_SALU"],
    "dram": ["GRBM_GUI_ACTIVE", "TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_DRAM_sum", "TCC_EA0_WRREQ_sum",
             "TCC_EA0_WRREQ_DRAM_sum"],
    "fetch": ["FETCH_SIZE"],
    "write": ["WRITE_SIZE"],
}


def commands(out: str = "$R/gpurun_out/counters") -> list[str]:
    return [f"rocprofv3 --pmc {' '.join(c)} --output-format csv -d {out}/{p} -o p -- python3 $R/bench_counters.py run"
            for p, c in PASSES.items()]


# ------------------------------------------------------------------ workload
def run() -> None:
    import torch

    import datagen
    import diffusion_transformer_image_amd as dit
    from datagen import device

    torch.cuda.set_device(0)
    src = torch.empty(COPY_N, dtype=torch.float32, device="cuda")
    dst = torch.empty(COPY_N, dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    cfg3 = datagen.get_config("c3")
    w = device.weights_to_device(datagen.block_weights(cfg3), "bf16")
    t, w_t1, w_t2 = datagen.timestep_inputs(cfg3)
    W1, W2 = device.to_device(w_t1, "f32"), device.to_device(w_t2, "f32")
    w8 = {n: w[n] for n in ("mod_bias", "norm1_w", "norm2_w")}
    for name, sname in (("w_qkvg", "s_qkvg"), ("w_o", "s_o"), ("w_13", "s_13"), ("w_2", "s_2")):
        w8[name] = torch.empty(w[name].shape, dtype=torch.uint8, device="cuda")
        w8[sname] = torch.empty(w[name].shape[0], dtype=torch.float32, device="cuda")
        dit.quantize_fp8(w[name], w8[name], w8[sname])
    torch.cuda.synchronize()
    for cfg, fp8 in ((cfg3, False), (datagen.get_config("c4"), False), (cfg3, True)):
        c = dit.config_of(cfg)
        X = device.to_device(datagen.activations(cfg).reshape(cfg.tokens, cfg.hidden), "bf16")
        Y = torch.empty_like(X)
        T = device.to_device(t[:cfg.batch], "f32")
        M = torch.empty((cfg.batch, 6, cfg.hidden), dtype=torch.float32, device="cuda")
        ws = torch.empty(dit.workspace_size_fp8(c) if fp8 else dit.workspace_size(c), dtype=torch.uint8,
                         device="cuda")
        for _ in range(2):
            dit.timestep_mod(c, T, W1, W2, M, ws)
            if fp8:
                dit.block_fwd_fp8(c, w8, X, Y, M, ws)
            else:
                dit.block_fwd(c, w, X, Y, M, ws)
        torch.cuda.synchronize()
        del X, Y, ws
    print("done", flush=True)


# ------------------------------------------------------------------ summary
def _short(name: str) -> str:
    m = re.search(r"dit(?:::|\d+)([a-z_0-9]+?)(?:I|E|\(|<|$)", name)
    if "dit" not in name:
        return "torch"
    for k in ("gemm_sk_fixup", "gemm_kernel", "gemm_pp_kernel", "gemm_fp8_kernel", "attn_kernel", "vtrans_kernel",
              "resid_modnorm_kernel", "resid_kernel", "modnorm_kernel", "tmod_stage1", "tmod_stage2_fewb",
              "tmod_stage2", "qk_prologue_kernel", "quantize_fp8_rows_reg", "quantize_fp8_kernel"):
        if k in name:
            return k
    return m.group(1) if m else name[:40]


def _dispatches(pass_dir: str) -> list[dict]:
    f = glob.glob(os.path.join(pass_dir, "**", "*counter_collection.csv"), recursive=True)
    if not f:
        raise SystemExit(f"no counter CSV under {pass_dir}")
    by = {}
    for r in csv.DictReader(open(f[0])):
        d = by.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"], "grid": int(r["Grid_Size"]),
                                                  "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"]),
                                                  "counters": {}})
        d["counters"][r["Counter_Name"]] = d["counters"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return [by[k] for k in sorted(by)]


def _label(disp: list[dict]) -> list[tuple[str, str, dict]]:
    """(workload, kernel label, counters) per dispatch of the block steps,
    fixup passes merged into their GEMM; plus ("calib", "copy", ...)."""
    out, step, gemm_i, quant_i = [], -1, 0, 0
    gemm_names = ["gemm_qkvg", "gemm_o", "gemm_w13", "gemm_w2"]
    for d in disp:
        k = _short(d["name"])
        if k == "torch":
            if step < 0 and "bfloat16_copy" in d["name"] and not any(w == "calib" for w, _, _ in out):
                out.append(("calib", "copy", d["counters"]))
            continue
        if k == "tmod_stage1":
            step += 1
            gemm_i = quant_i = 0
        if step < 0:  # set-up (the weights' quantisation)
            continue
        wl = WORKLOADS[min(step // 2, len(WORKLOADS) - 1)]
        cnt = dict(d["counters"], DURATION_NS=float(d["ns"]))
        if k in ("gemm_kernel", "gemm_pp_kernel", "gemm_fp8_kernel"):
            out.append((wl, gemm_names[min(gemm_i, 3)], cnt))
            gemm_i += 1
        elif k.startswith("quantize_fp8"):
            out.append((wl, ("quant_og", "quant_u")[min(quant_i, 1)], cnt))
            quant_i += 1
        elif k == "gemm_sk_fixup":
            prev = out[-1][2]  # the fixup pass belongs to the GEMM before it (its time too)
            for c, v in dict(d["counters"], DURATION_NS=float(d["ns"])).items():
                prev[c] = prev.get(c, 0.0) + v
        else:
            label = {"modnorm_kernel": "modnorm1", "resid_modnorm_kernel": "resid1+modnorm2",
                     "resid_kernel": "resid2", "attn_kernel": "attn", "vtrans_kernel": "vtrans",
                     "tmod_stage1": "tmod1", "tmod_stage2_fewb": "tmod2", "tmod_stage2": "tmod2"}.get(k, k)
            out.append((wl, label, cnt))
    return out


WORKLOADS = ["1024px_B2", "1024px_B1", "1024px_B2_fp8"]


def _tokens(wl: str) -> int:
    return 4608 if wl == "1024px_B1" else 9216


def _flops(wl: str, kern: str) -> float | None:
    T = _tokens(wl)
    L, D, F, nq = 4608, 4096, 11008, 10240
    per = {"gemm_qkvg": 2 * D * nq, "gemm_o": 2 * D * D, "gemm_w13": 2 * D * 2 * F, "gemm_w2": 2 * F * D,
           "attn": 4 * L * D}
    return per[kern] * T if kern in per else None


def _bytes(wl: str, kern: str) -> float | None:
    T, D, F = _tokens(wl), 4096, 11008
    # modnorm1: x, h1 bf16; resid1+modnorm2: x, A bf16 in, x1 fp32 and h2
    # bf16 out; resid2: x1 fp32 and M in, x_out bf16 out; the V^T pass: V
    # in, V^T out; W13: h2, W13 and U once.  8-bit block: h1 and h2 leave
    # as one-byte codes; the quantiser reads Og or U once and writes codes
    if wl.endswith("fp8"):
        per = {"modnorm1": 3 * D, "resid1+modnorm2": 9 * D, "resid2": 8 * D, "quant_og": 3 * D, "quant_u": 3 * F}
        if kern == "gemm_w13":
            return T * D + 2 * F * D + 2 * T * F
    else:
        per = {"modnorm1": 4 * D, "resid1+modnorm2": 10 * D, "resid2": 8 * D, "vtrans": 4 * 8 * 128}
        if kern == "gemm_w13":
            return 2 * (T * D + 2 * F * D + T * F)
    v = per.get(kern)
    return v * T if v else None


def summarize(out_dir: str) -> None:
    passes = {p: _label(_dispatches(os.path.join(out_dir, p))) for p in PASSES if os.path.isdir(os.path.join(out_dir, p))}
    # calibration factors (counter units per byte of the copy)
    calib = {}
    for p, rows in passes.items():
        for wl, k, c in rows:
            if wl == "calib":
                calib.update({n: v for n, v in c.items()})
    # per (workload, kernel): average over the two steps of every counter of every pass
    agg: dict = {}
    for p, rows in passes.items():
        for wl, k, c in rows:
            if wl == "calib":
                continue
            e = agg.setdefault((wl, k), {})
            for n, v in c.items():
                key = n if n not in ("GRBM_GUI_ACTIVE", "DURATION_NS") else f"{n}@{p}"
                e.setdefault(key, []).append(v)
    res = {}
    for (wl, k), e in agg.items():
        a = {n: sum(v) / len(v) for n, v in e.items()}
        # GRBM_GUI_ACTIVE is the sum over the 8 XCDs of their busy clocks (its
        # value per dispatch over 8, divided by the dispatch's duration, reads
        # 1.6-2.1 GHz for the long kernels, the shader clock under load)
        clk = a.get("GRBM_GUI_ACTIVE@mfma", 0.0) / XCDS
        dur = a.get("DURATION_NS@mfma")
        r = {"gpu_clocks": clk, "duration_us": dur / 1e3 if dur else None,
             "clock_ghz": clk / dur if dur else None}
        if clk and "SQ_VALU_MFMA_BUSY_CYCLES" in a:
            r["mfma_busy"] = a["SQ_VALU_MFMA_BUSY_CYCLES"] / (clk * CUS * SIMDS)
        fl = _flops(wl, k)
        if fl and clk:
            # the 8-bit products against the FP8 peak (twice the bf16 FLOPs per clock)
            peak = 2 * FLOP_PER_CLK_CU if (wl.endswith("fp8") and k.startswith("gemm")) else FLOP_PER_CLK_CU
            r["flops_per_clk_per_cu"] = fl / clk / CUS
            r["mfma_frac_of_clock_peak"] = fl / clk / CUS / peak
        if "SQ_WAVES" in a and a["SQ_WAVES"]:
            w = a["SQ_WAVES"]
            for n, lab in (("SQ_INSTS_VALU", "valu_per_wave"), ("SQ_INSTS_MFMA", "mfma_per_wave"),
                           ("SQ_INSTS_LDS", "lds_per_wave"), ("SQ_INSTS_VALU_TRANS_F32", "trans_per_wave"),
                           ("SQ_INSTS_SALU", "salu_per_wave")):
                if n in a:
                    r[lab] = a[n] / w
        if a.get("SQ_WAVE_CYCLES"):
            r["wait_frac"] = a.get("SQ_WAIT_INST_ANY", 0.0) / a["SQ_WAVE_CYCLES"]
        if a.get("SQ_ACTIVE_INST_LDS"):
            r["lds_bank_conflict_per_lds_cycle"] = a.get("SQ_LDS_BANK_CONFLICT", 0.0) / a["SQ_ACTIVE_INST_LDS"]
        if a.get("SQ_VALU_MFMA_BUSY_CYCLES") and "SQ_VALU_MFMA_COEXEC_CYCLES" in a:
            r["coexec_per_mfma_busy"] = a["SQ_VALU_MFMA_COEXEC_CYCLES"] / a["SQ_VALU_MFMA_BUSY_CYCLES"]
        for n, cal, lab, nbytes in (("TCC_EA0_RDREQ_DRAM_sum", "TCC_EA0_RDREQ_DRAM_sum", "dram_read_bytes", COPY_READ),
                                    ("TCC_EA0_WRREQ_DRAM_sum", "TCC_EA0_WRREQ_DRAM_sum", "dram_write_bytes", COPY_WRITE),
                                    ("FETCH_SIZE", "FETCH_SIZE", "fetch_bytes", COPY_READ),
                                    ("WRITE_SIZE", "WRITE_SIZE", "write_bytes", COPY_WRITE)):
            if n in a and calib.get(cal):
                r[lab] = a[n] / (calib[cal] / nbytes)
        ab = _bytes(wl, k)
        if ab:
            r["algorithmic_bytes"] = ab
        res[f"{wl}/{k}"] = r
    rec = {"kernels": res, "calibration": {n: v for n, v in calib.items()},
           "sources_sha256_16": {f: code_hash(os.path.join(ROOT, "diffusion_transformer_image_amd", "csrc", f))
                                 for f in ("gemm.hip", "attention.hip", "elementwise.hip", "fp8.hip")}}
    base = os.path.join(ROOT, "profiles", "counters_block_1024px")
    json.dump(rec, open(base + ".json", "w"), indent=1)
    cols = [("duration_us", "us", "{:.1f}"), ("clock_ghz", "GHz", "{:.2f}"), ("mfma_busy", "MFMA busy", "{:.3f}"), ("mfma_frac_of_clock_peak", "FLOPs / clock peak", "{:.3f}"),
            ("wait_frac", "wait share", "{:.2f}"), ("valu_per_wave", "VALU/wave", "{:.0f}"),
            ("trans_per_wave", "trans/wave", "{:.0f}"), ("mfma_per_wave", "MFMA/wave", "{:.0f}"),
            ("lds_per_wave", "LDS/wave", "{:.0f}"), ("lds_bank_conflict_per_lds_cycle", "bank confl.", "{:.3f}"),
            ("coexec_per_mfma_busy", "VALU coexec / MFMA busy", "{:.2f}"),
            ("dram_read_bytes", "DRAM-side read MB", "{:.1f}"), ("dram_write_bytes", "DRAM-side write MB", "{:.1f}"),
            ("fetch_bytes", "FETCH MB", "{:.1f}"), ("write_bytes", "WRITE MB", "{:.1f}"),
            ("algorithmic_bytes", "algorithmic MB", "{:.1f}")]
    md = ["# Hardware counters of the block's kernels, 1024 px\n\n",
          "Commands (R = repository root on the GPU box; one rocprofv3 run per counter pass):\n\n```\n",
          "cd /tmp && export TMPDIR=/tmp\n", "\n".join(commands()), "\n",
          "python3 $R/bench_counters.py summarize $R/gpurun_out/counters\n```\n\n",
          "Workloads: `1024px_B2` = the benchmarked block (B = 2, L = 4608); `1024px_B1` = the same block at "
          "B = 1 (the shapes of each block of the 60-block stack); `1024px_B2_fp8` = the 8-bit block "
          "(row-wise e4m3 projections) at B = 2, its GEMMs' FLOPs / clock peak against the FP8 rate "
          "(8192 FLOPs per clock and CU).  Averages of two steps.  MB columns are "
          "per launch (1e6 bytes), scaled by the counters' reading per byte of a calibration copy; "
          "DRAM-side requests include hits in the memory-side last-level cache.\n\n",
          "| kernel | " + " | ".join(c[1] for c in cols) + " |\n", "|---" * (len(cols) + 1) + "|\n"]
    for key in sorted(res, key=lambda s: (s.split("/")[0], s.split("/")[1])):
        r = res[key]
        cells = []
        for c, _, fmt in cols:
            v = r.get(c)
            if v is None:
                cells.append("")
            elif c.endswith("bytes"):
                cells.append(fmt.format(v / 1e6))
            else:
                cells.append(fmt.format(v))
        md.append(f"| {key} | " + " | ".join(cells) + " |\n")
    md.append(f"\nSource hashes (comments and whitespace removed): {rec['sources_sha256_16']}.\n")
    open(base + ".md", "w").write("".join(md))
    print("".join(md))
    # the W13 launch's HBM-side traffic, which bench.py reports as the
    # roofline's `traffic` while gemm.hip is unchanged
    w13 = res.get("1024px_B2/gemm_w13", {})
    if "fetch_bytes" in w13 and "write_bytes" in w13:
        tr = {"kernel": "gemm_kernel + gemm_sk_fixup (h2 * W13^T with the SwiGLU epilogue, split tail as in the "
                        "block), 1024 px shapes",
              "bytes_per_launch": w13["fetch_bytes"] + w13["write_bytes"], "fetch_bytes": w13["fetch_bytes"],
              "write_bytes": w13["write_bytes"], "algorithmic_bytes": w13["algorithmic_bytes"],
              "ratio_to_algorithmic": (w13["fetch_bytes"] + w13["write_bytes"]) / w13["algorithmic_bytes"],
              "copy_calibration": {"read_bytes": COPY_READ, "write_bytes": COPY_WRITE,
                                   "fetch_counter_per_byte": calib["FETCH_SIZE"] / COPY_READ,
                                   "write_counter_per_byte": calib["WRITE_SIZE"] / COPY_WRITE},
              "source_sha256_16": rec["sources_sha256_16"]["gemm.hip"],
              "counters": "profiles/counters_block_1024px.md"}
        json.dump(tr, open(os.path.join(ROOT, "profiles", "traffic_gemm_w13_1024px.json"), "w"), indent=1)


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


def code_hash(path: str) -> str:
    """sha256 prefix of a C++/HIP source with its comments and whitespace
    removed (string literals kept): a record stays valid across
    comment-only edits and lapses when the code changes."""
    text = open(path, encoding="utf-8").read()
    tok = re.compile(r'"(?:\\.|[^"\\\n])*"|//[^\n]*|/\*.*?\*/', re.S)
    code = tok.sub(lambda m: m.group(0) if m.group(0).startswith('"') else " ", text)
    code = " ".join(code.split())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


if __name__ == "__main__":
    if sys.argv[1:2] == ["run"]:
        run()
    elif sys.argv[1:2] == ["summarize"]:
        summarize(sys.argv[2])
    elif sys.argv[1:2] == ["stats"]:
        stats(*sys.argv[2:6])
    elif sys.argv[1:2] == ["commands"]:
        print("\n".join(commands()))
    else:
        raise SystemExit(__doc__)
