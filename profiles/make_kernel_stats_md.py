"""Render a rocprofv3 --stats kernel summary CSV as the markdown table kept here.

Usage: python profiles/make_kernel_stats_md.py <run_kernel_stats.csv> <out.md> <title> <command>
"""
import csv
import sys


def main(src, dst, title, command):
    rows = list(csv.DictReader(open(src)))
    out = [f"# {title}\n\n", "Command (R = repository root on the GPU box):\n\n```\n", command, "\n```\n\n",
           "| Kernel | Calls | Total (us) | Average (us) | Min (us) | Max (us) | % |\n|---|---|---|---|---|---|---|\n"]
    for r in rows:
        name = r["Name"]
        short = name if len(name) < 90 else name[:87] + "..."
        f = lambda k: float(r[k]) / 1e3
        out.append(f"| `{short}` | {r['Calls']} | {f('TotalDurationNs'):.1f} | {f('AverageNs'):.1f} | "
                   f"{f('MinNs'):.1f} | {f('MaxNs'):.1f} | {float(r['Percentage']):.2f} |\n")
    open(dst, "w").write("".join(out))


if __name__ == "__main__":
    main(*sys.argv[1:5])
