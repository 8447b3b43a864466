"""Turn a rocprofv3 --stats kernel_stats.csv into the markdown summary kept here.

usage: python profiles/make_summary.py <kernel_stats.csv> <out.md> "<title>" "<command>"
"""
import csv
import sys


def main(src, out, title, command):
    rows = list(csv.DictReader(open(src)))
    lines = [f"# {title}", "", "Command (MI355X, ROCm 7.2):", "", "```", command, "```", "",
             "`rocprofv3 --stats` kernel summary, library kernels only:", "",
             "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"]
        if "hyena::" not in name:
            continue
        short = name.split("(")[0].replace("void ", "")
        lines.append(f"| `{short}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} |")
    open(out, "w").write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main(*sys.argv[1:5])
