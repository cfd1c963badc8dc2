"""Turn rocprofv3 CSV output into the short summaries kept under profiles/.

    python profile_summary.py trace NAME TRACE_DIR "COMMAND ..." [--note TEXT]
        kernel durations (--kernel-trace --stats run) -> profiles/NAME.md
    python profile_summary.py traffic NAME TRACE_DIR FETCH_DIR WRITE_DIR "COMMANDS ..."
        durations plus HBM bytes per dispatch from a --pmc FETCH_SIZE run and a
        --pmc WRITE_SIZE run -> profiles/NAME.md and the NAME record of
        profiles/traffic.json (read by bench.py)

FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are scaled by what they read for
the 1 GiB device copy that bench.py runs as its copy probe (1 GiB read and
1 GiB written): known bytes / counted bytes.  The traffic record carries a
hash of the matvec kernel sources so that bench.py reports the figure only
while the kernels are the ones the counters were taken on.
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import re
import statistics
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
SOURCES = ["gemm_dequant_matvec_amd/csrc/matvec_xs.hip", "gemm_dequant_matvec_amd/csrc/qmv_internal.h"]
COPY_BYTES = 1 << 30


def short(name: str) -> str:
    """Kernel name without namespaces and parameter list."""
    name = name.strip()
    if name.endswith(")"):
        depth = 0
        for i in range(len(name) - 1, -1, -1):
            depth += name[i] == ")"
            depth -= name[i] == "("
            if depth == 0:
                name = name[:i]
                break
    name = re.sub(r"(\w+::|\(anonymous namespace\)::)", "", name)
    return re.sub(r"^void ", "", name.strip())


def _one(pattern: str, d: str) -> str:
    hits = sorted(glob.glob(os.path.join(d, "**", pattern), recursive=True))
    if not hits:
        raise SystemExit(f"no {pattern} under {d}")
    return hits[-1]


def durations(trace_dir: str):
    rows = []
    with open(_one("*kernel_stats.csv", trace_dir)) as f:
        for r in csv.DictReader(f):
            rows.append((short(r["Name"]), int(r["Calls"]), float(r["AverageNs"]), float(r["MinNs"]),
                         float(r["MaxNs"]), float(r["Percentage"])))
    rows.sort(key=lambda t: -t[5])
    return rows


def counters(pmc_dir: str, counter: str):
    """{kernel: [values per dispatch]} in KiB."""
    out = {}
    with open(_one("*counter_collection.csv", pmc_dir)) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            out.setdefault(short(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
    return out


def source_sha() -> str:
    h = hashlib.sha256()
    for f in SOURCES:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]


def duration_table(rows) -> list[str]:
    t = ["| kernel | calls | average ns | min ns | max ns | % time |", "|---|---|---|---|---|---|"]
    for n, c, a, lo, hi, p in rows:
        t.append(f"| `{n}` | {c} | {a:.0f} | {lo:.0f} | {hi:.0f} | {p:.1f} |")
    return t


def main(argv):
    mode, name = argv[0], argv[1]
    note = ""
    if "--note" in argv:
        i = argv.index("--note")
        note = argv[i + 1]
        argv = argv[:i] + argv[i + 2:]
    md = [f"# rocprofv3 summary: {name}", ""]
    if note:
        md += [note, ""]
    if mode == "trace":
        trace_dir, cmd = argv[2], argv[3]
        md += ["Commands (run from the repository root on one MI355X):", "", "```", "cd /tmp && export TMPDIR=/tmp",
               cmd, "```", "", "## Kernel durations (--kernel-trace --stats)", ""]
        md += duration_table(durations(trace_dir))
    elif mode == "traffic":
        trace_dir, fetch_dir, write_dir, cmds = argv[2], argv[3], argv[4], argv[5]
        fetch = counters(fetch_dir, "FETCH_SIZE")
        write = counters(write_dir, "WRITE_SIZE")
        copy = "__amd_rocclr_copyBuffer"
        fscale = COPY_BYTES / (max(fetch[copy]) * 1024)
        wscale = COPY_BYTES / (max(write[copy]) * 1024)
        sha = source_sha()
        md += ["Commands (run from the repository root on one MI355X):", "", "```", "cd /tmp && export TMPDIR=/tmp",
               *cmds.split(" ;; "), "```", "",
               f"Kernel source hash (sha256/16 of {', '.join(SOURCES)}): `{sha}`", "",
               "## Kernel durations (--kernel-trace --stats)", ""]
        md += duration_table(durations(trace_dir))
        md += ["", "## HBM traffic per dispatch (--pmc FETCH_SIZE, then --pmc WRITE_SIZE; median KiB)", "",
               f"Scale factors from the 1 GiB copy probe (known 1 GiB read + 1 GiB write): FETCH_SIZE reads "
               f"{max(fetch[copy]):.0f} KiB -> x{fscale:.4f}; WRITE_SIZE reads {max(write[copy]):.0f} KiB -> "
               f"x{wscale:.4f}.", "",
               "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled HBM bytes |", "|---|---|---|---|"]
        kernels = {}
        for k in sorted(set(fetch) & set(write)):
            fk, wk = statistics.median(fetch[k]), statistics.median(write[k])
            b = (fk * fscale + wk * wscale) * 1024
            kernels[k] = {"fetch_kib": fk, "write_kib": wk, "bytes": b}
            md.append(f"| `{k}` | {fk:.0f} | {wk:.0f} | {b:.0f} |")
        path = os.path.join(ROOT, "profiles", "traffic.json")
        try:
            allrec = json.load(open(path))
        except OSError:
            allrec = {}
        allrec[name] = {"fetch_scale": fscale, "write_scale": wscale, "kernels": kernels,
                        "source_sha": sha, "sources": SOURCES}
        with open(path, "w") as f:
            json.dump(allrec, f, indent=1, sort_keys=True)
            f.write("\n")
    else:
        raise SystemExit(__doc__)
    with open(os.path.join(ROOT, "profiles", f"{name}.md"), "w") as f:
        f.write("\n".join(md) + "\n")
    print(f"wrote profiles/{name}.md")


if __name__ == "__main__":
    main(sys.argv[1:])
