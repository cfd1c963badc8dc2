"""Turn rocprofv3 CSV output into the short summaries kept under profiles/.

    python profile_summary.py trace NAME TRACE_DIR "COMMAND ..." [--note TEXT]
        kernel durations (--kernel-trace --stats run) -> profiles/NAME.md
    python profile_summary.py traffic NAME TRACE_DIR FETCH_DIR WRITE_DIR "COMMANDS ..."
        durations plus HBM bytes per dispatch from a --pmc FETCH_SIZE run and a
        --pmc WRITE_SIZE run -> profiles/NAME.md and the NAME record of
        profiles/traffic.json (read by bench.py)
    python profile_summary.py pmc NAME KERNEL_REGEX TRACE_DIR "COMMANDS ..." PMC_DIR [PMC_DIR ...]
        kernel durations plus the median per dispatch of every counter collected
        in the --pmc runs, for the kernels whose name matches KERNEL_REGEX, with
        the derived MFMA figures -> profiles/NAME.md

Options: --note TEXT (a paragraph under the title); --span REGEX --replays R
(trace mode: the union of the busy intervals of the dispatches matching REGEX
against the sum of their durations, per replay, to reconcile with an
event-timed step).

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


def counters_all(pmc_dir: str, kregex: str):
    """{counter: [values per matching dispatch]}."""
    out = {}
    with open(_one("*counter_collection.csv", pmc_dir)) as f:
        for r in csv.DictReader(f):
            if re.search(kregex, r["Kernel_Name"]):
                out.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    return out


def span(trace_dir: str, regex: str, replays: int) -> list[str]:
    """Sum of durations vs union of busy intervals of the dispatches matching regex."""
    iv = []
    with open(_one("*kernel_trace.csv", trace_dir)) as f:
        for r in csv.DictReader(f):
            if re.search(regex, r["Kernel_Name"]):
                iv.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    iv.sort()
    total = sum(b - a for a, b in iv)
    union, cur = 0, None
    for a, b in iv:
        if cur is None or a > cur[1]:
            if cur:
                union += cur[1] - cur[0]
            cur = [a, b]
        else:
            cur[1] = max(cur[1], b)
    if cur:
        union += cur[1] - cur[0]
    return ["", f"## Busy time of the dispatches matching `{regex}`", "",
            f"{len(iv)} dispatches over {replays} replays: sum of durations {total / replays / 1e3:.1f} us "
            f"per replay; union of their busy intervals {union / replays / 1e3:.1f} us per replay "
            f"(dispatches overlap by {100 * (1 - union / total):.1f} % of the summed durations)."]


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
    sp = None
    if "--span" in argv:
        i = argv.index("--span")
        sp = (argv[i + 1], int(argv[argv.index("--replays") + 1]))
        j = argv.index("--replays")
        argv = [a for k, a in enumerate(argv) if k not in (i, i + 1, j, j + 1)]
    if mode == "trace":
        trace_dir, cmd = argv[2], argv[3]
        md += ["Commands (run from the repository root on one MI355X):", "", "```", "cd /tmp && export TMPDIR=/tmp",
               cmd, "```", "", "## Kernel durations (--kernel-trace --stats)", ""]
        md += duration_table(durations(trace_dir))
        if sp:
            md += span(trace_dir, *sp)
    elif mode == "pmc":
        kre, trace_dir, cmds, dirs = argv[2], argv[3], argv[4], argv[5:]
        md += ["Commands (run from the repository root on one MI355X):", "", "```", "cd /tmp && export TMPDIR=/tmp",
               *cmds.split(" ;; "), "```", "", "## Kernel durations (--kernel-trace --stats)", ""]
        rows = durations(trace_dir)
        md += duration_table(rows)
        c = {}
        for d in dirs:
            c.update(counters_all(d, kre))
        med = {k: statistics.median(v) for k, v in c.items()}
        md += ["", f"## Counters per dispatch of `{kre}` (median over {max(len(v) for v in c.values())} dispatches)",
               "", "| counter | value |", "|---|---|"]
        md += [f"| {k} | {v:.0f} |" for k, v in sorted(med.items())]
        der = []
        dur = [a for n, _, a, *_ in rows if re.search(kre, n)]
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in med:
            fl = med["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512
            der.append(f"bf16 MFMA flops per dispatch (MOPS x 512): {fl:.4g}")
            if dur:
                der.append(f"at the traced average duration {dur[0]:.0f} ns: {fl / dur[0] / 1e3:.1f} TFLOP/s, "
                           f"{fl / dur[0] / 1e3 / 2500:.3f} of the 2.5 PFLOP/s dense bf16 peak")
        simd_cycles = 1024 * dur[0] * 2.4 if dur else None  # 256 CUs x 4 SIMDs at 2.4 GHz, over the duration
        if "SQ_VALU_MFMA_BUSY_CYCLES" in med and simd_cycles:
            der.append(f"MFMA busy: SQ_VALU_MFMA_BUSY_CYCLES (summed over SIMDs) / (1024 SIMDs x duration x "
                       f"2.4 GHz) = {med['SQ_VALU_MFMA_BUSY_CYCLES'] / simd_cycles:.3f}; busy cycles per MFMA "
                       f"instruction {med['SQ_VALU_MFMA_BUSY_CYCLES'] / max(1, med.get('SQ_INSTS_MFMA', 1)):.1f}")
        if "SQ_INSTS_VALU" in med and "SQ_INSTS_MFMA" in med and med["SQ_INSTS_MFMA"]:
            other = med["SQ_INSTS_VALU"] - med["SQ_INSTS_MFMA"]
            der.append(f"VALU instructions other than MFMA: {other / med['SQ_INSTS_MFMA']:.2f} per MFMA instruction"
                       + (f"; at 4 cycles per wave64 VALU instruction they fill "
                          f"{4 * other / simd_cycles:.3f} of the SIMD cycles" if simd_cycles else ""))
        if "SQ_INSTS_LDS" in med and "SQ_INSTS_MFMA" in med and med["SQ_INSTS_MFMA"]:
            der.append(f"LDS instructions per MFMA instruction: {med['SQ_INSTS_LDS'] / med['SQ_INSTS_MFMA']:.2f}"
                       + (f"; bank conflicts (SQ_LDS_BANK_CONFLICT cycles) per LDS instruction "
                          f"{med['SQ_LDS_BANK_CONFLICT'] / med['SQ_INSTS_LDS']:.2f}"
                          if "SQ_LDS_BANK_CONFLICT" in med and med["SQ_INSTS_LDS"] else ""))
        if der:
            md += ["", "Derived:", ""] + [f"- {d}" for d in der]
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
