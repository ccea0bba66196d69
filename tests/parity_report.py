"""Markdown tables of the parity margins one GPU test run recorded.

``compare`` (tests/parity.py) appends one JSON line per comparison to the
file ``PA_PARITY_RECORD`` names.  This script turns that record into the
committed margin tables:

    PA_PARITY_RECORD=<run>.jsonl python -u -m pytest tests -m gpu -q -s
    python -m tests.parity_report <run>.jsonl > profiles/parity_margins.md
"""

from __future__ import annotations

import json
import re
import sys

from workloads import WORKLOADS

SPLITS = {"-1": "balanced + merge", "-2": "balanced, merged in the launch", "0": "unsplit"}

HEADER = """# Parity margins: HIP library against the oracle (MI355X)

Every comparison of the GPU test suite appends its margins to a JSON-lines
file when `PA_PARITY_RECORD` names one (`tests/parity.py`, `compare`). These
tables are that record for one full run of the suite on one MI355X, made by
`tests/parity_report.py`:

    PA_PARITY_RECORD=<run>.jsonl python -u -m pytest tests -m gpu -q -s
    python -m tests.parity_report <run>.jsonl > profiles/parity_margins.md

Columns: output rows compared (sequence x query head); `max_abs` = max
|gpu - oracle|; `max_rel` = max |gpu - oracle| / |oracle| over elements
with |oracle| >= 1e-2; `norm` = the largest, over rows, of a row's max error
over that row's max |oracle| (bar 1e-2; 1e-4 for f32); `atol needed` = the
smallest atol that, with the test's rtol, would still have passed
(max(|gpu - oracle| - rtol |oracle|)). The oracle is float64, the GPU
output bf16 (f32 for the f32 workload): bf16 rounding of the output alone
is up to 2^-9 of a value.
"""


def fmt(x: float) -> str:
    return f"{x:.2e}"


def split_name(p: str) -> str:
    return SPLITS.get(p, f"{p}-token partitions")


def report(records: list[dict]) -> str:
    out = [HEADER]
    out.append("## The five workloads at full size, every sequence\n")
    out.append("Outputs of all sequences of each batch against the oracle's decode over the\n"
               "oracle's own append (`tests/test_gpu_parity.py::test_workload_write_and_decode`,\n"
               "`tests/test_gpu_decode_append.py::test_full_size_step_as_the_bench_runs_it`).\n")
    out.append("| workload | split | rows | max_abs | max_rel | norm | atol needed | atol / rtol |")
    out.append("|---|---|---|---|---|---|---|---|")
    rows = []
    for r in records:
        m = re.fullmatch(r"full-size step (\S+)", r["label"])
        if m:
            rows.append((m.group(1), "the bench's step (append in the decode launch, balanced, merge)", r))
        m = re.fullmatch(r"workload (\d) P=(-?\d+)", r["label"])
        if m:
            rows.append((WORKLOADS[int(m.group(1))].name, split_name(m.group(2)), r))
    for name, split, r in rows:
        out.append(f"| {name} | {split} | {r['rows']} | {fmt(r['max_abs'])} | {fmt(r['max_rel'])} | "
                   f"{fmt(r['norm'])} | {fmt(r['atol_needed'])} | {r['atol']:g} / {r['rtol']:g} |")
    out.append("\n## Every comparison of the suite, by cache kind\n")
    out.append("| cache | comparisons | rows | max_abs | max norm | max atol needed | atol |")
    out.append("|---|---|---|---|---|---|---|")
    kinds: dict[str, list[dict]] = {}
    for r in records:
        kinds.setdefault(r["cache"], []).append(r)
    for cache in ("f32", "bf16", "fp8_e4m3", "fp8_e5m2", "int4"):
        rs = kinds.get(cache)
        if not rs:
            continue
        out.append(f"| {cache} | {len(rs)} | {sum(r['rows'] for r in rs)} | "
                   f"{fmt(max(r['max_abs'] for r in rs))} | {fmt(max(r['norm'] for r in rs))} | "
                   f"{fmt(max(r['atol_needed'] for r in rs))} | {rs[0]['atol']:g} |")
    out.append("\n## The comparisons with the least headroom\n")
    out.append("Largest `atol needed` relative to the comparison's atol (the ten closest to\n"
               "their bar).\n")
    out.append("| comparison | cache | rows | max_abs | norm | atol needed / atol |")
    out.append("|---|---|---|---|---|---|")
    for r in sorted(records, key=lambda r: -r["atol_needed"] / r["atol"])[:10]:
        out.append(f"| {r['label']} | {r['cache']} | {r['rows']} | {fmt(r['max_abs'])} | "
                   f"{fmt(r['norm'])} | {r['atol_needed'] / r['atol']:.2f} |")
    return "\n".join(out) + "\n"


def main(argv: list[str]) -> int:
    if len(argv) != 2:
        print(__doc__, file=sys.stderr)
        return 2
    with open(argv[1]) as f:
        records = [json.loads(line) for line in f if line.strip()]
    sys.stdout.write(report(records))
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv))
