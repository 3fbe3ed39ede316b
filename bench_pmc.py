"""Summarise rocprofv3 --pmc CSV output (counter_collection.csv) per kernel.

Usage: python bench_pmc.py <counter_collection.csv> [...]
Prints, per kernel name and counter, the mean value per dispatch, and the derived MFMA
busy fraction, MFMA flops and LDS utilisation when their base counters were collected.
"""
from __future__ import annotations

import collections
import csv
import sys


def load(paths):
    per = collections.defaultdict(lambda: collections.defaultdict(list))
    for path in paths:
        with open(path) as f:
            for row in csv.DictReader(f):
                name = row["Kernel_Name"].replace("gqla::(anonymous namespace)::", "").split("(")[0]
                per[name][row["Counter_Name"]].append(float(row["Counter_Value"]))
    return per


# MI355X: GRBM_GUI_ACTIVE is summed over the 8 XCDs; 256 CUs, 4 SIMDs each
XCDS, CUS, SIMDS = 8, 256, 1024


def derived(ctrs):
    """rocprofv3's MfmaUtil, MfmaFlops and LDS utilisation from the base counters, when present."""
    mean = lambda c: sum(ctrs[c]) / len(ctrs[c])  # noqa: E731
    out = {}
    if "GRBM_GUI_ACTIVE" not in ctrs:
        return out
    cycles = mean("GRBM_GUI_ACTIVE") / XCDS
    out["gpu_cycles"] = cycles
    if "SQ_VALU_MFMA_BUSY_CYCLES" in ctrs and cycles > 0:
        out["mfma_busy"] = mean("SQ_VALU_MFMA_BUSY_CYCLES") / (cycles * SIMDS)
    mops = [c for c in ctrs if c.startswith("SQ_INSTS_VALU_MFMA_MOPS_")]
    if mops:
        out["mfma_flops"] = 512.0 * sum(mean(c) for c in mops)
    if "SQ_LDS_IDX_ACTIVE" in ctrs and cycles > 0:
        out["lds_active"] = mean("SQ_LDS_IDX_ACTIVE") / (cycles * CUS)
        if "SQ_LDS_BANK_CONFLICT" in ctrs and mean("SQ_LDS_IDX_ACTIVE") > 0:
            out["lds_conflict_share"] = mean("SQ_LDS_BANK_CONFLICT") / mean("SQ_LDS_IDX_ACTIVE")
    return out


def main(argv=None) -> int:
    paths = (argv if argv is not None else sys.argv[1:])
    per = load(paths)
    for name, ctrs in per.items():
        print(name)
        for c, vals in sorted(ctrs.items()):
            print(f"    {c:28s} {sum(vals) / len(vals):16.1f}   (n={len(vals)})")
        for k, v in derived(ctrs).items():
            print(f"    = {k:26s} {v:16.4g}")
    return 0


if __name__ == "__main__":
    sys.exit(main())
