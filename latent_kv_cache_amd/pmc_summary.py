"""Summarise rocprofv3 --pmc CSV output (counter_collection.csv) per kernel.

Usage: python -m latent_kv_cache_amd.pmc_summary <counter_collection.csv> [...]
Prints, per kernel name and counter, the mean value per dispatch.
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


def main(argv=None) -> int:
    paths = (argv if argv is not None else sys.argv[1:])
    per = load(paths)
    for name, ctrs in per.items():
        print(name)
        for c, vals in sorted(ctrs.items()):
            print(f"    {c:28s} {sum(vals) / len(vals):16.1f}   (n={len(vals)})")
    return 0


if __name__ == "__main__":
    sys.exit(main())
