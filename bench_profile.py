"""Summarise a rocprofv3 kernel-trace database (rocpd SQLite) as a markdown table.

Usage: python bench_profile.py <results.db> [--command "..."]
Per kernel name: dispatch count, median / average / min / max duration (us), total (us),
grid and workgroup sizes, VGPR/AGPR counts and LDS bytes per workgroup.
"""
from __future__ import annotations

import argparse
import sqlite3
import sys


def summarise(db_path: str):
    db = sqlite3.connect(db_path)
    rows = db.execute(
        """select name, count(*), avg(end - start) / 1000.0, min(end - start) / 1000.0,
                  max(end - start) / 1000.0, sum(end - start) / 1000.0,
                  max(grid_x), max(grid_y), max(grid_z), max(workgroup_x),
                  max(vgpr_count), max(accum_vgpr_count), max(lds_size)
           from kernels group by name order by sum(end - start) desc""").fetchall()
    durs = {}
    for name, d in db.execute("select name, end - start from kernels"):
        durs.setdefault(name, []).append(d / 1000.0)
    med = {n: sorted(v)[len(v) // 2] for n, v in durs.items()}
    return [(r[0], r[1], med[r[0]]) + tuple(r[2:]) for r in rows]


def short(name: str) -> str:
    name = name.replace("gqla::(anonymous namespace)::", "")
    return name.split("(")[0] if "(" in name else name


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("db")
    ap.add_argument("--command", default="")
    a = ap.parse_args(argv)
    rows = summarise(a.db)
    if a.command:
        print(f"Command: `{a.command}`\n")
    print("| kernel | n | median us | avg us | min us | max us | total us | grid | wg | vgpr | agpr | lds B |")
    print("|---|---|---|---|---|---|---|---|---|---|---|---|")
    for r in rows:
        print(f"| {short(r[0])} | {r[1]} | {r[2]:.2f} | {r[3]:.2f} | {r[4]:.2f} | {r[5]:.2f} | {r[6]:.1f} | "
              f"{r[7]}x{r[8]}x{r[9]} | {r[10]} | {r[11]} | {r[12]} | {r[13]} |")
    return 0


if __name__ == "__main__":
    sys.exit(main())
