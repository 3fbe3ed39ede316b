"""HBM traffic per launch of the decode kernels, from rocprofv3 byte counters.

Two counter passes of bench.py (one counter each; a pass holds at most the
counters one hardware pass can collect):

  rocprofv3 --pmc FETCH_SIZE --output-format csv -d out/traffic_FETCH_SIZE -o pmc -- \
      python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline
  rocprofv3 --pmc WRITE_SIZE --output-format csv -d out/traffic_WRITE_SIZE -o pmc -- \
      python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline
  python bench_traffic.py \
      out/traffic_FETCH_SIZE/pmc_counter_collection.csv \
      out/traffic_WRITE_SIZE/pmc_counter_collection.csv BENCH_LINE_JSON [--write]

FETCH_SIZE and WRITE_SIZE are in KiB per dispatch.  bench.py runs one plain device
copy of 1 GiB before timing; its readings give the scale of each counter (bytes
actually moved per counted KiB), which is applied to every kernel.  The algorithmic
bytes per launch come from the bench line the same run printed.  --write stores
the records in profiles/traffic.json with a digest of each kernel's sources, so
that bench.py reports a record only while the sources are unchanged.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.abspath(__file__))
RECORDS = os.path.join(ROOT, "profiles", "traffic.json")
COPY_BYTES = 1 << 30

# sources whose digest a counter record must match, and the kernel-name prefixes the
# record covers
KERNEL_SOURCES = {
    "gqa_decode": ["latent_kv_cache_amd/csrc/decode_gqa.hip", "latent_kv_cache_amd/csrc/common.h"],
    "absorb_decode": ["latent_kv_cache_amd/csrc/decode_absorb.hip", "latent_kv_cache_amd/csrc/common.h"],
    "gqa_sparse": ["latent_kv_cache_amd/csrc/decode_sparse.hip", "latent_kv_cache_amd/csrc/common.h"],
}
KERNEL_PREFIXES = {
    "gqa_decode": ("gqa_decode_kernel", "gqa_dma_kernel"),
    "absorb_decode": ("absorb_decode_kernel",),
    "gqa_sparse": ("gqa_sparse_kernel",),
}


def sources_digest(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel_key: str, workload: str):
    """Counter-derived HBM bytes per launch from profiles/traffic.json, if taken on the
    current sources of the kernel and on this workload (records name their workload;
    older ones are of the flagship)."""
    if not os.path.exists(RECORDS):
        return None
    try:
        rec = json.load(open(RECORDS)).get(kernel_key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_digest") != sources_digest(KERNEL_SOURCES[kernel_key]):
        return None
    if rec.get("workload", "flagship") != workload:
        return None
    return rec.get("bytes_per_launch")


def _short(name: str) -> str:
    # "void gqla::(anonymous namespace)::gqa_decode_kernel<8, 8, 1>(...)" -> "gqa_decode_kernel<8, 8, 1>"
    name = name.replace("(anonymous namespace)::", "")
    name = name[5:] if name.startswith("void ") else name
    name = name[6:] if name.startswith("gqla::") else name
    return name.split("(")[0]


def per_dispatch(path: str, counter: str):
    """{kernel name: [value per dispatch]} of one counter (KiB)."""
    vals = defaultdict(lambda: defaultdict(float))
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] != counter:
                continue
            vals[_short(row["Kernel_Name"])][row["Dispatch_Id"]] += float(row["Counter_Value"])
    return {k: list(v.values()) for k, v in vals.items()}


def summarize(fetch_csv: str, write_csv: str, bench_line: dict):
    fetch = per_dispatch(fetch_csv, "FETCH_SIZE")
    write = per_dispatch(write_csv, "WRITE_SIZE")
    copy_kib = COPY_BYTES / 1024
    # the calibration copy: the copy dispatch that wrote the most
    cw = max(v for k, vs in write.items() if "copyBuffer" in k for v in vs)
    cf = max(v for k, vs in fetch.items() if "copyBuffer" in k for v in vs)
    read_scale, write_scale = copy_kib / cf, copy_kib / cw
    alg = {
        "gqa_decode": bench_line["paths"]["gqa"]["alg_bytes"],
        "absorb_decode": bench_line["paths"]["absorb"]["alg_bytes"],
    }
    nxt = bench_line.get("next") or {}
    if nxt.get("sparse_gqa"):
        alg["gqa_sparse"] = nxt["sparse_gqa"]["alg_bytes_per_launch"]
    workload = bench_line["config"]["workload"]
    out = {}
    for key, prefixes in KERNEL_PREFIXES.items():
        fk = [v for k, vs in fetch.items() if k.startswith(prefixes) for v in vs]
        wk = [v for k, vs in write.items() if k.startswith(prefixes) for v in vs]
        if not fk or not wk or key not in alg:
            continue
        rd = sum(fk) / len(fk) * read_scale * 1024
        wr = sum(wk) / len(wk) * write_scale * 1024
        out[key] = {"source_digest": sources_digest(KERNEL_SOURCES[key]), "workload": workload,
                    "kernels": sorted(k for k in fetch if k.startswith(prefixes)),
                    "bytes_per_launch": int(rd + wr), "read_bytes": int(rd), "write_bytes": int(wr),
                    "algorithmic_bytes": int(alg[key]),
                    "traffic_over_algorithmic": round((rd + wr) / alg[key], 4),
                    "fetch_kib_per_dispatch": round(sum(fk) / len(fk)), "write_kib_per_dispatch": round(sum(wk) / len(wk))}
    note = (f"HBM bytes per launch from rocprofv3 FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of "
            f"`python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline`, scaled by the counters' reading of "
            f"bench.py's 1 GiB device copy (reads x{read_scale:.3f}, writes x{write_scale:.3f}); written by "
            f"`python bench_traffic.py`. source_digest: sha256 (16 hex) of each kernel's sources "
            f"when the counters were taken.")
    return note, out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("fetch_csv")
    ap.add_argument("write_csv")
    ap.add_argument("bench_line", help="file holding the JSON line the profiled bench run printed")
    ap.add_argument("--write", action="store_true", help="store the records in profiles/traffic.json")
    args = ap.parse_args(argv)
    line = None
    for text in open(args.bench_line):
        text = text.strip()
        if text.startswith("{") and '"metric"' in text:
            line = json.loads(text)
    if line is None:
        print("no bench JSON line found", file=sys.stderr)
        return 1
    note, recs = summarize(args.fetch_csv, args.write_csv, line)
    print(note)
    print()
    print("| record | kernels | FETCH_SIZE KiB | WRITE_SIZE KiB | read GB | write GB | algorithmic GB | traffic / algorithmic |")
    print("|---|---|---|---|---|---|---|---|")
    for key, r in recs.items():
        print(f"| {key} | {', '.join(r['kernels'])} | {r['fetch_kib_per_dispatch']} | {r['write_kib_per_dispatch']} | "
              f"{r['read_bytes'] / 1e9:.4f} | {r['write_bytes'] / 1e9:.4f} | {r['algorithmic_bytes'] / 1e9:.4f} | "
              f"{r['traffic_over_algorithmic']:.3f} |")
    if args.write:
        data = {"_note": note}
        data.update(recs)
        with open(RECORDS, "w") as f:
            json.dump(data, f, indent=1)
            f.write("\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())
