"""Counter-traffic summary (host logic): calibration by the 1 GiB copy and per-launch
averages, on synthetic rocprofv3 CSV rows."""
import csv
import json

import bench_traffic as traffic

HEAD = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(HEAD)
        for d, (name, v) in enumerate(rows):
            w.writerow([d, name, counter, v])


def test_summary_scales_by_the_copy(tmp_path):
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    # the counters read half of the copy's bytes on fetch and all of them on write
    _csv(fetch, "FETCH_SIZE", [("__amd_rocclr_copyBuffer", 524288.0), ("void gqla::(anonymous namespace)::gqa_decode_kernel<8, 8, 1>(int)", 1000.0),
                               ("void gqla::(anonymous namespace)::gqa_decode_kernel<8, 8, 1>(int)", 3000.0),
                               ("void absorb_decode_kernel<8, 1, 1>(int)", 500.0)])
    _csv(write, "WRITE_SIZE", [("__amd_rocclr_copyBuffer", 1048576.0), ("void gqla::(anonymous namespace)::gqa_decode_kernel<8, 8, 1>(int)", 10.0),
                               ("void gqla::(anonymous namespace)::gqa_decode_kernel<8, 8, 1>(int)", 30.0),
                               ("void absorb_decode_kernel<8, 1, 1>(int)", 20.0)])
    line = {"config": {"workload": "w"}, "paths": {"gqa": {"alg_bytes": 4096 * 1024}, "absorb": {"alg_bytes": 1024 * 1024}},
            "next": None}
    note, recs = traffic.summarize(str(fetch), str(write), line)
    g = recs["gqa_decode"]
    assert g["read_bytes"] == 2000 * 2 * 1024 and g["write_bytes"] == 20 * 1024
    assert g["bytes_per_launch"] == g["read_bytes"] + g["write_bytes"]
    assert abs(g["traffic_over_algorithmic"] - (4000 + 20) / 4096) < 1e-4
    a = recs["absorb_decode"]
    assert a["read_bytes"] == 500 * 2 * 1024 and a["workload"] == "w"
    assert "gqa_sparse" not in recs and "x2.000" in note
    assert json.loads(json.dumps(recs)) == recs
