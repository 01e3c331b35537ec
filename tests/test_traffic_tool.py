"""The counter reducer behind profiles/traffic.json (host logic only)."""

import csv
import json

from dynamic_block_sparse_dsa_amd import traffic

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _csv(path, rows):
    path.mkdir(parents=True, exist_ok=True)
    with open(path / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(FIELDS)
        w.writerows(rows)


def test_copy_calibration_and_per_step_sum(tmp_path):
    # copy of 256 MiB: FETCH_SIZE reads half (two instances per dispatch), WRITE_SIZE exact
    _csv(tmp_path / "cf", [(1, "copy_kernel", "FETCH_SIZE", 65536), (1, "copy_kernel", "FETCH_SIZE", 65536),
                           (2, "fill", "FETCH_SIZE", 7)])
    _csv(tmp_path / "cw", [(1, "copy_kernel", "WRITE_SIZE", 262144)])
    # two kernels of one step; kernel a dispatched twice
    _csv(tmp_path / "kf", [(5, "dsa::decode_a", "FETCH_SIZE", 1000), (8, "dsa::decode_a", "FETCH_SIZE", 1200),
                           (6, "dsa::decode_b", "FETCH_SIZE", 50), (7, "other", "FETCH_SIZE", 1e9)])
    _csv(tmp_path / "kw", [(5, "dsa::decode_a", "WRITE_SIZE", 10), (6, "dsa::decode_b", "WRITE_SIZE", 2)])
    src = tmp_path / "k.hip"
    src.write_text("kernel")
    out = tmp_path / "traffic.json"
    args = ["--workload", "w", "--src", str(src), "--kernel-regex", "dsa::decode_", "--fetch", str(tmp_path / "kf"),
            "--write", str(tmp_path / "kw"), "--copy-fetch", str(tmp_path / "cf"), "--copy-write", str(tmp_path / "cw"),
            "--copy-mib", "256", "--out", str(out), "--cmd", "c"]
    assert traffic.main(args) == 0
    e = json.load(open(out))["w"]
    assert e["copy_calibration"]["fetch_factor"] == 2.0
    assert e["copy_calibration"]["write_factor"] == 1.0
    assert e["fetch_bytes"] == round((1100 + 50) * 1024 * 2.0)
    assert e["write_bytes"] == (10 + 2) * 1024
    assert e["bytes_per_launch"] == e["fetch_bytes"] + e["write_bytes"]
    # a second workload merges into the same file
    args[1] = "w2"
    traffic.main(args)
    assert set(json.load(open(out))) == {"w", "w2"}
