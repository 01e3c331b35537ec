"""HBM bytes per launch from rocprofv3 counter runs, calibrated on a copy.

rocprofv3 ``--pmc FETCH_SIZE`` and ``--pmc WRITE_SIZE`` (separate runs, csv
output) report KiB per dispatch.  The same two counters are read for a plain
device copy of known size (profile_run copy: it reads and writes exactly
``--copy-mib`` MiB), and each counter is scaled by known / measured of that
copy.  For a path of several kernels (decode) the per-dispatch averages of
each kernel are added: the result is bytes per step.

    python3 -m dynamic_block_sparse_dsa_amd.traffic --workload W --src FILE \\
        --kernel-regex RE --fetch DIR --write DIR --copy-fetch DIR --copy-write DIR \\
        --copy-mib 256 --out traffic.json --cmd "..." [--cmd "..."]

Writes (merges) one entry keyed by the workload into ``--out``; the entry
holds the sha256 prefix of ``--src`` so that a reader can tell when the kernel
changed after the counters were taken.
"""

import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import re
import sys


def per_kernel_kib(run_dir, counter, regex):
    """{kernel name: mean over dispatches of the counter summed over its
    instances} for the kernels whose name matches regex."""
    paths = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not paths:
        raise SystemExit(f"no counter_collection.csv under {run_dir}")
    pat = re.compile(regex)
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    for path in paths:
        with open(path) as f:
            for row in csv.DictReader(f):
                name = row.get("Kernel_Name", "")
                if row.get("Counter_Name") != counter or not pat.search(name):
                    continue
                per[name][row["Dispatch_Id"]] += float(row["Counter_Value"])
    if not per:
        raise SystemExit(f"no {counter} samples for /{regex}/ under {run_dir}")
    return {name: sum(d.values()) / len(d) for name, d in per.items()}, {name: len(d) for name, d in per.items()}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--workload", required=True)
    ap.add_argument("--src", required=True)
    ap.add_argument("--kernel-regex", required=True)
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--copy-fetch", required=True)
    ap.add_argument("--copy-write", required=True)
    ap.add_argument("--copy-regex", default="copy")
    ap.add_argument("--copy-mib", type=int, default=256)
    ap.add_argument("--out", required=True)
    ap.add_argument("--cmd", action="append", default=[])
    a = ap.parse_args(argv)

    known_kib = a.copy_mib * 1024.0
    cf, _ = per_kernel_kib(a.copy_fetch, "FETCH_SIZE", a.copy_regex)
    cw, _ = per_kernel_kib(a.copy_write, "WRITE_SIZE", a.copy_regex)
    copy_fetch = max(cf.values())  # the copy itself is the largest matching kernel
    copy_write = max(cw.values())
    f_fetch = known_kib / copy_fetch
    f_write = known_kib / copy_write

    kf, nf = per_kernel_kib(a.fetch, "FETCH_SIZE", a.kernel_regex)
    kw, nw = per_kernel_kib(a.write, "WRITE_SIZE", a.kernel_regex)
    fetch_b = sum(kf.values()) * 1024.0 * f_fetch
    write_b = sum(kw.values()) * 1024.0 * f_write
    entry = dict(
        bytes_per_launch=round(fetch_b + write_b),
        fetch_bytes=round(fetch_b),
        write_bytes=round(write_b),
        kernels={name: dict(fetch_kib=kf.get(name), write_kib=kw.get(name), dispatches=nf.get(name))
                 for name in sorted(set(kf) | set(kw))},
        copy_calibration=dict(mib=a.copy_mib, fetch_kib=copy_fetch, write_kib=copy_write, fetch_factor=f_fetch,
                              write_factor=f_write),
        src=a.src,
        src_sha256_16=hashlib.sha256(open(a.src, "rb").read()).hexdigest()[:16],
        commands=a.cmd,
    )
    data = {}
    if os.path.exists(a.out):
        with open(a.out) as f:
            data = json.load(f)
    data[a.workload] = entry
    with open(a.out, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps({a.workload: entry}, indent=1))
    return 0


if __name__ == "__main__":
    sys.exit(main())
