"""Turn two rocprofv3 counter runs of `bench.py --counters` (FETCH_SIZE, then
WRITE_SIZE) into per-launch HBM traffic per kernel, calibrated by the 1 GiB
device copy that the counters pass performs first, and write traffic.json.

Usage: python profiles/traffic_from_counters.py <fetch run_counter_collection.csv> <write ...csv>
"""
import csv
import json
import sys
from collections import defaultdict
from pathlib import Path

ROOT = Path(__file__).resolve().parent.parent
sys.path.insert(0, str(ROOT))
from kda_gated_delta_chunk_amd.source_hash import csrc_hash  # noqa: E402

COPY_BYTES = 1 << 30


def per_kernel(path, counter):
    rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
    copy = max(float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"])
    vals = defaultdict(list)
    for r in rows:
        name = r["Kernel_Name"].split("(")[0].replace("void ", "")
        if "kda" in name:
            vals[name].append(float(r["Counter_Value"]))
    return copy, {k: sum(v) / len(v) for k, v in vals.items()}


def main(fetch_csv, write_csv):
    fcopy, f = per_kernel(fetch_csv, "FETCH_SIZE")
    wcopy, w = per_kernel(write_csv, "WRITE_SIZE")
    # the copy reads and writes COPY_BYTES; counters are in KiB
    fscale = COPY_BYTES / (fcopy * 1024.0)
    wscale = COPY_BYTES / (wcopy * 1024.0)
    out = {"csrc_hash": csrc_hash(), "fetch_scale": fscale, "write_scale": wscale, "kernels": {}}
    for k in sorted(set(f) | set(w)):
        fb = f.get(k, 0.0) * 1024.0 * fscale
        wb = w.get(k, 0.0) * 1024.0 * wscale
        out["kernels"][k] = {"fetch_bytes": fb, "write_bytes": wb, "traffic_bytes": fb + wb}
    p = Path(__file__).resolve().parent / "traffic.json"
    p.write_text(json.dumps(out, indent=1) + "\n")
    print(json.dumps(out, indent=1))


if __name__ == "__main__":
    main(sys.argv[1], sys.argv[2])
