"""HBM traffic per decode step from rocprofv3 counter runs.

Two counter runs of `bench.py ... --calibrate-copy-mib 256` (one with
`--pmc FETCH_SIZE`, one with `--pmc WRITE_SIZE`, csv output) hold, per
dispatch, the counter in KiB.  The calibration copy (torch.mul on 256 MiB of
fp32, three times) reads and writes a known number of bytes; the ratio of
that size to what the counter reads for it scales the decode kernel's
readings.  The `steps` timed steps are the last `dispatches` decode
dispatches (one launch of all of them by default; `--dispatches` = steps
for one step per launch).

    python -m quantized_gemv_amd.traffic --workload qwen3_0p6b_bf16 --steps 256 --dispatches 1 \\
        --fetch <fetch run dir>/run_counter_collection.csv \\
        --write <write run dir>/run_counter_collection.csv \\
        --out profiles/decode_kernel_traffic.json
"""
from __future__ import annotations

import argparse
import csv
import json
import os
import sys

COPY_KIB = 256 * 1024


def _values(path: str, kernel_part: str):
    out = []
    with open(path) as f:
        for r in csv.DictReader(f):
            if kernel_part in r["Kernel_Name"]:
                out.append((int(r["Dispatch_Id"]), float(r["Counter_Value"]), r["Kernel_Name"]))
    out.sort()
    return [v for _, v, _ in out], (out[0][2] if out else "")


def summarise(fetch_csv: str, write_csv: str, steps: int, dispatches: int) -> dict:
    fetch, name = _values(fetch_csv, "decode_kernel")
    write, _ = _values(write_csv, "decode_kernel")
    cf, _ = _values(fetch_csv, "MulFunctor")
    cw, _ = _values(write_csv, "MulFunctor")
    if len(fetch) < dispatches or len(write) < dispatches or not cf or not cw:
        raise SystemExit("counter files lack the decode launches or the calibration copy")
    sf, sw = COPY_KIB / (sum(cf) / len(cf)), COPY_KIB / (sum(cw) / len(cw))
    fk = sum(fetch[-dispatches:]) / steps   # KiB per step
    wk = sum(write[-dispatches:]) / steps
    return {"kernel": name.split("(")[0].replace("void ", ""),
            "calibration": {"fetch_kib_read": round(sum(cf) / len(cf), 3), "write_kib_read": round(sum(cw) / len(cw), 3),
                            "fetch_scale": round(sf, 5), "write_scale": round(sw, 5)},
            "steps": steps, "dispatches": dispatches,
            "fetch_kib_per_step": round(fk, 3), "write_kib_per_step": round(wk, 3),
            "fetch_bytes_per_step": int(round(fk * 1024 * sf)), "write_bytes_per_step": int(round(wk * 1024 * sw))}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", required=True)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--dispatches", type=int, default=1, help="decode dispatches the timed steps ran in")
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--algorithmic-bytes", type=int, default=0, help="per step, mean over the timed positions")
    ap.add_argument("--out", required=True)
    args = ap.parse_args()
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    sys.path.insert(0, root)
    import bench
    e = summarise(args.fetch, args.write, args.steps, args.dispatches)
    e["window"] = (f"the {args.steps} timed steps (the last {args.dispatches} decode dispatches) of bench.py "
                   f"--workload {args.workload} --steps {args.steps} --warmup 16 --repeats 1")
    if args.algorithmic_bytes:
        e["algorithmic_bytes_per_step"] = args.algorithmic_bytes
    try:
        with open(args.out) as f:
            d = json.load(f)
    except (OSError, ValueError):
        d = {}
    h = bench.kernel_source_hash()
    if d.get("kernel_source_sha256") != h:
        d = {"kernel_source_sha256": h, "workloads": {}}
    d["workloads"][args.workload] = e
    with open(args.out, "w") as f:
        json.dump(d, f, indent=1)
    print(json.dumps(e))


if __name__ == "__main__":
    main()
