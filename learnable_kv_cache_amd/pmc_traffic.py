"""HBM traffic per launch from rocprofv3 counter runs (writes profiles/traffic.json).

Inputs are the counter_collection CSVs of four ``rocprofv3 --pmc ... --output-format
csv`` runs: FETCH_SIZE and WRITE_SIZE (KiB per dispatch) over a bench run, and the
same two counters over ``bench.py --copy-calibration MIB``, whose copies move a known
number of bytes.  Each counter is scaled by known bytes / counted bytes of the copy,
then summed per kernel; the record keeps the sha256 (first 16 hex digits) of the
kernel's source so that bench.py reports it only while the kernel is unchanged.

Usage:
  python -m learnable_kv_cache_amd.pmc_traffic --fetch F.csv --write W.csv \\
      --copy-fetch CF.csv --copy-write CW.csv --copy-bytes N \\
      --kernel attend_prefill=attend_prefill_kernel:csrc/attend.hip \\
      --kernel decode_step=decode_step_kernel:csrc/decode.hip --out profiles/traffic.json
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))


def per_dispatch(path: str, counter: str) -> dict[str, list[float]]:
    """kernel name -> counter value of each dispatch (summed over the CSV's rows)."""
    acc: dict[tuple[str, str], float] = defaultdict(float)
    with open(path) as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] != counter:
                continue
            acc[(row["Kernel_Name"], row["Dispatch_Id"])] += float(row["Counter_Value"])
    out: dict[str, list[float]] = defaultdict(list)
    for (name, _), val in acc.items():
        out[name].append(val)
    return out


def copy_scale(path: str, counter: str, copy_bytes: int) -> float:
    """known bytes / counted bytes for the calibration copies (the largest dispatches)."""
    vals = [v for name, vs in per_dispatch(path, counter).items() for v in vs]
    if not vals:
        raise SystemExit(f"no {counter} rows in {path}")
    counted = sorted(vals)[-1] * 1024.0          # KiB -> bytes
    return copy_bytes / counted


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--copy-fetch", required=True)
    ap.add_argument("--copy-write", required=True)
    ap.add_argument("--copy-bytes", type=int, required=True)
    ap.add_argument("--kernel", action="append", required=True,
                    help="record=kernel-name-substring:source-path-relative-to-the-package")
    ap.add_argument("--command", default="", help="the profiled command, for the record")
    ap.add_argument("--out", required=True)
    a = ap.parse_args()
    sf = copy_scale(a.copy_fetch, "FETCH_SIZE", a.copy_bytes)
    sw = copy_scale(a.copy_write, "WRITE_SIZE", a.copy_bytes)
    fetch = per_dispatch(a.fetch, "FETCH_SIZE")
    write = per_dispatch(a.write, "WRITE_SIZE")
    try:
        with open(a.out) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        rec = {}
    for spec in a.kernel:
        key, rest = spec.split("=", 1)
        sub, src = rest.split(":", 1)
        fv = [v for n, vs in fetch.items() if sub in n for v in vs]
        wv = [v for n, vs in write.items() if sub in n for v in vs]
        if not fv or not wv:
            raise SystemExit(f"no dispatches of {sub}")
        fb = sum(fv) / len(fv) * 1024.0 * sf
        wb = sum(wv) / len(wv) * 1024.0 * sw
        with open(os.path.join(PKG, src), "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()[:16]
        rec[key] = {"kernel": sub, "source_sha": sha, "fetch_bytes": fb, "write_bytes": wb,
                    "bytes_per_launch": fb + wb, "dispatches": [len(fv), len(wv)],
                    "scale_fetch": sf, "scale_write": sw, "command": a.command}
        print(f"{key}: fetch {fb / 1e6:.1f} MB, write {wb / 1e6:.1f} MB per launch "
              f"(scales {sf:.3f}, {sw:.3f})")
    with open(a.out, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)


if __name__ == "__main__":
    main()
