"""Turn rocprofv3 counter output into per-launch HBM traffic (profiles/traffic.json).

Usage, after four rocprofv3 counter runs: `bench.py` with `--pmc FETCH_SIZE` and with
`--pmc WRITE_SIZE`, and `bench.py --calibrate-copy` with each of the two:

    python -m dsa_sparse_attention_amd.profiling traffic \
        --fetch <bench FETCH dir>/run_counter_collection.csv \
        --write <bench WRITE dir>/run_counter_collection.csv \
        --cal-fetch <copy FETCH dir>/run_counter_collection.csv \
        --cal-write <copy WRITE dir>/run_counter_collection.csv --out profiles/traffic.json

FETCH_SIZE and WRITE_SIZE are reported in KiB per dispatch, summed over the
TCC (L2) channels. They are converted to bytes with a factor calibrated on the
plain copy that `bench.py --calibrate-copy` launches (the only large kernel of
that run): a device-to-device copy of COPY_BYTES bytes must fetch and write
COPY_BYTES each, so factor = COPY_BYTES / (counter KiB * 1024). The per-launch traffic of each
kernel of the verify step is the mean over its dispatches, times that factor.
Each entry records the sha256 of the kernel's source file, so bench.py reports
the traffic only while the kernel is unchanged.
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
COPY_BYTES = 1 << 30  # size of the calibration copy (bench.py --calibrate-copy)

# kernel-name substring -> (entry key used by bench.py, source file)
KERNELS = {
    "quantize_kernel": ("quantize_q", "quantize.hip"),
    "verify_write_kernel": ("cache_write", "quantize.hip"),
    "index_score_kernel": ("index_score", "index_score.hip"),
    "topk_kernel": ("topk", "topk.hip"),
    "mla_decode_kernel": ("sparse_mla", "sparse_mla.hip"),
    "mla_combine_kernel": ("sparse_mla", "sparse_mla.hip"),
    "argmax_slices_kernel": ("greedy_accept", "greedy_accept.hip"),
    "accept_kernel": ("greedy_accept", "greedy_accept.hip"),
    "ra_stats_kernel": ("rejection_accept", "rejection_accept.hip"),
    "ra_decide_kernel": ("rejection_accept", "rejection_accept.hip"),
    "ra_weights_kernel": ("rejection_accept", "rejection_accept.hip"),
    "ra_draw_kernel": ("rejection_accept", "rejection_accept.hip"),
}
# later kernels of a multi-kernel call (counted in its traffic, not as launches)
SECOND = ("mla_combine_kernel", "accept_kernel", "ra_decide_kernel", "ra_weights_kernel",
          "ra_draw_kernel")


def source_sha(name: str) -> str:
    p = os.path.join(ROOT, "dsa_sparse_attention_amd", "csrc", name)
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def per_dispatch(path: str, counter: str):
    """{dispatch id: (kernel name, summed counter value)} from a counter_collection.csv."""
    out = {}
    with open(path) as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] != counter:
                continue
            d = row["Dispatch_Id"]
            name, v = out.get(d, (row["Kernel_Name"], 0.0))
            out[d] = (name, v + float(row["Counter_Value"]))
    return out


def classify(name: str):
    for key, (entry, src) in KERNELS.items():
        if key in name:
            return entry, src
    return None, None


def traffic(fetch_csv: str, write_csv: str, cal_fetch_csv: str, cal_write_csv: str):
    fetch = per_dispatch(fetch_csv, "FETCH_SIZE")
    write = per_dispatch(write_csv, "WRITE_SIZE")
    # calibration: the largest dispatch of the --calibrate-copy run is the COPY_BYTES copy
    cal_f = [v for _, v in per_dispatch(cal_fetch_csv, "FETCH_SIZE").values()]
    cal_w = [v for _, v in per_dispatch(cal_write_csv, "WRITE_SIZE").values()]
    if not cal_f or not cal_w:
        raise SystemExit("no dispatch in the calibration counter files")
    f_factor = COPY_BYTES / (max(cal_f) * 1024.0)
    w_factor = COPY_BYTES / (max(cal_w) * 1024.0)
    # sum the kernels of one API call (the MLA is decode + combine), averaged per call
    fsum, wsum, nlaunch, srcs = (collections.defaultdict(float), collections.defaultdict(float),
                                 collections.defaultdict(int), {})
    for d, (n, v) in fetch.items():
        e, src = classify(n)
        if e:
            fsum[e] += v * 1024.0 * f_factor
            srcs[e] = src
            if not any(k in n for k in SECOND):
                nlaunch[e] += 1
    for d, (n, v) in write.items():
        e, _ = classify(n)
        if e:
            wsum[e] += v * 1024.0 * w_factor
    out = {"calibration": {"copy_bytes": COPY_BYTES, "fetch_factor": round(f_factor, 4),
                           "write_factor": round(w_factor, 4)}}
    for e in fsum:
        n = max(nlaunch[e], 1)
        fb, wb = fsum[e] / n, wsum[e] / n
        out[e] = {"source_sha": source_sha(srcs[e]), "launches": n,
                  "fetch_bytes_per_launch": round(fb), "write_bytes_per_launch": round(wb),
                  "hbm_bytes_per_launch": round(fb + wb)}
    return out


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--cal-fetch", required=True)
    t.add_argument("--cal-write", required=True)
    t.add_argument("--out", default=os.path.join(ROOT, "profiles", "traffic.json"))
    a = ap.parse_args()
    if a.cmd == "traffic":
        rec = traffic(a.fetch, a.write, a.cal_fetch, a.cal_write)
        with open(a.out, "w") as f:
            json.dump(rec, f, indent=1, sort_keys=True)
            f.write("\n")
        print(json.dumps(rec, indent=1, sort_keys=True))


if __name__ == "__main__":
    main()
