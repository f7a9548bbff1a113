"""Turn rocprofv3 counter output into per-launch HBM traffic (profiles/traffic.json), per-dispatch
byte tables and MFMA-utilisation tables.

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
the traffic only while the kernel is unchanged. Several --fetch/--write pairs may be given
(say the separate and the fused top-k path, each its own bench run).

`dispatches` prints the same bytes per dispatch grouped by kernel and grid size (calls of one
kernel over different row counts, such as verify and draft rows, stay apart). `mfma` reads one
run with the MFMA counters (MFMA_COUNTERS, one rocprofv3 pass: 7 SQ counters and one GRBM
counter) and prints, per kernel, the MFMA utilisation (rocprofv3's MfmaUtil and the same busy
cycles over the kernel's own span), the co-issue fraction and the VALU:MFMA instruction ratio.
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

# kernel-name substring -> (entry key used by bench.py, source file). Every kernel of a call
# adds to its traffic; the call's launches are counted on the kernel that runs exactly once
# per call (PRIMARY).
KERNELS = {
    "quantize_kernel": ("quantize_q", "quantize.hip"),
    "verify_write_kernel": ("cache_write", "quantize.hip"),
    "index_score_kernel": ("index_score", "index_score.hip"),
    "topk_scale_max_kernel": ("topk", "topk.hip"),
    "topk_chunk_kernel": ("topk", "topk.hip"),
    "topk_merge_kernel": ("topk", "topk.hip"),
    "topk_band_classify_kernel": ("topk", "topk.hip"),
    "topk_band_rescore_kernel": ("topk", "topk.hip"),
    "topk_band_finish_kernel": ("topk", "topk.hip"),
    "topk_kernel": ("topk", "topk.hip"),
    "sample_tau_kernel": ("index_topk", "index_score.hip"),
    "fused_select_kernel": ("index_topk", "index_score.hip"),
    "mla_fp8_pack_kernel": ("cache_write", "quantize.hip"),
    "mla_decode_kernel": ("sparse_mla", "sparse_mla.hip"),
    "mla_combine_kernel": ("sparse_mla", "sparse_mla.hip"),
    "argmax_slices_kernel": ("greedy_accept", "greedy_accept.hip"),
    "accept_kernel": ("greedy_accept", "greedy_accept.hip"),
    "ra_stats_kernel": ("rejection_accept", "rejection_accept.hip"),
    "ra_decide_kernel": ("rejection_accept", "rejection_accept.hip"),
    "ra_weights_kernel": ("rejection_accept", "rejection_accept.hip"),
    "ra_draw_kernel": ("rejection_accept", "rejection_accept.hip"),
}
PRIMARY = ("quantize_kernel", "verify_write_kernel", "topk_kernel", "topk_merge_kernel",
           "fused_select_kernel", "mla_decode_kernel", "argmax_slices_kernel", "ra_stats_kernel")
# the fused call's sources: its selection kernels live in topk.hip, its scorer in index_score.hip
SOURCES = {"index_topk": ("index_score.hip", "topk.hip")}
SIMDS = 256 * 4  # MI355X: 256 compute units of 4 SIMDs each
XCDS = 8         # accelerator complex dies, each with its own GRBM instance
SES = 32         # shader engines (4 per XCD)


def short_name(name: str) -> str:
    """`dsa::(anonymous namespace)::index_score_kernel<128, 4, 6, 0>(...)` -> the template id."""
    i = name.find("namespace)::")
    n = name[i + 12:] if i >= 0 else name
    depth, out = 0, []
    for ch in n:  # cut at the argument list, keeping template arguments
        if ch == "(" and depth == 0:
            break
        depth += ch == "<"
        depth -= ch == ">"
        out.append(ch)
    return "".join(out).strip()


def index_score_mode(name: str) -> int:
    """The MODE template argument of index_score_kernel<D, HT, NRV, MODE> (0: plain scores;
    1, 2: the sampling and compaction passes of the fused index + top-k call)."""
    sn = short_name(name)
    try:
        return int(sn[sn.index("<") + 1:sn.rindex(">")].split(",")[3])
    except (ValueError, IndexError):
        return 0


def source_sha(name: str) -> str:
    """Hash of the source file(s) of a call: one file name, or several joined by '+'."""
    h = hashlib.sha256()
    for n in name.split("+"):
        h.update(open(os.path.join(ROOT, "dsa_sparse_attention_amd", "csrc", n), "rb").read())
    return h.hexdigest()[:16]


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


def dispatch_table(path: str):
    """{dispatch id: {"name", "grid", "ns", counter: summed value, ...}} of every counter."""
    out = {}
    with open(path) as f:
        for row in csv.DictReader(f):
            d = out.setdefault(row["Dispatch_Id"], {
                "name": row["Kernel_Name"], "grid": int(row["Grid_Size"]),
                "ns": int(row["End_Timestamp"]) - int(row["Start_Timestamp"])})
            c = row["Counter_Name"]
            d[c] = d.get(c, 0.0) + float(row["Counter_Value"])
    return out


def classify(name: str, fp8_mla: bool = False):
    """(call entry, source) of a kernel; index_score_kernel's fused modes belong to index_topk,
    and the FP8 decode (mla_decode_kernel<true>, with the combine of its run: fp8_mla) to
    sparse_mla_fp8."""
    if "index_score_kernel" in name and index_score_mode(name) != 0:
        return "index_topk", "+".join(SOURCES["index_topk"])
    if "mla_decode_kernel<true>" in name or (fp8_mla and "mla_combine_kernel" in name):
        return "sparse_mla_fp8", "sparse_mla.hip"
    for key, (entry, src) in KERNELS.items():
        if key in name:
            if entry in SOURCES:
                src = "+".join(SOURCES[entry])
            return entry, src
    return None, None


def primary(name: str) -> bool:
    """True for the kernel that runs once per call (the scorer's plain mode, or PRIMARY)."""
    if "index_score_kernel" in name:
        return index_score_mode(name) == 0
    return any(k in name for k in PRIMARY)


def calibration(cal_fetch_csv: str, cal_write_csv: str):
    """(fetch factor, write factor): bytes per counted KiB, from the --calibrate-copy runs whose
    largest dispatch is the COPY_BYTES copy."""
    cal_f = [v for _, v in per_dispatch(cal_fetch_csv, "FETCH_SIZE").values()]
    cal_w = [v for _, v in per_dispatch(cal_write_csv, "WRITE_SIZE").values()]
    if not cal_f or not cal_w:
        raise SystemExit("no dispatch in the calibration counter files")
    return COPY_BYTES / (max(cal_f) * 1024.0), COPY_BYTES / (max(cal_w) * 1024.0)


def traffic(fetch_csvs, write_csvs, cal_fetch_csv: str, cal_write_csv: str):
    """Per-call HBM bytes per launch over one or more (FETCH run, WRITE run) pairs; a call seen
    in several runs takes the figures of the last run that has it."""
    f_factor, w_factor = calibration(cal_fetch_csv, cal_write_csv)
    out = {"calibration": {"copy_bytes": COPY_BYTES, "fetch_factor": round(f_factor, 4),
                           "write_factor": round(w_factor, 4)}}
    for fetch_csv, write_csv in zip(fetch_csvs, write_csvs):
        fetch = per_dispatch(fetch_csv, "FETCH_SIZE")
        write = per_dispatch(write_csv, "WRITE_SIZE")
        fp8 = any("mla_decode_kernel<true>" in n for n, _ in fetch.values())
        # sum the kernels of one API call (the MLA is decode + combine), averaged per call
        fsum, wsum, nlaunch, srcs = (collections.defaultdict(float), collections.defaultdict(float),
                                     collections.defaultdict(int), {})
        for d, (n, v) in fetch.items():
            e, src = classify(n, fp8)
            if e:
                fsum[e] += v * 1024.0 * f_factor
                srcs[e] = src
                nlaunch[e] += primary(n)
        for d, (n, v) in write.items():
            e, _ = classify(n, fp8)
            if e:
                wsum[e] += v * 1024.0 * w_factor
        for e in fsum:
            n = max(nlaunch[e], 1)
            fb, wb = fsum[e] / n, wsum[e] / n
            out[e] = {"source_sha": source_sha(srcs[e]), "launches": n,
                      "fetch_bytes_per_launch": round(fb), "write_bytes_per_launch": round(wb),
                      "hbm_bytes_per_launch": round(fb + wb)}
    return out


def dispatches(fetch_csv: str, write_csv: str, cal_fetch_csv: str, cal_write_csv: str):
    """Markdown table of HBM bytes per dispatch, grouped by kernel and grid size (so that calls
    of one kernel over different row counts stay apart)."""
    f_factor, w_factor = calibration(cal_fetch_csv, cal_write_csv)
    fetch = per_dispatch(fetch_csv, "FETCH_SIZE")
    write = per_dispatch(write_csv, "WRITE_SIZE")
    grids = {d: r["grid"] for d, r in dispatch_table(fetch_csv).items()}
    groups = collections.defaultdict(lambda: [0, 0.0, 0.0])
    for d, (n, v) in fetch.items():
        if classify(n)[0] is None:
            continue
        g = groups[(short_name(n), grids[d])]
        g[0] += 1
        g[1] += v * 1024.0 * f_factor
    wgrids = {d: r["grid"] for d, r in dispatch_table(write_csv).items()}
    for d, (n, v) in write.items():
        key = (short_name(n), wgrids[d])
        if key in groups:
            groups[key][2] += v * 1024.0 * w_factor
    lines = ["| kernel | grid (threads) | dispatches | fetch MB | write MB |", "|---|---|---|---|---|"]
    for (n, grid), (c, fb, wb) in sorted(groups.items(), key=lambda kv: -kv[1][1] / kv[1][0]):
        lines.append(f"| {n} | {grid} | {c} | {fb / c / 1e6:.1f} | {wb / c / 1e6:.1f} |")
    return "\n".join(lines)


MFMA_COUNTERS = ("SQ_INSTS_MFMA", "SQ_INSTS_VALU", "SQ_VALU_MFMA_BUSY_CYCLES",
                 "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE",
                 "SQ_INSTS_VALU_MFMA_MOPS_F8", "SQ_INSTS_VALU_MFMA_MOPS_BF16")


def mfma_summary(csv_path: str):
    """Per kernel (and grid): mean of each MFMA counter per dispatch and three utilisations.

    * rocprofv3's MfmaUtil, sum(SQ_VALU_MFMA_BUSY_CYCLES) / (max GRBM_GUI_ACTIVE * SIMDs). The
      csv holds GRBM_GUI_ACTIVE summed over the XCDs, so its max is taken as the sum / XCDS.
    * the same busy cycles over SIMDs * the kernel's own span in cycles, SQ_BUSY_CYCLES / SES
      (SQ_BUSY_CYCLES is summed over the shader engines while they run the kernel). GRBM's
      window also holds the profiler's set-up around the dispatch; SQ_BUSY_CYCLES does not.
    * the MFMA work as FLOPs, 512 per count of the MOPS counters.
    The clock of the dispatch is SQ_BUSY_CYCLES / SES over its duration.
    """
    table = dispatch_table(csv_path)
    groups = collections.defaultdict(list)
    for r in table.values():
        if classify(r["name"])[0] is not None:
            groups[(short_name(r["name"]), r["grid"])].append(r)
    rows = []
    for (n, grid), rs in groups.items():
        mean = {c: sum(r.get(c, 0.0) for r in rs) / len(rs) for c in MFMA_COUNTERS + ("ns",)}
        busy = mean["SQ_VALU_MFMA_BUSY_CYCLES"]
        span = mean["SQ_BUSY_CYCLES"] / SES
        gui = mean["GRBM_GUI_ACTIVE"] / XCDS
        rows.append({
            "kernel": n, "grid": grid, "dispatches": len(rs), "mean_us": mean["ns"] / 1e3,
            "clock_ghz": span / mean["ns"] if mean["ns"] else 0.0,
            "mfma_util_rocprof": busy / (gui * SIMDS) if gui else 0.0,
            "mfma_util_span": busy / (span * SIMDS) if span else 0.0,
            "coexec_frac": mean["SQ_VALU_MFMA_COEXEC_CYCLES"] / busy if busy else 0.0,
            "valu_per_mfma": (mean["SQ_INSTS_VALU"] / mean["SQ_INSTS_MFMA"]
                              if mean["SQ_INSTS_MFMA"] else 0.0),
            "f8_flops": 512.0 * mean["SQ_INSTS_VALU_MFMA_MOPS_F8"],
            "bf16_flops": 512.0 * mean["SQ_INSTS_VALU_MFMA_MOPS_BF16"],
            **{c: mean[c] for c in MFMA_COUNTERS},
        })
    rows.sort(key=lambda r: -r["mean_us"] * r["dispatches"])
    return rows


def mfma_markdown(rows) -> str:
    cols = ["kernel", "grid", "dispatches", "mean us", "clock GHz", "MfmaUtil % (GRBM)",
            "MFMA busy % (SQ span)", "coexec / busy", "VALU / MFMA insts", "SQ_INSTS_MFMA",
            "SQ_INSTS_VALU", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_VALU_MFMA_COEXEC_CYCLES",
            "SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE", "F8 MFMA GFLOP", "BF16 MFMA GFLOP"]
    lines = ["| " + " | ".join(cols) + " |", "|" + "---|" * len(cols)]
    for r in rows:
        lines.append("| " + " | ".join([
            r["kernel"], str(r["grid"]), str(r["dispatches"]), f"{r['mean_us']:.1f}",
            f"{r['clock_ghz']:.2f}", f"{100 * r['mfma_util_rocprof']:.1f}",
            f"{100 * r['mfma_util_span']:.1f}", f"{r['coexec_frac']:.2f}",
            f"{r['valu_per_mfma']:.1f}", f"{r['SQ_INSTS_MFMA']:.4g}", f"{r['SQ_INSTS_VALU']:.4g}",
            f"{r['SQ_VALU_MFMA_BUSY_CYCLES']:.4g}", f"{r['SQ_VALU_MFMA_COEXEC_CYCLES']:.4g}",
            f"{r['SQ_BUSY_CYCLES']:.4g}", f"{r['GRBM_GUI_ACTIVE']:.4g}",
            f"{r['f8_flops'] / 1e9:.2f}", f"{r['bf16_flops'] / 1e9:.2f}"]) + " |")
    return "\n".join(lines)


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("traffic", help="per-call HBM bytes per launch -> profiles/traffic.json")
    t.add_argument("--fetch", required=True, action="append")
    t.add_argument("--write", required=True, action="append")
    t.add_argument("--cal-fetch", required=True)
    t.add_argument("--cal-write", required=True)
    t.add_argument("--out", default=os.path.join(ROOT, "profiles", "traffic.json"))
    d = sub.add_parser("dispatches", help="HBM bytes per dispatch by kernel and grid (markdown)")
    for a in ("--fetch", "--write", "--cal-fetch", "--cal-write"):
        d.add_argument(a, required=True)
    m = sub.add_parser("mfma", help="MFMA counters per kernel and MfmaUtil (markdown)")
    m.add_argument("--csv", required=True)
    a = ap.parse_args()
    if a.cmd == "traffic":
        if len(a.fetch) != len(a.write):
            raise SystemExit("give one --write run per --fetch run")
        rec = traffic(a.fetch, a.write, a.cal_fetch, a.cal_write)
        with open(a.out, "w") as f:
            json.dump(rec, f, indent=1, sort_keys=True)
            f.write("\n")
        print(json.dumps(rec, indent=1, sort_keys=True))
    elif a.cmd == "dispatches":
        print(dispatches(a.fetch, a.write, a.cal_fetch, a.cal_write))
    else:
        print(mfma_markdown(mfma_summary(a.csv)))


if __name__ == "__main__":
    main()
