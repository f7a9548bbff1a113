"""Host logic of the rocprofv3 summaries: kernel classification and the counter arithmetic,
on a small hand-written counter csv (no GPU)."""
import csv
import os

from dsa_sparse_attention_amd import profiling

NS = "void dsa::(anonymous namespace)::"
FIELDS = ["Dispatch_Id", "Grid_Size", "Kernel_Name", "Counter_Name", "Counter_Value",
          "Start_Timestamp", "End_Timestamp"]


def write_csv(path, rows):
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=FIELDS)
        wr.writeheader()
        for r in rows:
            wr.writerow(r)


def test_classify_modes_and_launch_counting():
    score = NS + "index_score_kernel<128, 4, 6, 0>(unsigned char const*, int)"
    compact = NS + "index_score_kernel<128, 4, 6, 2>(unsigned char const*, int)"
    assert profiling.short_name(score) == "index_score_kernel<128, 4, 6, 0>"
    assert profiling.classify(score)[0] == "index_score" and profiling.primary(score)
    assert profiling.classify(compact)[0] == "index_topk" and not profiling.primary(compact)
    assert profiling.primary(NS + "fused_select_kernel(int)")
    # a refined top-k call: the scale pre-pass is part of it, the select kernel counts it
    assert profiling.classify(NS + "topk_scale_max_kernel(float)")[0] == "topk"
    assert not profiling.primary(NS + "topk_scale_max_kernel(float)")
    assert profiling.primary(NS + "topk_kernel(float)")
    assert profiling.classify(NS + "mla_combine_kernel(int)")[0] == "sparse_mla"
    assert not profiling.primary(NS + "mla_combine_kernel(int)")
    assert profiling.classify("void at::native::elementwise_kernel<128>(int)") == (None, None)


def test_traffic_and_mfma_arithmetic(tmp_path):
    k = NS + "index_score_kernel<128, 4, 6, 0>(int)"
    cal = os.path.join(tmp_path, "cal.csv")
    # the calibration copy: 2^30 bytes counted as 2^19 KiB fetched (factor 2) and 2^20 written
    write_csv(cal, [dict(Dispatch_Id=1, Grid_Size=1, Kernel_Name="copy", Counter_Name=c,
                         Counter_Value=v, Start_Timestamp=0, End_Timestamp=1)
                    for c, v in (("FETCH_SIZE", 2 ** 19), ("WRITE_SIZE", 2 ** 20))])
    run = os.path.join(tmp_path, "run.csv")
    write_csv(run, [dict(Dispatch_Id=d, Grid_Size=64, Kernel_Name=k, Counter_Name=c,
                         Counter_Value=v, Start_Timestamp=0, End_Timestamp=1000)
                    for d in (1, 2) for c, v in (("FETCH_SIZE", 1000), ("WRITE_SIZE", 10))])
    rec = profiling.traffic([run], [run], cal, cal)
    assert rec["calibration"]["fetch_factor"] == 2.0
    e = rec["index_score"]
    assert e["launches"] == 2
    assert e["fetch_bytes_per_launch"] == 2 * 1000 * 1024
    assert e["write_bytes_per_launch"] == 10 * 1024
    # MFMA busy 1024 SIMDs x 500 cycles over a span of 1000 cycles (32 shader engines): 50%
    mf = os.path.join(tmp_path, "mfma.csv")
    vals = {"SQ_INSTS_MFMA": 100, "SQ_INSTS_VALU": 800, "SQ_VALU_MFMA_BUSY_CYCLES": 1024 * 500,
            "SQ_VALU_MFMA_COEXEC_CYCLES": 1024 * 250, "SQ_BUSY_CYCLES": 32 * 1000,
            "GRBM_GUI_ACTIVE": 8 * 2000, "SQ_INSTS_VALU_MFMA_MOPS_F8": 4,
            "SQ_INSTS_VALU_MFMA_MOPS_BF16": 0}
    write_csv(mf, [dict(Dispatch_Id=1, Grid_Size=64, Kernel_Name=k, Counter_Name=c,
                        Counter_Value=v, Start_Timestamp=0, End_Timestamp=500)
                   for c, v in vals.items()])
    (r,) = profiling.mfma_summary(mf)
    assert abs(r["mfma_util_span"] - 0.5) < 1e-12
    assert abs(r["mfma_util_rocprof"] - 0.25) < 1e-12  # GRBM window of 2000 cycles per XCD
    assert abs(r["coexec_frac"] - 0.5) < 1e-12
    assert r["valu_per_mfma"] == 8.0 and r["f8_flops"] == 2048.0
    assert abs(r["clock_ghz"] - 2.0) < 1e-12  # 1000 cycles in 500 ns
    assert "index_score_kernel<128, 4, 6, 0>" in profiling.mfma_markdown([r])
