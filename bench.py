"""Benchmark of the DSA verify step on one MI355X.

One step = one pass of the whole hot path over a batch of verify rows:
quantise the indexer queries (Hadamard + e4m3fn), score every visible index key
(FP8 MFMA), select the per-row top-k, run sparse MLA over the selected latent rows,
and take the greedy acceptance of the drafts. The index K cache (keys quantised once,
as at cache-write time), the latent cache and the logits are resident in HBM before
timing starts; three copies of every input rotate across steps so that no step is
served from the 256 MB MALL left warm by the previous one.

Prints one JSON line. ``value`` is verify query rows per second (rows of the batch /
step time), from a pass of K steps with nothing recorded between kernels. Per-kernel
times come from a second pass of K steps with HIP events recorded between consecutive
kernels on the stream they run on.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0         # MI355X HBM3E
FP8_PEAK_TFLOPS = 5000.0      # dense FP8 MFMA
BF16_PEAK_TFLOPS = 2500.0     # dense BF16 MFMA


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--min-warmup-s", type=float, default=0.3,
                    help="keep warming up past --warmup steps until this much wall time has "
                         "passed (the GPU clock ramps up under sustained load; 0 disables)")
    ap.add_argument("--workload", default="mtp5_verify_64k")
    ap.add_argument("--copies", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--accept", choices=("greedy", "rejection"), default="greedy",
                    help="acceptance rule of the step: greedy argmax prefix, or rejection "
                         "sampling against a draft law (uniforms drawn per step copy)")
    ap.add_argument("--no-refine", action="store_true",
                    help="top-k on the float32 scores alone (default: the exact-boundary refine, "
                         "so the step's top-k sets are the oracle's)")
    ap.add_argument("--topk-path", choices=("fused", "separate"), default="separate",
                    help="fused: dsa_index_topk (scores and refined top-k in one call, no score "
                         "rows); separate: dsa_index_score, then dsa_topk with the refine")
    ap.add_argument("--err-scale", type=float, default=0.0,
                    help="C of the refine's error bound (0: the library default, 4)")
    ap.add_argument("--mla-cache", choices=("bf16", "fp8"), default="bf16",
                    help="latent cache of the sparse MLA: bf16 rows (1152 B) or FP8 rows (656 B: "
                         "512 e4m3fn codes, 4 float32 block scales, 64 bf16 rope), written by "
                         "the step's cache write and read by dsa_sparse_mla_decode_fp8")
    ap.add_argument("--no-share", action="store_true",
                    help="draft steps select their own top-k (quantise q, index score over the "
                         "whole context, refined top-k) instead of reusing the step-0 top-k; "
                         "only for workloads with draft steps")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (HBM counter calibration) and exit")
    return ap.parse_args()


def calibrate_copy():
    """A plain elementwise kernel that reads and writes exactly 1 GiB each (5 launches): the
    reference against which rocprofv3 FETCH_SIZE / WRITE_SIZE are converted to bytes."""
    import torch

    n = (1 << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print("[bench] calibration copy done (5 x 1 GiB read + 1 GiB write)", file=sys.stderr, flush=True)


class Inputs:
    """One resident copy of the step's inputs (device tensors)."""

    rejection = False  # also draw rejection-sampling inputs (bench --accept rejection)
    no_share = False   # also draw the draft rows' indexer queries (bench --no-share)
    fp8_cache = False  # also hold the latent cache as FP8 rows (bench --mla-cache fp8)

    def __init__(self, w, lengths, copy: int):
        import torch

        from dsa_sparse_attention_amd import api, synth

        dev = "cuda"
        ix = synth.indexer_inputs(w, lengths, device=dev, seed_offset=copy)
        self.q_f32 = ix["q"]
        self.w = ix["w"]
        # the history's keys are quantised once when the index cache is filled; every step
        # writes the verify rows' keys and latent rows again (cache rows `dst`)
        self.dst = synth.verify_cache_rows(lengths, w.rows).to(dev)
        self.k_fp8, self.k_scale = api.quantize_fp8(ix["k"])
        # the key-scale table kept beside the index cache (the refine's eps reads it); each
        # step's cache write raises its entries for the rows it writes
        self.k_smax = api.key_scale_max(self.k_scale)
        self.k_new = ix["k"][self.dst].contiguous()
        self.k_f32_sample = ix["k"][: lengths[0]].cpu() if copy == 0 else None
        del ix
        m = synth.mla_inputs(w, lengths, device=dev, seed_offset=copy)
        self.q_mla, self.kv = m["q"], m["kv"]
        self.latent_new = self.kv[self.dst].contiguous()
        self.kv8 = api.mla_fp8_pack(self.kv) if Inputs.fp8_cache else None
        self.q_draft = None
        if w.share_steps:  # one draft row per request for each reuse step, same latent cache
            self.q_draft = [synth.mla_inputs(w, lengths, device=dev, rows=1,
                                             seed_offset=100 * (copy + 1) + j, kv=self.kv)["q"]
                            for j in range(w.share_steps)]
        self.ix_draft = None
        if w.share_steps and Inputs.no_share:  # each draft row's own indexer query and weights
            self.ix_draft = [synth.indexer_queries(w, 1, seed_offset=100 * (copy + 1) + j, device=dev)
                             for j in range(w.share_steps)]
        self.rej = synth.rejection_inputs(w, device=dev, seed_offset=copy) if Inputs.rejection else None
        a = synth.accept_inputs(w, device=dev) if copy == 0 else None
        if a is None:
            a = Inputs.accept_cache
        else:
            Inputs.accept_cache = a
        self.logits = a["logits"].clone()
        self.draft = a["draft"].clone()
        torch.cuda.synchronize()


def source_sha(name: str) -> str:
    """Hash of a call's source file(s): one name, or several joined by '+'."""
    h = hashlib.sha256()
    for n in name.split("+"):
        h.update(open(os.path.join(ROOT, "dsa_sparse_attention_amd", "csrc", n), "rb").read())
    return h.hexdigest()[:16]


def traffic_for(kernel_file: str, launches_key: str):
    """HBM traffic per launch from the committed rocprofv3 --pmc summary, if still current."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    rec = json.load(open(p)).get(launches_key)
    if not rec or rec.get("source_sha") != source_sha(kernel_file):
        return None  # counters were taken on a different kernel source
    return rec.get("hbm_bytes_per_launch")


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, lengths, inp0, target_s: float):
    """Time the oracle (as it stands) on a bounded sample: whole requests of this workload.

    Per sampled request the timed stages are the ones the GPU step runs: quantising the
    step's queries and its verify rows' new keys (the cache write), the index score over the
    request's whole history, top-k, sparse MLA and the acceptance. The history's keys are
    quantised once beforehand, as the index cache is filled before the step on the GPU too.
    """
    import numpy as np

    import oracle

    t_ = __import__("torch")
    q_all = inp0.q_f32.cpu().numpy()
    w_all = inp0.w.cpu().numpy()
    qm_all = inp0.q_mla.view(t_.uint16)
    logits = inp0.logits
    draft = inp0.draft.cpu().numpy()
    L = lengths[0]
    kf = inp0.k_f32_sample.numpy()
    kc, ks = oracle.quantize(kf)  # the index cache of the sampled history (not timed)
    k_new = np.ascontiguousarray(kf[L - w.rows:])
    kv_host = inp0.kv[:L].view(t_.uint16).cpu().numpy()
    rej_host = None
    if inp0.rej is not None:
        rl = inp0.rej["logits"]
        rej_host = {k: v.cpu().numpy() for k, v in inp0.rej.items() if k != "logits"}
        rej_host["logits"] = (rl.view(t_.uint16) if rl.dtype == t_.bfloat16 else rl).cpu().numpy()
    stages = {"cache_write": 0.0, "index_score": 0.0, "topk": 0.0, "sparse_mla": 0.0,
              "accept": 0.0}
    done_rows, t_total = 0, 0.0
    b = 0
    while b < w.batch and (t_total < target_s or b == 0):
        # every sampled request reuses request 0's caches (same shapes) with its own rows
        rows = slice(b * w.rows, (b + 1) * w.rows)
        q = np.ascontiguousarray(q_all[rows])
        wt = np.ascontiguousarray(w_all[rows])
        qm = qm_all[rows].cpu().numpy()
        lg = logits[rows].view(t_.uint16).cpu().numpy()
        qo1 = np.array([0, w.rows], np.int32)
        ko1 = np.array([0, L], np.int64)
        nvis = np.array([L - w.rows + r + 1 for r in range(w.rows)])
        t0 = time.perf_counter()
        qc, qs = oracle.quantize(q)
        oracle.quantize(k_new)
        t1 = time.perf_counter()
        sc = oracle.index_score(qc, qs, wt, kc, ks, qo1, ko1)
        t2 = time.perf_counter()
        tk = oracle.topk(sc, nvis, w.topk)
        t3 = time.perf_counter()
        oracle.sparse_mla(qm, kv_host, tk, qo1, ko1, w.sm_scale)
        t4 = time.perf_counter()
        if inp0.rej is None:
            oracle.greedy_accept(lg, draft[b:b + 1], w.drafts)
        else:
            r = rej_host
            oracle.rejection_accept(r["logits"][rows], r["draft_probs"][b:b + 1], r["draft"][b:b + 1],
                                    r["u"][b:b + 1], r["us"][b:b + 1], w.drafts)
        t5 = time.perf_counter()
        for name, dt in zip(stages, (t1 - t0, t2 - t1, t3 - t2, t4 - t3, t5 - t4)):
            stages[name] += dt
        t_total += t5 - t0
        done_rows += w.rows
        b += 1
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": done_rows / t_total, "unit": "rows/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(),
            "stages_s": {k: round(v, 3) for k, v in stages.items()},
            "sample": f"{b} request(s) x {w.rows} rows at context {L}: quantise the step's "
                      f"queries and new keys, index score, top-k, sparse MLA, "
                      f"{'greedy' if inp0.rej is None else 'rejection-sampling'} accept "
                      f"({t_total:.1f} s; history keys quantised beforehand, untimed)"}


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the verify step is "
              "data-parallel per request and this build measures one GPU's share.",
              file=sys.stderr)
        sys.exit(2)
    import torch

    from dsa_sparse_attention_amd import accounting, api, synth, workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    w = workloads.ALL[args.workload]
    lengths = synth.context_lengths(w)
    T = w.batch * w.rows
    max_kv = max(lengths)
    dev = "cuda"
    print(f"[bench] workload {w.name}: B={w.batch} ctx={max_kv} rows={w.rows} T={T}", file=sys.stderr,
          flush=True)
    Inputs.rejection = args.accept == "rejection"
    if args.no_share and not w.share_steps:
        sys.exit(f"bench.py: --no-share needs a workload with draft steps ({w.name} has none)")
    if args.no_share and (args.no_refine or args.topk_path == "fused"):
        sys.exit("bench.py: --no-share runs the separate path with the refine")
    Inputs.no_share = args.no_share
    Inputs.fp8_cache = fp8 = args.mla_cache == "fp8"
    copies = [Inputs(w, lengths, c) for c in range(args.copies)]
    qo = synth.q_row_offsets(w).to(dev)
    ko = synth.kv_row_offsets(lengths).to(dev)
    ld = (max_kv + 3) // 4 * 4
    scores = torch.empty((T, ld), dtype=torch.float32, device=dev)
    topk = torch.empty((T, w.topk), dtype=torch.int32, device=dev)
    qc = torch.empty((T, w.index_heads, w.index_dim), dtype=torch.uint8, device=dev)
    qs = torch.empty((T, w.index_heads), dtype=torch.float32, device=dev)
    out = torch.empty((T, w.mla_heads, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((T, w.mla_heads), dtype=torch.float32, device=dev)
    ws_need = api.sparse_mla_workspace_size(T, w.mla_heads, w.topk)
    ws_mla = torch.empty(max(ws_need, 16), dtype=torch.uint8, device=dev)
    from dsa_sparse_attention_amd import _lib
    fused = args.topk_path == "fused"
    if fused and args.no_refine:
        sys.exit("bench.py: the fused path always refines (--no-refine needs --topk-path separate)")
    refine = not args.no_refine
    tk_need = api.topk_workspace_size(w.batch, T, max_kv, w.topk, refine)
    status = torch.zeros(T, dtype=torch.int32, device=dev)
    path = torch.zeros(T, dtype=torch.int32, device=dev)
    ws_fused = None
    if fused:
        ws_fused = torch.empty(api.index_topk_workspace_size(w.batch, T, w.rows, w.index_heads, max_kv),
                               dtype=torch.uint8, device=dev)
    ws_tk = torch.empty(max(tk_need, 16), dtype=torch.uint8, device=dev)
    ga_need = _lib.load().greedy_accept_workspace_size(w.batch, w.drafts, w.vocab)
    ws_ga = torch.empty(max(ga_need, 16), dtype=torch.uint8, device=dev)
    ra_need = _lib.load().rejection_accept_workspace_size(w.batch, w.drafts, w.vocab)
    ws_ra = torch.empty(max(ra_need, 16), dtype=torch.uint8, device=dev)
    print(f"[bench] inputs resident ({args.copies} copies); mla workspace {ws_need/1e6:.1f} MB",
          file=sys.stderr, flush=True)

    acc_name = "greedy_accept" if args.accept == "greedy" else "rejection_accept"
    names = (["cache_write", "index_topk", "sparse_mla", acc_name] if args.topk_path == "fused" else
             ["cache_write", "index_score", "topk", "sparse_mla", acc_name])
    if w.share_steps:
        names.append("draft_steps" if args.no_share else "share_mla")
        qo1 = torch.arange(w.batch + 1, dtype=torch.int32, device=dev)
        n_acc = synth.accepted_lengths(w).to(dev)
        out1 = torch.empty((w.batch, w.mla_heads, 512), dtype=torch.bfloat16, device=dev)
        lse1 = torch.empty((w.batch, w.mla_heads), dtype=torch.float32, device=dev)
        ws1_need = api.sparse_mla_workspace_size(w.batch, w.mla_heads, w.topk)
        ws1 = torch.empty(max(ws1_need, 16), dtype=torch.uint8, device=dev)
        if args.no_share:  # one draft row per request, visible to the whole cached context
            qc1 = torch.empty((w.batch, w.index_heads, w.index_dim), dtype=torch.uint8, device=dev)
            qs1 = torch.empty((w.batch, w.index_heads), dtype=torch.float32, device=dev)
            scores1 = torch.empty((w.batch, ld), dtype=torch.float32, device=dev)
            top1 = torch.empty((w.batch, w.topk), dtype=torch.int32, device=dev)
            status1 = torch.zeros(w.batch, dtype=torch.int32, device=dev)
            tk1 = api.topk_workspace_size(w.batch, w.batch, max_kv, w.topk, True)
            ws_tk1 = torch.empty(max(tk1, 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def mla(qm, inp, tk, q_off, rows, o, l, ws, **share):
        if fp8:
            api.sparse_mla_decode_fp8(qm, inp.kv8, tk, q_off, ko, rows, w.sm_scale, out=o, lse=l,
                                      workspace=ws, **share)
        else:
            api.sparse_mla_decode(qm, inp.kv, tk, q_off, ko, rows, w.sm_scale, out=o, lse=l,
                                  workspace=ws, **share)

    def step(inp, ev=None):
        e = iter(ev) if ev else None
        mark = (lambda: next(e).record(stream)) if ev else (lambda: None)
        mark()
        if not fp8:
            api.verify_cache_write(inp.k_new, inp.dst, inp.k_fp8, inp.k_scale, inp.latent_new, inp.kv,
                                   q=inp.q_f32, q_fp8=qc, q_scale=qs, k_scale_max=inp.k_smax)
        else:  # index keys and queries, then the verify rows' latent rows packed to FP8
            api.verify_cache_write(inp.k_new, inp.dst, inp.k_fp8, inp.k_scale, q=inp.q_f32, q_fp8=qc,
                                   q_scale=qs, k_scale_max=inp.k_smax)
            api.mla_fp8_pack(inp.latent_new, inp.kv8, dst_rows=inp.dst)
        mark()
        if fused:
            api.index_topk(qc, qs, inp.w, inp.k_fp8, inp.k_scale, qo, ko, w.rows, max_kv, w.topk,
                           out=topk, status=status, path=path, err_scale=args.err_scale,
                           workspace=ws_fused)
            mark()
        else:
            api.index_score(qc, qs, inp.w, inp.k_fp8, inp.k_scale, qo, ko, w.rows, max_kv, scores=scores)
            mark()
            rf = (dict(q_fp8=qc, q_scale=qs, w=inp.w, k_fp8=inp.k_fp8, k_scale=inp.k_scale,
                       status=status, err_scale=args.err_scale, k_scale_max=inp.k_smax)
                  if refine else None)
            api.topk(scores, qo, ko, w.rows, max_kv, w.topk, out=topk, refine=rf, workspace=ws_tk)
            mark()
        mla(inp.q_mla, inp, topk, qo, w.rows, out, lse, ws_mla)
        mark()
        if inp.rej is None:
            api.greedy_accept(inp.logits, inp.draft, w.drafts, argmax=False, workspace=ws_ga)
        else:
            r = inp.rej
            api.rejection_accept(r["logits"], r["draft_probs"], r["draft"], r["u"], r["us"],
                                 w.drafts, workspace=ws_ra)
        mark()
        for j, qd in enumerate(inp.q_draft or []):
            if inp.ix_draft is None:  # index share: the step-0 top-k row at the accepted position
                mla(qd, inp, topk, qo1, 1, out1, lse1, ws1, share_base=qo, num_accepted=n_acc)
                continue
            ixd = inp.ix_draft[j]  # no share: the draft row runs the indexer over the whole cache
            api.quantize_fp8(ixd["q"], out=qc1, scale=qs1)
            api.index_score(qc1, qs1, ixd["w"], inp.k_fp8, inp.k_scale, qo1, ko, 1, max_kv,
                            scores=scores1)
            api.topk(scores1, qo1, ko, 1, max_kv, w.topk, out=top1, workspace=ws_tk1,
                     refine=dict(q_fp8=qc1, q_scale=qs1, w=ixd["w"], k_fp8=inp.k_fp8,
                                 k_scale=inp.k_scale, status=status1, err_scale=args.err_scale,
                                 k_scale_max=inp.k_smax))
            mla(qd, inp, top1, qo1, 1, out1, lse1, ws1)
        if inp.q_draft:
            mark()

    # Warm-up: at least --warmup steps, and steps in groups of 50 until --min-warmup-s of
    # wall time has passed. Under sustained load the GPU raises its clock within tens of
    # milliseconds; a handful of steps times the kernels at a lower clock than a serving loop
    # runs them.
    warm0 = time.perf_counter()
    n_warm = 0
    while n_warm < args.warmup or time.perf_counter() - warm0 < args.min_warmup_s:
        for _ in range(args.warmup if n_warm < args.warmup else 50):
            step(copies[n_warm % len(copies)])
            n_warm += 1
        torch.cuda.synchronize()
    # timed pass: the steps alone (no event between kernels), bracketed by events and
    # device synchronisation
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(args.steps):
        step(copies[i % len(copies)])
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)
    ms_step = total_ms / args.steps
    # breakdown pass: the same steps again with an event between consecutive kernels
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
           for _ in range(args.steps)]
    for i in range(args.steps):
        step(copies[i % len(copies)], evs[i])
    torch.cuda.synchronize()
    per = {n: sum(evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(args.steps)) / args.steps
           for j, n in enumerate(names)}
    refine_rec = None
    if refine:
        # every row of the last step must be refined (status >= 0): its top-k set is then
        # the oracle's, provided the float32 errors stay within the bound (see dsa.h)
        st = status.cpu() if not args.no_share else torch.cat([status.cpu(), status1.cpu()])
        assert int(st.min()) >= 0, f"refine left rows unresolved: statuses {sorted(set(st.tolist()))}"
        refine_rec = {"status_min": int(st.min()), "band_max": int(st.max()),
                      "band_mean": round(float(st.float().mean()), 2),
                      "err_scale": args.err_scale or 4.0}
        if fused:
            refine_rec["rows_rescored"] = int(path.sum().item())
    print(f"[bench] {args.steps} steps: {ms_step:.4f} ms/step (wall {wall / args.steps * 1e3:.4f} ms); "
          + ", ".join(f"{n} {v * 1e3:.1f} us" for n, v in per.items()), file=sys.stderr, flush=True)

    # algorithmic work (bytes / flops the method must move or do)
    wi = accounting.index_score_work(lengths, w.rows, w.index_heads, w.index_dim)
    wt = accounting.topk_work(lengths, w.rows, w.topk)
    row_bytes = accounting.FP8_ROW_BYTES if fp8 else 2 * 576
    wm = accounting.sparse_mla_work(T, w.mla_heads, w.topk, row_bytes=row_bytes)
    wg = (accounting.greedy_accept_work if args.accept == "greedy" else
          accounting.rejection_accept_work)(w.batch, w.drafts, w.vocab, 2)
    wq = dict(bytes=T * (w.index_heads + 1) * (w.index_dim * 4 + w.index_dim + 4) + T * (1152 + row_bytes))
    kern = {
        "cache_write": dict(bytes=wq["bytes"], bound="hbm", file="quantize.hip"),
        "sparse_mla": dict(bytes=wm["bytes"], flops=wm["flops"], bound="hbm", file="sparse_mla.hip",
                           traffic_key="sparse_mla_fp8" if fp8 else "sparse_mla"),
        acc_name: dict(bytes=wg["bytes"], bound="hbm",
                       file="greedy_accept.hip" if args.accept == "greedy" else "rejection_accept.hip"),
    }
    if fused:
        wf = accounting.index_topk_work(lengths, w.rows, w.index_heads, w.index_dim, w.topk)
        kern["index_topk"] = dict(bytes=wf["bytes"], flops=wf["flops"], bound="mfma",
                                  file="index_score.hip+topk.hip")
    else:
        kern["index_score"] = dict(bytes=wi["bytes"], flops=wi["flops"], bound="mfma",
                                   file="index_score.hip")
        kern["topk"] = dict(bytes=wt["bytes"], bound="hbm", file="topk.hip")
    if w.share_steps and not args.no_share:
        ws_ = accounting.sparse_mla_work(w.batch, w.mla_heads, w.topk, row_bytes=row_bytes)
        kern["share_mla"] = dict(bytes=w.share_steps * ws_["bytes"],
                                 flops=w.share_steps * ws_["flops"], bound="hbm")
    elif w.share_steps:  # several kernels per draft step: reported, never the roofline kernel
        ws_ = accounting.sparse_mla_work(w.batch, w.mla_heads, w.topk, row_bytes=row_bytes)
        wi1 = accounting.index_score_work(lengths, 1, w.index_heads, w.index_dim)
        wt1 = accounting.topk_work(lengths, 1, w.topk)
        kern["draft_steps"] = dict(bytes=w.share_steps * (ws_["bytes"] + wi1["bytes"] + wt1["bytes"]),
                                   bound="hbm", composite=True)
    kernels = {}
    for n, kd in kern.items():
        t_s = per[n] * 1e-3
        e = {"us": round(per[n] * 1e3, 2), "GB/s": round(kd["bytes"] / t_s / 1e9, 1),
             "hbm_frac": round(kd["bytes"] / t_s / 1e9 / HBM_PEAK_GBS, 4)}
        if "flops" in kd:
            peak = FP8_PEAK_TFLOPS if n in ("index_score", "index_topk") else BF16_PEAK_TFLOPS
            e["TFLOP/s"] = round(kd["flops"] / t_s / 1e12, 1)
            e["mfma_frac"] = round(kd["flops"] / t_s / 1e12 / peak, 4)
        kernels[n] = e
    dom = max((n for n in per if not kern[n].get("composite")), key=per.get)
    kd = kern[dom]
    t_dom = per[dom] * 1e-3
    if kd["bound"] == "mfma":
        peak = FP8_PEAK_TFLOPS
        ach = kd["flops"] / t_dom / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(ach / peak, 4)}
    else:
        ach = kd["bytes"] / t_dom / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4)}
    roof["kernel"] = dom
    roof["traffic"] = (traffic_for(kd["file"], kd.get("traffic_key", dom))
                       if kd.get("file") and not (fp8 and dom == "cache_write") else None)

    rows_step = T + w.share_steps * w.batch  # verify rows, plus one draft row per reuse step
    value = rows_step / (ms_step * 1e-3)
    rec = {
        "metric": "verify query rows/sec (indexer+top-k+sparse MLA) at 64K ctx; HBM GB/s, MFMA %",
        "value": round(value, 1), "unit": "rows/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "warmup_steps_run": n_warm, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8+bf16", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "context": max_kv, "rows_per_request": w.rows,
                   "index_heads": w.index_heads, "index_dim": w.index_dim, "topk": w.topk,
                   "mla_heads": w.mla_heads, "vocab": w.vocab, "global_batch": rows_step,
                   "seq_len": max_kv, "share_steps": w.share_steps, "topk_refine": refine,
                   "topk_path": args.topk_path, "mla_cache": args.mla_cache, "index_share": (not args.no_share) if w.share_steps else None,
                   "accept": args.accept,
                   "parallelism": "single-gpu"},
        "step_includes": names,
        "rows_per_s_indexer_topk_mla": round(T / ((per.get("index_topk", 0.0) + per.get("index_score", 0.0) +
                                                  per.get("topk", 0.0) + per["sparse_mla"]) * 1e-3), 1),
        "kernels": kernels,
        "roofline": roof,
        "refine": refine_rec,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(w, lengths, copies[0], args.cpu_seconds)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec, ensure_ascii=False), flush=True)


if __name__ == "__main__":
    main()
