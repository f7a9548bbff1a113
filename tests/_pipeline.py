"""Shared helpers of the parity tests: run the HIP path and the oracle on the same seeded inputs.

The HIP side quantises, scores, selects and attends with libdsa.so; the oracle side does
every step again from the same float inputs with the CPU oracle. Nothing computed by the
HIP path is ever fed to the oracle.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from dsa_sparse_attention_amd import api, synth
from dsa_sparse_attention_amd.workloads import Workload

DEV = "cuda"


class Case:
    """Seeded inputs of one workload, on the host (for the oracle) and on the device."""

    def __init__(self, w: Workload, gen_device: str = "cpu", with_mla: bool = True,
                 with_accept: bool = True):
        self.w = w
        self.lengths = synth.context_lengths(w)
        self.qo = synth.q_row_offsets(w)
        self.ko = synth.kv_row_offsets(self.lengths)
        self.T = int(self.qo[-1])
        self.max_kv = max(self.lengths)
        ix = synth.indexer_inputs(w, self.lengths, device=gen_device)
        self.spike_pos = ix["spike_pos"]
        self.q_f32 = ix["q"].to(DEV)
        self.k_f32 = ix["k"].to(DEV)
        self.w_f32 = ix["w"].to(DEV)
        self.qo_d = self.qo.to(DEV)
        self.ko_d = self.ko.to(DEV)
        self.mla = None
        if with_mla:
            m = synth.mla_inputs(w, self.lengths, device=gen_device)
            self.mla = {k: v.to(DEV) for k, v in m.items()}
        self.acc = None
        if with_accept:
            a = synth.accept_inputs(w, device=gen_device)
            self.acc = {k: (v.to(DEV) if k != "planted_n" else v) for k, v in a.items()}

    # ---- host copies for the oracle ----
    def host(self, name):
        return getattr(self, name).cpu().numpy()

    def visible(self, t: int) -> int:
        return oracle.row_visible(self.qo.numpy(), self.ko.numpy(), t)


def gpu_indexer(case: Case):
    """HIP path: quantise q/k, score, top-k. Returns device tensors."""
    w = case.w
    qc, qs = api.quantize_fp8(case.q_f32)
    kc, ks = api.quantize_fp8(case.k_f32)
    scores = api.index_score(qc, qs, case.w_f32, kc, ks, case.qo_d, case.ko_d, w.rows, case.max_kv)
    top = api.topk(scores, case.qo_d, case.ko_d, w.rows, case.max_kv, w.topk)
    return dict(qc=qc, qs=qs, kc=kc, ks=ks, scores=scores, topk=top)


def oracle_quant(case: Case, rows=None, requests=None):
    """Oracle quantisation of q (all rows) and of the keys of the given requests (None = all)."""
    qc, qs = oracle.quantize(case.host("q_f32"))
    if requests is None:
        kc, ks = oracle.quantize(case.host("k_f32"))
        return qc, qs, kc, ks, case.ko.numpy()
    # only the keys of the listed requests, laid out compactly with re-based offsets
    ko = case.ko.numpy()
    parts_c, parts_s, offs = [], [], [0]
    k_all = case.k_f32
    for b in range(len(case.lengths)):
        if b in requests:
            c, s = oracle.quantize(k_all[int(ko[b]):int(ko[b + 1])].cpu().numpy())
        else:
            c = np.zeros((0, case.w.index_dim), np.uint8)
            s = np.zeros(0, np.float32)
        parts_c.append(c)
        parts_s.append(s)
        offs.append(offs[-1] + len(s) if b in requests else offs[-1])
    return (qc, qs, np.concatenate(parts_c), np.concatenate(parts_s),
            np.array(offs, np.int64))


# The refine's default error scale C = 4 is 1/32 of the per-head worst case of the FP8 MFMA's
# accumulation (C = 128, the model score_tolerance states per key), and a row's band is
# resolved only if every float32 score lies within half of its eps of the exact value. So the
# default refine is exact only while the scores stay within 1/64 of score_tolerance; the score
# tests hold them to that margin as well as to the bound.
REFINE_MARGIN = 1.0 / 64.0


def score_tolerance(qc, qs, w, kc, ks, rows, qo, ko, width):
    """Bound on |I_gpu - I_oracle| per (row, key) from the arithmetic of the HIP path.

    Per head the FP8 MFMA sums the 128 exact products on a grid 16 bits below the
    largest product (measured behaviour of v_mfma_f32_16x16x128_f8f6f4), so
    |d_gpu - d| <= 128 * 2^-16 * max_i |q_i k_i| <= 2^-9 * max|q_hat_j| * max|k_hat_s|.
    ReLU is 1-Lipschitz; the float32 epilogue (u = w*s_q, H products, H adds, the
    key-scale multiply) adds (H+3) * 2^-24 relative to sum_j |u_j| |d_j| (bounded via
    sum_j |u_j| * 448 * max|k_hat| * D).
    """
    dec = oracle.fp8_decode(np.arange(256, dtype=np.uint8))
    qmax = np.abs(dec[qc]).max(axis=-1)                    # [T, H]
    kmax = np.abs(dec[kc]).max(axis=-1)                    # [N]
    H, D = qc.shape[1], qc.shape[2]
    u = np.abs(w.astype(np.float64) * qs.astype(np.float64))  # [T, H]
    out = np.zeros((len(rows), width))
    for i, t in enumerate(rows):
        b = int(np.searchsorted(qo, t, side="right") - 1)
        L = int(ko[b + 1] - ko[b])
        km = kmax[ko[b]:ko[b] + L]
        kss = ks[ko[b]:ko[b] + L].astype(np.float64)
        mfma = 2.0 ** -9 * (u[t] * qmax[t]).sum() * km
        f32 = (H + 3) * 2.0 ** -24 * (u[t] * qmax[t]).sum() * km * D
        out[i, :L] = kss * (mfma + f32)
    return out


def check_topk_valid(gpu_rows, ref_rows, ref_scores, nvis, tol, k):
    """Compare top-k sets: equal, or differing only inside the error band of the k-th score.

    Returns the number of rows whose sets differ (all differences validated).
    """
    ndiff = 0
    for i in range(len(gpu_rows)):
        g = gpu_rows[i]
        r = ref_rows[i]
        assert np.all(np.diff(g[g >= 0]) > 0), "HIP top-k not strictly ascending"
        assert np.array_equal(g >= 0, r >= 0), "valid-entry count differs"
        gs, rs = set(g[g >= 0].tolist()), set(r[r >= 0].tolist())
        if gs == rs:
            continue
        ndiff += 1
        n = int(nvis[i])
        theta = np.sort(ref_scores[i, :n])[::-1][min(k, n) - 1]
        band = 2.0 * tol[i, :n].max()
        for s in gs ^ rs:
            assert abs(ref_scores[i, s] - theta) <= band, (
                f"row {i}: position {s} differs but lies outside the error band "
                f"({ref_scores[i, s]} vs theta {theta}, band {band})")
    return ndiff


LSE_TOL = 1e-3  # the sparse-MLA tolerance's lse term, |d lse| <= 1e-3 (natural log)


def mla_check(out_gpu, lse_gpu, out_ref, lse_ref):
    """Sparse-MLA tolerance: |d| <= 2e-2*max|o_ref| (per row/head) + 1e-2*|o_ref|, and
    |d lse| <= 1e-3. Prints the worst ratio to the bound and the worst |d lse|."""
    og = out_gpu.float().cpu().numpy().astype(np.float64)
    scale = np.abs(out_ref).max(axis=-1, keepdims=True)
    bound = 2e-2 * scale + 1e-2 * np.abs(out_ref)
    err = np.abs(og - out_ref)
    worst = float((err / np.maximum(bound, 1e-30)).max()) if err.size else 0.0
    lg = lse_gpu.cpu().numpy().astype(np.float64)
    fin = np.isfinite(lse_ref)
    dl = np.abs(lg[fin] - lse_ref[fin])
    worst_lse = float(dl.max()) if dl.size else 0.0
    print(f"  mla: worst |d|/bound {worst:.3f}, worst |d lse| {worst_lse:.2e}", flush=True)
    assert np.all(err <= bound), f"sparse MLA out of tolerance (worst ratio {worst:.3f})"
    assert np.array_equal(np.isfinite(lg), fin)
    assert worst_lse <= LSE_TOL, f"lse off by {worst_lse:.2e}"
    return worst


def refine_args(gi, case, status: bool = True):
    """dsa_topk refine inputs: the HIP path's own quantised q/k (device), weights, status."""
    d = dict(q_fp8=gi["qc"], q_scale=gi["qs"], w=case.w_f32, k_fp8=gi["kc"], k_scale=gi["ks"])
    if status:
        d["status"] = torch.zeros(case.T, dtype=torch.int32, device=DEV)
    return d


def refine_eps(qc, qs, w, ks, qo, ko, rows, theta, C: float = 4.0):
    """Per-row refine bound, written from the statement of dsa_topk in include/dsa.h on the
    host copies: eps_t = C 2^-16 448 smax_t sum_j |u_j| max|q_hat_j| + (H + 3) 2^-23 |theta_t|,
    smax_t the largest key scale of the 2048-position chunks holding the row's visible keys,
    theta_t the row's k-th largest float32 score (given)."""
    dec = oracle.fp8_decode(np.arange(256, dtype=np.uint8))
    qmax = np.abs(dec[qc]).max(axis=-1)                                # [T, H]
    u = np.abs(w.astype(np.float64) * qs.astype(np.float64))          # [T, H]
    H = qc.shape[1]
    out = np.zeros(len(rows))
    for i, t in enumerate(rows):
        b = int(np.searchsorted(qo, t, side="right") - 1)
        n = oracle.row_visible(qo, ko, int(t))
        L = int(ko[b + 1] - ko[b])
        end = min(L, -(-n // 2048) * 2048)
        smax = float(np.abs(ks[ko[b]:ko[b] + end]).max()) if n else 0.0
        out[i] = (C * 2.0 ** -16 * 448.0 * smax * float((u[t] * qmax[t]).sum())
                  + (H + 3) * 2.0 ** -23 * abs(float(theta[i])))
    return out


def kth_largest(scores, nvis, k):
    """The k-th largest of each row's visible scores (the smallest score when k > visible)."""
    out = np.zeros(len(nvis))
    for i, n in enumerate(nvis):
        if n:
            row = np.sort(scores[i, :n])[::-1]
            out[i] = row[min(k, n) - 1]
    return out
