"""Parity at full workload sizes, in the launch configuration bench.py times.

Workloads, each at its full size:
* 32 requests x 65536 positions, 6 verify rows (the bench step); the same with ragged
  contexts drawn in [8192, 65536];
* 8 requests x 16384, 2 rows, sparse MLA 128 heads (lists split over blocks and merged);
* 4 requests x 262144, 6 rows, sparse MLA 128 heads, 1% planted identical spike keys;
* 64 requests x 32768, 6 rows at step 0, then one draft row per request reusing the
  step-0 top-k at its accepted position (index share).
Indexer 64 heads x 128 (FP8) and top-k 2048 throughout. Inputs come from the seeded
generators (on the device, then copied to the host for the oracle); the HIP calls are
made with the same shapes, leading dimensions and workspaces as the bench step.

The oracle cannot score every (row, key) pair at this size in seconds, so:
* quantised codes: every query vector and a sample of 4096 key vectors, bit-exact;
* indexer scores: per sampled row, a sample of keys scored one by one by the oracle
  (a score does not depend on the key's position, only its visibility does), within the
  FP8-MFMA error bound; every row's visible prefix is written and the rest untouched;
* top-k on generated score rows (continuous and heavily tied): every row, bit-exact;
* end-to-end top-k: a few rows scored in full by the oracle; the float32 sets are equal
  up to the error band around the k-th score, the refined sets exactly;
* sparse MLA on generated index sets: a sample of rows, all heads, within the
  sparse-MLA tolerance;
* planted spikes: the top-k of every row is the request's first 2048 spike positions;
* index share: sampled requests' draft rows against the oracle's share rule;
* greedy accept at 32 x 6 x 151552 is covered by test_gpu_parity (all rows, bit-exact).
"""
import numpy as np
import pytest
import torch

import oracle
from dsa_sparse_attention_amd import api, synth, workloads
from tests._pipeline import (DEV, check_topk_valid, kth_largest, mla_check, refine_eps,
                             score_tolerance, REFINE_MARGIN)

pytestmark = pytest.mark.gpu

NAMES = ["mtp5_verify_64k", "mtp5_verify", "decode_verify", "long_ctx", "draft_share"]


def _say(*a):
    print(*a, flush=True)


class Full:
    """Device inputs and the bench-shaped launch state of one full workload."""

    def __init__(self, w):
        self.wl = w
        self.lengths = synth.context_lengths(w)
        self.T = w.batch * w.rows
        self.max_kv = max(self.lengths)
        self.ld = (self.max_kv + 3) // 4 * 4
        self.qo = synth.q_row_offsets(w)
        self.ko = synth.kv_row_offsets(self.lengths)
        self.qo_d, self.ko_d = self.qo.to(DEV), self.ko.to(DEV)
        ix = synth.indexer_inputs(w, self.lengths, device=DEV)
        self.q, self.k, self.w = ix["q"], ix["k"], ix["w"]
        self.spike_pos = ix["spike_pos"]
        self.kc, self.ks = api.quantize_fp8(self.k)
        self.qc = torch.empty((self.T, w.index_heads, w.index_dim), dtype=torch.uint8, device=DEV)
        self.qs = torch.empty((self.T, w.index_heads), dtype=torch.float32, device=DEV)
        api.quantize_fp8(self.q, out=self.qc, scale=self.qs)
        self.scores = torch.full((self.T, self.ld), float("nan"), dtype=torch.float32, device=DEV)
        api.index_score(self.qc, self.qs, self.w, self.kc, self.ks, self.qo_d, self.ko_d, w.rows,
                        self.max_kv, scores=self.scores)
        self.top = torch.empty((self.T, w.topk), dtype=torch.int32, device=DEV)
        api.topk(self.scores, self.qo_d, self.ko_d, w.rows, self.max_kv, w.topk, out=self.top)
        # the same selection with the exact-boundary refine
        self.rstatus = torch.zeros(self.T, dtype=torch.int32, device=DEV)
        self.top_ref = api.topk(self.scores, self.qo_d, self.ko_d, w.rows, self.max_kv, w.topk,
                                refine=dict(q_fp8=self.qc, q_scale=self.qs, w=self.w,
                                            k_fp8=self.kc, k_scale=self.ks, status=self.rstatus))
        # the fused path (no score rows), on the same inputs
        self.fstatus = torch.zeros(self.T, dtype=torch.int32, device=DEV)
        self.fpath = torch.zeros(self.T, dtype=torch.int32, device=DEV)
        self.top_fused = api.index_topk(self.qc, self.qs, self.w, self.kc, self.ks, self.qo_d,
                                        self.ko_d, w.rows, self.max_kv, w.topk,
                                        status=self.fstatus, path=self.fpath)
        torch.cuda.synchronize()

    def visible(self, t: int) -> int:
        return oracle.row_visible(self.qo.numpy(), self.ko.numpy(), t)

    def request(self, t: int) -> int:
        return t // self.wl.rows


@pytest.fixture(scope="module", params=NAMES)
def f(request):
    """One workload's inputs; pytest groups the tests by workload, so each is built once."""
    w = workloads.ALL[request.param]
    _say(f"building {w.name}: {w.batch} requests, context <= {w.ctx}, {w.rows} rows")
    full = Full(w)
    yield full
    del full
    torch.cuda.empty_cache()


def _sample_rows(T, R, extra, seed):
    rng = np.random.default_rng(seed)
    fixed = [0, R - 1, R, T - R, T - 1]   # first/last row of the first and last requests
    return sorted(set(fixed) | set(rng.choice(T, extra, replace=False).tolist()))


def test_full_quantize_sampled_bitexact(f):
    _say("full quantize: all query vectors, 4096 sampled key vectors")
    rc, rs = oracle.quantize(f.q.cpu().numpy())
    assert np.array_equal(f.qc.cpu().numpy(), rc)
    assert np.array_equal(f.qs.cpu().numpy(), rs)
    N = int(f.ko[-1])
    rng = np.random.default_rng(101)
    pick = np.unique(np.concatenate([[0, N - 1], rng.choice(N, 4096, replace=False)]))
    pick_d = torch.from_numpy(pick).to(DEV)
    rc, rs = oracle.quantize(f.k[pick_d].cpu().numpy())
    assert np.array_equal(f.kc[pick_d].cpu().numpy(), rc)
    assert np.array_equal(f.ks[pick_d].cpu().numpy(), rs)


def test_full_index_score_prefix_written_rest_untouched(f):
    _say("full index_score: visible prefix written, tail untouched, every row")
    vis = torch.tensor([f.visible(t) for t in range(f.T)], device=DEV)
    col = torch.arange(f.ld, device=DEV)[None, :]
    inside = col < vis[:, None]
    assert bool(torch.isfinite(f.scores[inside]).all())
    assert bool(torch.isnan(f.scores[~inside]).all())


def test_full_index_score_sampled_within_bound(f):
    W = f.wl
    rows = _sample_rows(f.T, W.rows, 7, seed=7)
    _say(f"full index_score: rows {rows}, 2048 sampled keys each")
    rng = np.random.default_rng(17)
    worst = 0.0
    for t in rows:
        b = f.request(t)
        n = f.visible(t)
        pos = np.unique(np.concatenate([[0, n - 1], rng.choice(n, 2048, replace=False)]))
        base = int(f.ko[b])
        k_host = f.k[torch.from_numpy(base + pos).to(DEV)].cpu().numpy()
        kc, ks = oracle.quantize(k_host)
        qc, qs = oracle.quantize(f.q[t:t + 1].cpu().numpy())
        wt = f.w[t:t + 1].cpu().numpy()
        # one-row request holding only the sampled keys: the row sees all of them
        qo1 = np.array([0, 1], np.int32)
        ko1 = np.array([0, len(pos)], np.int64)
        ref = oracle.index_score(qc, qs, wt, kc, ks, qo1, ko1)[0]
        tol = score_tolerance(qc, qs, wt, kc, ks, [0], qo1, ko1, len(pos))[0]
        got = f.scores[t, torch.from_numpy(pos).to(DEV)].cpu().numpy().astype(np.float64)
        err = np.abs(got - ref)
        assert np.all(err <= tol), f"row {t}: score error above bound"
        worst = max(worst, float((err / tol).max()))
    _say(f"  worst |err|/bound = {worst:.3e}")
    assert worst <= REFINE_MARGIN, "scores drift past the margin the default refine relies on"


@pytest.mark.parametrize("levels", [0, 7, 2000])
def test_full_topk_bitexact_every_row(f, levels):
    W = f.wl
    _say(f"full topk on generated scores, tie levels {levels}: all {f.T} rows")
    s = synth.random_scores(f.T, f.ld, seed=900 + levels, tie_levels=levels)
    got = torch.empty((f.T, W.topk), dtype=torch.int32, device=DEV)
    api.topk(s.to(DEV), f.qo_d, f.ko_d, W.rows, f.max_kv, W.topk, out=got)
    nvis = np.array([f.visible(t) for t in range(f.T)])
    ref = oracle.topk(s.double().numpy(), nvis, W.topk)
    assert np.array_equal(got.cpu().numpy(), ref)


def test_full_end_to_end_topk_sampled_rows(f):
    # float32 selection: equal to the oracle's set up to the error band; refined selection:
    # equal to it exactly, with the float32 scores within half the refine bound
    W = f.wl
    rows = [0, W.rows - 1, f.T - 1]
    _say(f"full end-to-end top-k: rows {rows} scored in full by the oracle")
    st = f.rstatus.cpu().numpy()
    assert st.min() >= 0, "refine band overflow"
    _say(f"  refine band sizes over all rows: max {st.max()}, mean {st.mean():.1f}")
    for t in rows:
        b = f.request(t)
        n = f.visible(t)
        base = int(f.ko[b])
        kc, ks = oracle.quantize(f.k[base:base + f.lengths[b]].cpu().numpy())
        R = W.rows
        qc, qs = oracle.quantize(f.q[b * R:(b + 1) * R].cpu().numpy())
        wt = f.w[b * R:(b + 1) * R].cpu().numpy()
        r = t - b * R                  # the row keeps its place in its request
        qo1 = np.array([0, R], np.int32)
        ko1 = np.array([0, f.lengths[b]], np.int64)
        assert oracle.row_visible(qo1, ko1, r) == n
        ref_s = oracle.index_score(qc, qs, wt, kc, ks, qo1, ko1, rows=[r], width=f.max_kv)
        ref_k = oracle.topk(ref_s, [n], W.topk)
        tol = score_tolerance(qc, qs, wt, kc, ks, [r], qo1, ko1, f.max_kv)
        nd = check_topk_valid(f.top[t:t + 1].cpu().numpy(), ref_k, ref_s, [n], tol, W.topk)
        got_s = f.scores[t, :n].cpu().numpy().astype(np.float64)
        eps = refine_eps(qc, qs, wt, ks, qo1, ko1, [r], kth_largest(got_s[None, :], [n], W.topk))[0]
        ratio = float(np.abs(got_s - ref_s[0, :n]).max() / eps)
        assert ratio <= 0.5, f"row {t}: float32 error {ratio:.3f} of the refine bound"
        assert np.array_equal(f.top_ref[t].cpu().numpy(), ref_k[0]), f"row {t}: refined set"
        _say(f"  row {t}: float32 set {'equal' if nd == 0 else 'band-only differences'}, "
             f"refined set equal (error/eps {ratio:.3f}, band {st[t]})")


def test_full_fused_topk_every_row(f):
    # the fused score + top-k and the refined top-k of the written scores both give the exact
    # sets: they must agree on every row (three rows are checked against the oracle above)
    W = f.wl
    st, path = f.fstatus.cpu().numpy(), f.fpath.cpu().numpy()
    _say(f"full fused top-k: all {f.T} rows; status min {st.min()}, band max {st.max()}, "
         f"rows rescored {int((path == 1).sum())}")
    assert st.min() >= 0
    assert np.array_equal(f.top_fused.cpu().numpy(), f.top_ref.cpu().numpy())
    if f.spike_pos is not None:
        top = f.top_fused.cpu().numpy()
        for t in range(f.T):
            assert np.array_equal(top[t], f.spike_pos[f.request(t)][:W.topk].numpy()), f"row {t}"


def test_full_sparse_mla_sampled_rows(f):
    w = f.wl
    _say(f"full sparse_mla on generated index sets: sampled rows, all {w.mla_heads} heads")
    m = synth.mla_inputs(w, f.lengths, device=DEV)
    idx = synth.random_topk(w, f.lengths, f.qo, w.topk)
    out = torch.empty((f.T, w.mla_heads, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((f.T, w.mla_heads), dtype=torch.float32, device=DEV)
    need = api.sparse_mla_workspace_size(f.T, w.mla_heads, w.topk)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=DEV)
    api.sparse_mla_decode(m["q"], m["kv"], idx.to(DEV), f.qo_d, f.ko_d, w.rows, w.sm_scale,
                          out=out, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    rows = _sample_rows(f.T, w.rows, 4, seed=23)
    u16 = lambda x: x.view(torch.uint16).cpu().numpy()
    ref_o, ref_l = oracle.sparse_mla(u16(m["q"]), u16(m["kv"]), idx.numpy(), f.qo.numpy(),
                                     f.ko.numpy(), w.sm_scale, rows=np.array(rows))
    sel = torch.tensor(rows, device=DEV)
    worst = mla_check(out[sel], lse[sel], ref_o, ref_l)
    _say(f"  rows {rows}: worst err/bound = {worst:.3f}")


def test_full_planted_spikes_topk_closed_form(f):
    # 1% of each request's keys (2621 of 262144, all visible to every row) are one identical
    # spike vector aligned with the request's weighted queries: they tie exactly and beat
    # every other key, so the top-2048 is the first 2048 spike positions of the request
    if f.spike_pos is None:
        pytest.skip("no planted spikes in this workload")
    _say(f"full planted spikes: all {f.T} rows")
    top = f.top.cpu().numpy()
    top_ref = f.top_ref.cpu().numpy()
    for t in range(f.T):
        exp = f.spike_pos[f.request(t)][:f.wl.topk].numpy()
        assert len(exp) == f.wl.topk
        assert np.array_equal(top[t], exp), f"row {t}"
        assert np.array_equal(top_ref[t], exp), f"row {t} (refined)"


def test_full_index_share_draft_rows(f):
    # one draft row per request gathers the step-0 top-k row of its accepted position;
    # step-0 sets are generated (not taken from the HIP top-k)
    w = f.wl
    if not w.share_steps:
        pytest.skip("no draft steps in this workload")
    _say(f"full index share: {w.batch} draft rows over {w.batch} x {w.ctx}")
    qo0 = f.qo
    step0 = synth.random_topk(w, f.lengths, qo0, w.topk)
    n_acc = synth.accepted_lengths(w)
    qo1 = torch.arange(w.batch + 1, dtype=torch.int32)
    m = synth.mla_inputs(w, f.lengths, device=DEV, rows=1, seed_offset=1)
    need = api.sparse_mla_workspace_size(w.batch, w.mla_heads, w.topk)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=DEV)
    d = lambda x: x.to(DEV)
    o_sh, l_sh = api.sparse_mla_decode(m["q"], m["kv"], d(step0), d(qo1), f.ko_d, 1, w.sm_scale,
                                       share_base=d(qo0), num_accepted=d(n_acc), workspace=ws)
    compact = step0[qo0[:-1].long() + n_acc.long()].contiguous()
    o_cp, l_cp = api.sparse_mla_decode(m["q"], m["kv"], d(compact), d(qo1), f.ko_d, 1, w.sm_scale,
                                       workspace=ws)
    assert torch.equal(o_sh, o_cp) and torch.equal(l_sh, l_cp)
    rows = sorted({0, 1, w.batch - 1} | set(np.random.default_rng(5).choice(w.batch, 5).tolist()))
    u16 = lambda x: x.view(torch.uint16).cpu().numpy()
    ref_o, ref_l = oracle.sparse_mla(u16(m["q"]), u16(m["kv"]), step0.numpy(), qo1.numpy(),
                                     f.ko.numpy(), w.sm_scale, rows=np.array(rows),
                                     share_base=qo0.numpy(), num_accepted=n_acc.numpy())
    sel = torch.tensor(rows, device=DEV)
    worst = mla_check(o_sh[sel], l_sh[sel], ref_o, ref_l)
    _say(f"  requests {rows} (accepted {n_acc[rows].tolist()}): worst err/bound = {worst:.3f}")
