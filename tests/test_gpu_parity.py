"""Parity of the HIP path (through the C ABI) against the CPU oracle, CPU-sized cases.

Bars: quantised codes/scales, top-k sets on shared fp32 scores, accepted lengths and
argmaxes are bit-exact; indexer scores lie within the bound derived from the FP8 MFMA
and float32 epilogue arithmetic; end-to-end top-k sets are equal or differ only inside
that bound around the k-th score; sparse MLA meets max|d| <= 2e-2*max|o| + 1e-2*|o|;
rejection-sampling acceptance equals the oracle wherever no decision or draw sits within
float rounding of its boundary, and is one of the oracle's nudged outcomes where one does.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from dsa_sparse_attention_amd import api, synth, workloads
from tests._pipeline import (DEV, Case, check_topk_valid, gpu_indexer, kth_largest, mla_check,
                             oracle_quant, refine_args, refine_eps, score_tolerance,
                             REFINE_MARGIN)

pytestmark = pytest.mark.gpu

W = workloads
SMALL = {
    "tiny": W.TINY,
    "decode_verify@4096": W.scaled(W.DECODE_VERIFY, ctx=4096, batch=3, topk=512),
    "mtp5_verify@6000": W.scaled(W.MTP5_VERIFY, ctx=6000, batch=3, topk=512),
    "long_ctx@12800": W.scaled(W.LONG_CTX, ctx=12800, batch=1, topk=64),
}


def _say(*a):
    print(*a, flush=True)


# ---------------------------------------------------------------- quantiser
@pytest.mark.parametrize("dim", [64, 128])
def test_quantize_bitexact(dim):
    _say(f"quantize dim={dim}")
    g = torch.Generator().manual_seed(dim)
    x = torch.randn((1027, dim), generator=g) * torch.rand((1027, 1), generator=g) * 100
    x[0] = 0.0                    # zero vector -> scale 1, codes 0
    x[1, :] = 1e-30               # underflow to subnormal / zero codes
    x[2, 5] = 3e4                 # one dominant element
    codes, scale = api.quantize_fp8(x.to(DEV))
    rc, rs = oracle.quantize(x.numpy())
    assert np.array_equal(codes.cpu().numpy(), rc)
    assert np.array_equal(scale.cpu().numpy(), rs)


@pytest.mark.parametrize("D,H,with_latent,with_q", [(128, 64, True, True), (64, 8, False, True),
                                                    (128, 16, True, False)])
def test_verify_cache_write_bitexact(D, H, with_latent, with_q):
    # the verify rows' keys land quantised (oracle codes and scales) in their cache rows,
    # their latent rows are copied, the queries are quantised, and no other row changes
    _say(f"verify_cache_write D={D} H={H} latent={with_latent} q={with_q}")
    rng = np.random.default_rng(D + H)
    N, T = 3000, 37
    dst = np.sort(rng.choice(N, T, replace=False)).astype(np.int64)
    rng.shuffle(dst)
    k_new = rng.standard_normal((T, D)).astype(np.float32)
    k_cache = rng.integers(0, 256, (N, D), dtype=np.uint8)
    k_scale = rng.random(N).astype(np.float32)
    d = lambda a: torch.from_numpy(a).to(DEV)
    kc_d, ks_d = d(k_cache), d(k_scale)
    lat = kv_d = None
    if with_latent:
        lat = torch.randn((T, 576), generator=synth.generator(5)).to(torch.bfloat16)
        kv = torch.randn((N, 576), generator=synth.generator(6)).to(torch.bfloat16)
        kv_d = kv.to(DEV)
    q = qc = qs = None
    if with_q:
        q = rng.standard_normal((T, H, D)).astype(np.float32)
    got_qc, got_qs = api.verify_cache_write(d(k_new), d(dst), kc_d, ks_d,
                                            latent_new=None if lat is None else lat.to(DEV),
                                            kv_cache=kv_d, q=None if q is None else d(q))
    codes, scales = oracle.quantize(k_new)
    want_c, want_s = k_cache.copy(), k_scale.copy()
    want_c[dst], want_s[dst] = codes, scales
    assert np.array_equal(kc_d.cpu().numpy(), want_c)
    assert np.array_equal(ks_d.cpu().numpy(), want_s)
    if with_latent:
        want_kv = kv.clone()
        want_kv[torch.from_numpy(dst)] = lat
        assert torch.equal(kv_d.cpu().view(torch.int16), want_kv.view(torch.int16))
    if with_q:
        qc, qs = oracle.quantize(q)
        assert np.array_equal(got_qc.cpu().numpy(), qc) and np.array_equal(got_qs.cpu().numpy(), qs)
    with pytest.raises(api.DsaError, match="UNSUPPORTED"):
        api.verify_cache_write(d(k_new[:, :32].copy()), d(dst), kc_d[:, :32].contiguous(), ks_d)


# ---------------------------------------------------------------- indexer score
@pytest.mark.parametrize("name", list(SMALL))
def test_index_score_within_bound(name):
    w = SMALL[name]
    _say(f"index_score {name}")
    case = Case(w, with_mla=False, with_accept=False)
    gi = gpu_indexer(case)
    qc, qs, kc, ks, ko = oracle_quant(case)
    assert np.array_equal(gi["qc"].cpu().numpy(), qc) and np.array_equal(gi["kc"].cpu().numpy(), kc)
    rows = np.arange(case.T)
    ref = oracle.index_score(qc, qs, case.host("w_f32"), kc, ks, case.qo.numpy(), ko,
                             rows=rows, width=case.max_kv)
    tol = score_tolerance(qc, qs, case.host("w_f32"), kc, ks, rows, case.qo.numpy(), ko,
                          case.max_kv)
    got = gi["scores"].cpu().numpy()[:, :case.max_kv].astype(np.float64)
    worst = 0.0
    for t in rows:
        n = case.visible(int(t))
        err = np.abs(got[t, :n] - ref[t, :n])
        assert np.all(err <= tol[t, :n]), f"row {t}: score error above bound"
        worst = max(worst, float((err / np.maximum(tol[t, :n], 1e-300)).max()))
    _say(f"  worst |err|/bound = {worst:.3e}")
    assert worst <= REFINE_MARGIN, "scores drift past the margin the default refine relies on"


def test_index_score_exact_grid_bitexact():
    # q_hat, k_hat integers in [-4, 4] (exact in e4m3fn), unit scales, w = m/16: every
    # partial sum is exact in any accumulator, so the HIP scores must equal the oracle's
    _say("index_score exact grid")
    rng = np.random.default_rng(11)
    T, H, D, L = 4, 64, 128, 3000
    vals = np.array([-4, -3, -2, -1, 0, 1, 2, 3, 4], np.float32)
    q = oracle.fp8_encode(rng.choice(vals, (T, H, D)))
    k = oracle.fp8_encode(rng.choice(vals, (L, D)))
    w = (rng.integers(0, 16, (T, H)) / 16).astype(np.float32)
    qs = np.ones((T, H), np.float32)
    ks = np.ones(L, np.float32)
    qo = np.array([0, T], np.int32)
    ko = np.array([0, L], np.int64)
    ref = oracle.index_score(q, qs, w, k, ks, qo, ko)
    d = lambda a: torch.from_numpy(a).to(DEV)
    got = api.index_score(d(q), d(qs), d(w), d(k), d(ks), d(qo), d(ko), T, L)
    got = got.cpu().numpy()[:, :L].astype(np.float64)
    for t in range(T):
        n = L - T + t + 1
        assert np.array_equal(got[t, :n], ref[t, :n])


@pytest.mark.parametrize("H,D,seed,signed", [(64, 128, 0, False), (128, 128, 1, False), (8, 64, 2, False),
                                              (1, 128, 3, True), (37, 128, 4, True), (100, 64, 5, True)])
def test_index_score_ragged_many_requests_exact_grid(H, D, seed, signed):
    # Many requests with ragged lengths (empty ones, a few keys, tile multiples) and a
    # varying number of rows (up to 9, so rows split into row groups): the key ranges of
    # the blocks cross request boundaries at arbitrary points. Integer codes keep every
    # sum exact, so every visible score must equal the oracle's, and every entry past a
    # row's visible prefix must keep its prefilled value. Head counts that fill no whole
    # 16-head tile (1, 37, 100) and head weights of either sign are covered too.
    _say(f"index_score ragged exact grid H={H} D={D} signed={signed}")
    rng = np.random.default_rng(100 + seed)
    B = 120
    lens = rng.integers(0, 300, B)
    lens[rng.choice(B, 12, replace=False)] = 0
    lens[rng.choice(B, 8, replace=False)] = 64 * rng.integers(1, 5, 8)
    R = rng.integers(1, 10, B)
    qo = np.concatenate([[0], np.cumsum(R)]).astype(np.int32)
    ko = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T, N, L = int(qo[-1]), int(ko[-1]), int(lens.max())
    vals = np.array([-4, -3, -2, -1, 0, 1, 2, 3, 4], np.float32)
    q = oracle.fp8_encode(rng.choice(vals, (T, H, D)))
    k = oracle.fp8_encode(rng.choice(vals, (N, D)))
    w = (rng.integers(-16 if signed else 0, 16, (T, H)) / 16).astype(np.float32)
    qs = np.ones((T, H), np.float32)
    ks = np.ones(N, np.float32)
    ref = oracle.index_score(q, qs, w, k, ks, qo, ko, width=L)
    d = lambda a: torch.from_numpy(a).to(DEV)
    ld = (L + 3) // 4 * 4
    scores = torch.full((T, ld), float("nan"), device=DEV)
    api.index_score(d(q), d(qs), d(w), d(k), d(ks), d(qo), d(ko), int(R.max()), L, scores=scores)
    got = scores.cpu().numpy().astype(np.float64)
    for t in range(T):
        n = oracle.row_visible(qo, ko, t)
        assert np.array_equal(got[t, :n], ref[t, :n]), f"row {t} (visible {n})"
        assert np.all(np.isnan(got[t, n:])), f"row {t}: written past its visible prefix"


# ---------------------------------------------------------------- top-k
@pytest.mark.parametrize("levels", [0, 5, 1000])
def test_topk_bitexact_on_shared_scores(levels):
    _say(f"topk levels={levels}")
    lens = [5000, 130, 2049, 4099]
    R = 3
    qo = torch.tensor([0, 3, 6, 9, 12], dtype=torch.int32)
    ko = synth.kv_row_offsets(lens)
    ld = 5000 + 4 - 5000 % 4
    s = synth.random_scores(12, ld, seed=levels, tie_levels=levels)
    s[0, :50] = 0.0
    s[0, 50:100] = -0.0                # -0 ties +0
    k = 2048
    got = api.topk(s.to(DEV), qo.to(DEV), ko.to(DEV), R, max(lens), k).cpu().numpy()
    for t in range(12):
        n = oracle.row_visible(qo.numpy(), ko.numpy(), t)
        ref = oracle.topk(s[t:t + 1].double().numpy(), [n], k)[0]
        assert np.array_equal(got[t], ref), f"row {t} (visible {n})"


@pytest.mark.parametrize("levels", [0, 3, 600])
def test_topk_long_rows_chunked(levels):
    # rows above 65536 positions are selected per 65536-position chunk and merged: boundary
    # lengths (a one-key last chunk, exact multiples), a short row in the same grid, ties
    _say(f"topk long rows levels={levels}")
    lens = [65537, 131072, 200003, 3000]
    R = 2
    qo = torch.tensor([0, 2, 4, 6, 8], dtype=torch.int32)
    ko = synth.kv_row_offsets(lens)
    ld = 200004
    s = synth.random_scores(8, ld, seed=50 + levels, tie_levels=levels)
    for k in (7, 2048):
        ws = torch.zeros(max(api.topk_workspace_size(4, 8, max(lens), k), 16), dtype=torch.uint8,
                         device=DEV)
        got = api.topk(s.to(DEV), qo.to(DEV), ko.to(DEV), R, max(lens), k,
                       workspace=ws).cpu().numpy()
        for t in range(8):
            n = oracle.row_visible(qo.numpy(), ko.numpy(), t)
            ref = oracle.topk(s[t:t + 1].double().numpy(), [n], k)[0]
            assert np.array_equal(got[t], ref), f"k={k} row {t} (visible {n})"


@pytest.mark.parametrize("ctx,batch,rows,topk", [(100000, 2, 3, 2048), (100000, 2, 3, 512),
                                                  (300000, 1, 2, 512)])
def test_refined_topk_long_rows(ctx, batch, rows, topk):
    # Rows above 65536 positions: the chunked float32 selection, then the refine. Up to 2^18
    # positions the band is classified and rescored over many blocks and ranked by a radix
    # select; longer rows refine in one block. 1% identical spike keys per request: with
    # top-k 2048 they are all kept above a small band, with 512 every spike ties in the band
    # (1000 and 3000 keys) and the lowest positions must win. Every row against the oracle.
    _say(f"refined top-k long rows ctx={ctx} topk={topk}")
    w = W.replace(W.scaled(W.LONG_CTX, ctx=ctx, batch=batch, topk=topk), rows=rows)
    case = Case(w, with_mla=False, with_accept=False)
    gi = gpu_indexer(case)
    qc, qs, kc, ks, ko = oracle_quant(case)
    rows_all = np.arange(case.T)
    ref_s = oracle.index_score(qc, qs, case.host("w_f32"), kc, ks, case.qo.numpy(), ko,
                               rows=rows_all, width=case.max_kv)
    nvis = np.array([case.visible(int(t)) for t in rows_all])
    assert nvis.min() > 65536
    ref_k = oracle.topk(ref_s, nvis, w.topk)
    ra = refine_args(gi, case)
    ws = torch.zeros(api.topk_workspace_size(w.batch, case.T, case.max_kv, w.topk, True),
                     dtype=torch.uint8, device=DEV)
    for call in range(2):  # the workspace is reused as it comes
        got = api.topk(gi["scores"], case.qo_d, case.ko_d, w.rows, case.max_kv, w.topk,
                       refine=ra, workspace=ws)
        st = ra["status"].cpu().numpy()
        _say(f"  call {call}: band sizes {st.tolist()}")
        assert st.min() >= 0
        assert np.array_equal(got.cpu().numpy(), ref_k)
    if topk < len(case.spike_pos[0]):
        for t in rows_all:  # every spike ties: the lowest spike positions
            b = int(t) // w.rows
            assert list(got[t].cpu().numpy()) == list(case.spike_pos[b][:w.topk].numpy())


def test_refined_topk_long_rows_band_overflow():
    # 5% identical spike keys in 100K-position rows: every row's band holds 5000 exact ties,
    # more than the refine rescores (4096). The row reports -1 and keeps the float32
    # selection, which ties resolve by position just as the exact order does.
    _say("refined top-k long rows, band overflow")
    w = W.replace(W.scaled(W.LONG_CTX, ctx=100000, batch=1, topk=512), rows=2, spike_frac=0.05)
    case = Case(w, with_mla=False, with_accept=False)
    gi = gpu_indexer(case)
    ra = refine_args(gi, case)
    got = api.topk(gi["scores"], case.qo_d, case.ko_d, w.rows, case.max_kv, w.topk, refine=ra)
    assert ra["status"].cpu().tolist() == [-1, -1]
    assert torch.equal(got, gi["topk"])
    for t in range(case.T):
        assert list(got[t].cpu().numpy()) == list(case.spike_pos[0][:w.topk].numpy())


@pytest.mark.parametrize("cluster", [2500, 600, 0])
def test_topk_identical_clusters_across_row_lengths(cluster):
    # Rows at each register-path size class (up to 8192, 16384 and 65536 positions, with
    # the boundaries) carry a cluster of identical keys far above the rest: more copies
    # than k (theta is the cluster value), fewer (theta lies far below it), or none. A
    # second, smaller cluster sits between the first and the bulk in every other row.
    _say(f"topk clusters={cluster}")
    lens = [3000, 8192, 8193, 16384, 16385, 40000, 65536]
    B = len(lens)
    qo = torch.arange(B + 1, dtype=torch.int32)
    ko = synth.kv_row_offsets(lens)
    ld = 65536
    s = synth.random_scores(B, ld, seed=70 + cluster)
    g = synth.generator(71 + cluster)
    for t, n in enumerate(lens):
        if cluster:
            pos = torch.randperm(n, generator=g)[:min(cluster, n // 2)]
            s[t, pos] = 3.0e7
        if t % 2:
            pos = torch.randperm(n, generator=g)[:300]
            s[t, pos] = 2.5e4
    for k in (64, 2048):
        got = api.topk(s.to(DEV), qo.to(DEV), ko.to(DEV), 1, max(lens), k).cpu().numpy()
        for t in range(B):
            ref = oracle.topk(s[t:t + 1].double().numpy(), [lens[t]], k)[0]
            assert np.array_equal(got[t], ref), f"k={k} row {t} (visible {lens[t]})"


def test_topk_small_k_and_padding():
    _say("topk k=1 and padding")
    lens = [10, 1, 300]
    qo = torch.tensor([0, 1, 2, 3], dtype=torch.int32)
    ko = synth.kv_row_offsets(lens)
    s = synth.random_scores(3, 300, seed=3, tie_levels=3)
    for k in (1, 7, 300, 301):
        got = api.topk(s.to(DEV), qo.to(DEV), ko.to(DEV), 1, 300, k).cpu().numpy()
        for t in range(3):
            ref = oracle.topk(s[t:t + 1].double().numpy(), [lens[t]], k)[0]
            assert np.array_equal(got[t], ref), (k, t)


def test_requests_without_keys_or_rows():
    # Requests with no keys, a request with no rows, and rows placed before their request's
    # first key (more rows than keys), beside ordinary requests: a row that sees no key
    # selects nothing (all -1) and attends to nothing (out 0, lse -inf); every row equals
    # the oracle's.
    _say("requests without keys or rows")
    lens, rows = [0, 300, 0, 40, 3], [2, 3, 0, 1, 5]
    qo, ko = synth.prefix(rows, torch.int32), synth.kv_row_offsets(lens)
    T, k, heads, sm = sum(rows), 64, 16, 0.0417
    nvis = np.array([max(0, min(L, L - R + r + 1)) for L, R in zip(lens, rows) for r in range(R)])
    s = synth.random_scores(T, 300, seed=9, tie_levels=3)
    top = api.topk(s.to(DEV), qo.to(DEV), ko.to(DEV), max(rows), max(lens), k).cpu().numpy()
    ref = np.asarray(oracle.topk(s.double().numpy(), nvis, k), dtype=np.int32)
    assert np.array_equal(top, ref)
    assert np.all(top[nvis == 0] == -1) and np.any(nvis == 0)
    g = synth.generator(10)
    q = torch.randn((T, heads, 576), generator=g).to(torch.bfloat16)
    kv = torch.randn((sum(lens), 576), generator=g).to(torch.bfloat16)
    out, lse = api.sparse_mla_decode(q.to(DEV), kv.to(DEV), torch.from_numpy(ref).to(DEV),
                                     qo.to(DEV), ko.to(DEV), max(rows), sm)
    u16 = lambda x: x.view(torch.uint16).numpy()
    ref_o, ref_l = oracle.sparse_mla(u16(q), u16(kv), ref, qo.numpy(), ko.numpy(), sm)
    mla_check(out, lse, ref_o, ref_l)
    empty = torch.from_numpy(nvis == 0).to(DEV)
    assert torch.all(out[empty] == 0) and torch.all(torch.isneginf(lse[empty]))


@pytest.mark.parametrize("name", list(SMALL))
def test_end_to_end_topk_sets(name):
    w = SMALL[name]
    _say(f"end-to-end top-k {name}")
    case = Case(w, with_mla=False, with_accept=False)
    gi = gpu_indexer(case)
    qc, qs, kc, ks, ko = oracle_quant(case)
    rows = np.arange(case.T)
    ref_s = oracle.index_score(qc, qs, case.host("w_f32"), kc, ks, case.qo.numpy(), ko,
                               rows=rows, width=case.max_kv)
    nvis = np.array([case.visible(int(t)) for t in rows])
    ref_k = oracle.topk(ref_s, nvis, w.topk)
    tol = score_tolerance(qc, qs, case.host("w_f32"), kc, ks, rows, case.qo.numpy(), ko,
                          case.max_kv)
    ndiff = check_topk_valid(gi["topk"].cpu().numpy(), ref_k, ref_s, nvis, tol, w.topk)
    _say(f"  rows with band-only differences: {ndiff}/{len(rows)}")
    if w.spike_frac:
        for t in rows:  # planted spikes: closed-form answer, decided purely by position
            assert list(gi["topk"][t].cpu().numpy()) == list(case.spike_pos[0][:w.topk].numpy())


@pytest.mark.parametrize("name", list(SMALL))
def test_end_to_end_topk_refined_equals_oracle(name):
    # exact-boundary refine: the HIP set must equal the oracle's set on every row, and the
    # float32 scores must sit within half of the refine's error bound (its constant is
    # validated by this measurement, not derived)
    w = SMALL[name]
    _say(f"end-to-end refined top-k {name}")
    case = Case(w, with_mla=False, with_accept=False)
    gi = gpu_indexer(case)
    qc, qs, kc, ks, ko = oracle_quant(case)
    rows = np.arange(case.T)
    ref_s = oracle.index_score(qc, qs, case.host("w_f32"), kc, ks, case.qo.numpy(), ko,
                               rows=rows, width=case.max_kv)
    nvis = np.array([case.visible(int(t)) for t in rows])
    ref_k = oracle.topk(ref_s, nvis, w.topk)
    got_s = gi["scores"].cpu().numpy()[:, :case.max_kv].astype(np.float64)
    eps = refine_eps(qc, qs, case.host("w_f32"), ks, case.qo.numpy(), ko, rows,
                     kth_largest(got_s, nvis, w.topk))
    ratio = max(float(np.abs(got_s[t, :nvis[t]] - ref_s[t, :nvis[t]]).max() / eps[t])
                for t in rows if nvis[t])
    _say(f"  max |I_f32 - I_exact| / eps = {ratio:.3f}")
    assert ratio <= 0.5
    ra = refine_args(gi, case)
    got = api.topk(gi["scores"], case.qo_d, case.ko_d, w.rows, case.max_kv, w.topk, refine=ra)
    st = ra["status"].cpu().numpy()
    _say(f"  band sizes: max {st.max()}, mean {st.mean():.1f}")
    assert st.min() >= 0
    assert np.array_equal(got.cpu().numpy(), ref_k)


@pytest.mark.parametrize("ctx", [2050, 8195, 16387, 65539])
def test_refined_topk_row_lengths_at_path_boundaries(ctx):
    # six verify rows of one request see ctx - 5 .. ctx keys. With k = 2048 at ctx 2050 they
    # cross n < k (every visible key), n = k and n = k + 1; the other sizes straddle the
    # register path's 8, 16 and 64 scores per lane (8192 and 16384 positions) and its end
    # at 65536 (past it, the LDS selection and the generic refine). Every row's refined set
    # must be the oracle's.
    w = W.replace(W.scaled(W.MTP5_VERIFY, ctx=ctx, batch=1, topk=2048), ctx_min=0)
    _say(f"refined top-k at row lengths {ctx - 5}..{ctx}")
    case = Case(w, with_mla=False, with_accept=False)
    gi = gpu_indexer(case)
    qc, qs, kc, ks, ko = oracle_quant(case)
    rows = np.arange(case.T)
    ref_s = oracle.index_score(qc, qs, case.host("w_f32"), kc, ks, case.qo.numpy(), ko,
                               rows=rows, width=case.max_kv)
    nvis = np.array([case.visible(int(t)) for t in rows])
    assert list(nvis) == list(range(ctx - 5, ctx + 1))
    ref_k = oracle.topk(ref_s, nvis, w.topk)
    ra = refine_args(gi, case)
    got = api.topk(gi["scores"], case.qo_d, case.ko_d, w.rows, case.max_kv, w.topk, refine=ra)
    st = ra["status"].cpu().numpy()
    _say(f"  status per row: {list(st)}")
    assert st.min() >= 0
    assert np.array_equal(got.cpu().numpy(), ref_k)


@pytest.mark.parametrize("ctx", [5000, 20000])
def test_refined_topk_largest_k(ctx):
    # k = 4096, the largest the refine takes, through the separate and the fused path; at
    # 20000 positions the register path's per-wave candidate regions overflow, so the rows
    # take the LDS selection and the generic refine
    k = 4096
    w = W.replace(W.scaled(W.MTP5_VERIFY, ctx=ctx, batch=1, topk=k), ctx_min=0)
    _say(f"refined top-k k={k} at row lengths {ctx - 5}..{ctx}")
    case = Case(w, with_mla=False, with_accept=False)
    gi = gpu_indexer(case)
    qc, qs, kc, ks, ko = oracle_quant(case)
    rows = np.arange(case.T)
    ref_s = oracle.index_score(qc, qs, case.host("w_f32"), kc, ks, case.qo.numpy(), ko,
                               rows=rows, width=case.max_kv)
    nvis = np.array([case.visible(int(t)) for t in rows])
    ref_k = oracle.topk(ref_s, nvis, k)
    ra = refine_args(gi, case)
    got = api.topk(gi["scores"], case.qo_d, case.ko_d, w.rows, case.max_kv, k, refine=ra)
    st = ra["status"].cpu().numpy()
    _say(f"  separate: status {list(st)}")
    assert st.min() >= 0
    assert np.array_equal(got.cpu().numpy(), ref_k)
    fst = torch.full((case.T,), -9, dtype=torch.int32, device=DEV)
    fused = api.index_topk(gi["qc"], gi["qs"], case.w_f32, gi["kc"], gi["ks"], case.qo_d,
                           case.ko_d, w.rows, case.max_kv, k, status=fst)
    _say(f"  fused: status {list(fst.cpu().numpy())}")
    assert int(fst.min()) >= 0
    assert np.array_equal(fused.cpu().numpy(), ref_k)


def test_topk_largest_k_unrefined():
    # k = 8192, the largest dsa_topk takes without the refine, on shared scores with ties:
    # rows just below, at and past 8192 positions, a register-path row and a chunked row
    _say("topk k=8192")
    lens = [8190, 8192, 8193, 30000, 100000]
    qo = torch.arange(len(lens) + 1, dtype=torch.int32)
    ko = synth.kv_row_offsets(lens)
    s = synth.random_scores(len(lens), max(lens), seed=21, tie_levels=50)
    got = api.topk(s.to(DEV), qo.to(DEV), ko.to(DEV), 1, max(lens), 8192).cpu().numpy()
    ref = oracle.topk(s.double().numpy(), lens, 8192)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("name", list(SMALL))
def test_end_to_end_topk_refined_signed_weights(name):
    # head weights of either sign (w -> 2w - 1, so about half are negative): the scorer's
    # weighted ReLU sum and the refine's bound (which takes |w_j q_scale_j|) must still give
    # the oracle's exact sets
    w = SMALL[name]
    _say(f"end-to-end refined top-k, signed weights {name}")
    case = Case(w, with_mla=False, with_accept=False)
    case.w_f32 = 2.0 * case.w_f32 - 1.0
    assert bool((case.w_f32 < 0).any()) and bool((case.w_f32 > 0).any())
    gi = gpu_indexer(case)
    qc, qs, kc, ks, ko = oracle_quant(case)
    rows = np.arange(case.T)
    ref_s = oracle.index_score(qc, qs, case.host("w_f32"), kc, ks, case.qo.numpy(), ko,
                               rows=rows, width=case.max_kv)
    nvis = np.array([case.visible(int(t)) for t in rows])
    ref_k = oracle.topk(ref_s, nvis, w.topk)
    got_s = gi["scores"].cpu().numpy()[:, :case.max_kv].astype(np.float64)
    eps = refine_eps(qc, qs, case.host("w_f32"), ks, case.qo.numpy(), ko, rows,
                     kth_largest(got_s, nvis, w.topk))
    ratio = max(float(np.abs(got_s[t, :nvis[t]] - ref_s[t, :nvis[t]]).max() / eps[t])
                for t in rows if nvis[t])
    _say(f"  max |I_f32 - I_exact| / eps = {ratio:.3f}")
    assert ratio <= 0.5
    ra = refine_args(gi, case)
    got = api.topk(gi["scores"], case.qo_d, case.ko_d, w.rows, case.max_kv, w.topk, refine=ra)
    st = ra["status"].cpu().numpy()
    _say(f"  band sizes: max {st.max()}, mean {st.mean():.1f}")
    assert st.min() >= 0
    assert np.array_equal(got.cpu().numpy(), ref_k)


def test_topk_refine_rejects_bad_arguments():
    _say("topk refine error paths")
    s = torch.zeros((2, 64), device=DEV)
    qo = torch.tensor([0, 2], dtype=torch.int32, device=DEV)
    ko = torch.tensor([0, 64], dtype=torch.int64, device=DEV)
    ra = dict(q_fp8=torch.zeros((2, 8, 96), dtype=torch.uint8, device=DEV),
              q_scale=torch.ones((2, 8), device=DEV), w=torch.ones((2, 8), device=DEV),
              k_fp8=torch.zeros((64, 96), dtype=torch.uint8, device=DEV),
              k_scale=torch.ones(64, device=DEV))
    with pytest.raises(api.DsaError, match="INVALID_ARGUMENT"):
        api.topk(s, qo, ko, 2, 64, 8, refine=ra)          # D_I = 96
    ra["q_fp8"] = torch.zeros((2, 8, 64), dtype=torch.uint8, device=DEV)
    ra["k_fp8"] = torch.zeros((64, 64), dtype=torch.uint8, device=DEV)
    with pytest.raises(api.DsaError, match="INVALID_ARGUMENT"):
        api.topk(s, qo, ko, 2, 64, 4097, refine=ra)       # k above the refine's limit


def _chunk_max(ks: np.ndarray) -> np.ndarray:
    """Largest scale of every 2048 consecutive rows (the last chunk ragged)."""
    n = len(ks)
    return np.array([np.abs(ks[c:c + 2048]).max() for c in range(0, n, 2048)], np.float32)


def test_key_scale_table_build_range_and_cache_write():
    # the table's entries are the chunk maxima; a range rebuild recomputes only the chunks it
    # meets; a cache write with the table raises each chunk's entry to the new rows' scales
    _say("key-scale table")
    rng = np.random.default_rng(7)
    N = 3 * 2048 + 777
    ks = (np.abs(rng.standard_normal(N)) * 0.01 + 1e-3).astype(np.float32)
    ks_d = torch.from_numpy(ks).to(DEV)
    tab = api.key_scale_max(ks_d)
    assert np.array_equal(tab.cpu().numpy(), _chunk_max(ks))
    ks[4100:4110] = 5.0
    ks_d[4100:4110] = 5.0
    before = tab.cpu().numpy()
    api.key_scale_max(ks_d, out=tab, row_begin=4100, row_end=4110)
    after = tab.cpu().numpy()
    assert after[2] == 5.0 and np.array_equal(np.delete(after, 2), np.delete(before, 2))
    assert np.array_equal(after, _chunk_max(ks))
    # the verify rows' keys: some far larger than any cached key, some smaller
    T = 37
    dst = rng.choice(N, T, replace=False).astype(np.int64)
    k_new = rng.standard_normal((T, 128)).astype(np.float32)
    k_new[::3] *= 1000.0
    kc_d = torch.zeros((N, 128), dtype=torch.uint8, device=DEV)
    api.verify_cache_write(torch.from_numpy(k_new).to(DEV), torch.from_numpy(dst).to(DEV), kc_d,
                           ks_d, k_scale_max=tab)
    _, new_s = oracle.quantize(k_new)
    want = after.copy()
    for d, sc in zip(dst, new_s):
        want[d // 2048] = max(want[d // 2048], sc)
    got = tab.cpu().numpy()
    assert np.array_equal(got, want)
    assert (got > after).any()  # the scaled-up keys raised some entries
    assert np.array_equal(ks_d.cpu().numpy()[dst], new_s)
    with pytest.raises(api.DsaError, match="INVALID_ARGUMENT"):
        api.key_scale_max(ks_d, out=tab, row_begin=10, row_end=N + 1)


@pytest.mark.parametrize("name", ["mtp5_verify@6000", "decode_verify@4096", "long100k"])
def test_refined_topk_with_key_scale_table(name):
    # smax_t from the caller's table (global 2048-row chunks, which straddle the requests'
    # boundaries here, so it can only exceed the per-request maxima): every row is refined
    # and its set equals the oracle's, as with the pre-pass
    _say(f"refined top-k with the key-scale table, {name}")
    if name == "long100k":
        w = W.replace(W.scaled(W.LONG_CTX, ctx=100000, batch=2, topk=512), rows=3)
    else:
        w = SMALL[name]
    case = Case(w, with_mla=False, with_accept=False)
    gi = gpu_indexer(case)
    qc, qs, kc, ks, ko = oracle_quant(case)
    rows = np.arange(case.T)
    ref_s = oracle.index_score(qc, qs, case.host("w_f32"), kc, ks, case.qo.numpy(), ko,
                               rows=rows, width=case.max_kv)
    nvis = np.array([case.visible(int(t)) for t in rows])
    ref_k = oracle.topk(ref_s, nvis, w.topk)
    ra = refine_args(gi, case)
    ra["k_scale_max"] = api.key_scale_max(gi["ks"])
    assert np.array_equal(ra["k_scale_max"].cpu().numpy(), _chunk_max(gi["ks"].cpu().numpy()))
    got = api.topk(gi["scores"], case.qo_d, case.ko_d, w.rows, case.max_kv, w.topk, refine=ra)
    st = ra["status"].cpu().numpy()
    _say(f"  band sizes: max {st.max()}, mean {st.mean():.1f}")
    assert st.min() >= 0
    assert np.array_equal(got.cpu().numpy(), ref_k)


def test_refined_topk_short_key_scale_table_keeps_float32():
    # a table that ends before a row's cache rows gives that row an infinite eps: status -2
    # and the float32 selection
    _say("refined top-k, key-scale table too short")
    w = SMALL["mtp5_verify@6000"]
    case = Case(w, with_mla=False, with_accept=False)
    gi = gpu_indexer(case)
    ra = refine_args(gi, case)
    ra["k_scale_max"] = api.key_scale_max(gi["ks"])[:1].contiguous()
    got = api.topk(gi["scores"], case.qo_d, case.ko_d, w.rows, case.max_kv, w.topk, refine=ra)
    assert ra["status"].cpu().tolist() == [-2] * case.T
    assert torch.equal(got, gi["topk"])


# ---------------------------------------------------------------- sparse MLA
@pytest.mark.parametrize("heads,pad", [(16, 0.0), (64, 0.1), (128, 0.0), (48, 0.5), (80, 0.1),
                                       (112, 0.0)])
def test_sparse_mla_matches_oracle(heads, pad):
    _say(f"sparse_mla heads={heads} pad={pad}")
    w = W.replace(W.scaled(W.MTP5_VERIFY, ctx=3000, batch=3, topk=512), mla_heads=heads)
    lens = synth.context_lengths(w)
    qo, ko = synth.q_row_offsets(w), synth.kv_row_offsets(lens)
    m = synth.mla_inputs(w, lens)
    idx = synth.random_topk(w, lens, qo, w.topk, pad_frac=pad)
    idx[1, :] = -1                     # a row with nothing selected
    idx[2, 5] = 10 ** 6                # out-of-range entry is skipped
    out, lse = api.sparse_mla_decode(m["q"].to(DEV), m["kv"].to(DEV), idx.to(DEV), qo.to(DEV),
                                     ko.to(DEV), w.rows, w.sm_scale)
    u16 = lambda x: x.view(torch.uint16).numpy()
    ref_o, ref_l = oracle.sparse_mla(u16(m["q"]), u16(m["kv"]), idx.numpy(), qo.numpy(),
                                     ko.numpy(), w.sm_scale)
    worst = mla_check(out, lse, ref_o, ref_l)
    assert torch.all(out[1] == 0) and torch.all(torch.isneginf(lse[1]))
    _say(f"  worst err/bound = {worst:.3f}")


@pytest.mark.parametrize("where", [0, 300])
def test_sparse_mla_extreme_logit_spread(where):
    # Every row's list holds, at list position `where`, a key whose logit lies about 185
    # above the others in base 2 (its rope aligned with a shift of the queries' rope), and seven
    # places later one as far below: the other keys' weights fall below 2^-126 of the
    # dominant one, where the kernel's exponential flushes to zero. At position 300 the
    # dominant key arrives after nine chunks, so the reference max jumps and the earlier
    # accumulators are rescaled by a factor below 2^-126. The output dims carry no spike, so
    # the tolerance stays at the scale of ordinary values. Both latent caches.
    _say(f"sparse_mla extreme logit spread at list position {where}")
    w = W.replace(W.scaled(W.MTP5_VERIFY, ctx=3000, batch=2, topk=512), mla_heads=16)
    lens = synth.context_lengths(w)
    qo, ko = synth.q_row_offsets(w), synth.kv_row_offsets(lens)
    m = synth.mla_inputs(w, lens)
    idx = synth.random_topk(w, lens, qo, w.topk, pad_frac=0.0)
    q = m["q"].float()
    kv = m["kv"].float()
    q[:, :, 512:] += 4.0
    T = int(qo[-1])
    for t in range(T):
        b = int(np.searchsorted(qo.numpy(), t, side="right") - 1)
        kv[int(ko[b]) + int(idx[t, where]), 512:] = 12.0
        kv[int(ko[b]) + int(idx[t, where + 7]), 512:] = -12.0
    q, kv = q.to(torch.bfloat16), kv.to(torch.bfloat16)
    u16 = lambda x: x.view(torch.uint16).numpy()
    ref_o, ref_l = oracle.sparse_mla(u16(q), u16(kv), idx.numpy(), qo.numpy(), ko.numpy(),
                                     w.sm_scale)
    assert np.all(ref_l > 100.0), "the spike must dominate every row by more than 126 in base 2"
    out, lse = api.sparse_mla_decode(q.to(DEV), kv.to(DEV), idx.to(DEV), qo.to(DEV), ko.to(DEV),
                                     w.rows, w.sm_scale)
    _say(f"  bf16 rows: worst err/bound = {mla_check(out, lse, ref_o, ref_l):.3f}")
    kv8 = oracle.mla_fp8_pack(u16(kv))
    ref8_o, ref8_l = oracle.sparse_mla_fp8(u16(q), kv8, idx.numpy(), qo.numpy(), ko.numpy(),
                                           w.sm_scale)
    out8, lse8 = api.sparse_mla_decode_fp8(q.to(DEV), torch.from_numpy(kv8).to(DEV), idx.to(DEV),
                                           qo.to(DEV), ko.to(DEV), w.rows, w.sm_scale)
    _say(f"  FP8 rows: worst err/bound = {mla_check(out8, lse8, ref8_o, ref8_l):.3f}")


def test_sparse_mla_index_share_equals_compacted_copy():
    _say("sparse_mla index share")
    w = W.replace(W.scaled(W.DRAFT_SHARE, ctx=3000, batch=5, topk=256), rows=6)
    lens = synth.context_lengths(w)
    qo0, ko = synth.q_row_offsets(w), synth.kv_row_offsets(lens)
    step0 = synth.random_topk(w, lens, qo0, w.topk, pad_frac=0.05)
    n_acc = synth.accepted_lengths(w)
    qo1 = torch.arange(w.batch + 1, dtype=torch.int32)
    m = synth.mla_inputs(w, lens, rows=1, seed_offset=1)
    d = lambda x: x.to(DEV)
    o_sh, l_sh = api.sparse_mla_decode(d(m["q"]), d(m["kv"]), d(step0), d(qo1), d(ko), 1, w.sm_scale,
                                       share_base=d(qo0), num_accepted=d(n_acc))
    compact = step0[qo0[:-1].long() + n_acc.long()].contiguous()
    o_cp, l_cp = api.sparse_mla_decode(d(m["q"]), d(m["kv"]), d(compact), d(qo1), d(ko), 1, w.sm_scale)
    assert torch.equal(o_sh, o_cp) and torch.equal(l_sh, l_cp)
    u16 = lambda x: x.view(torch.uint16).numpy()
    ref_o, ref_l = oracle.sparse_mla(u16(m["q"]), u16(m["kv"]), step0.numpy(), qo1.numpy(), ko.numpy(),
                                     w.sm_scale, share_base=qo0.numpy(), num_accepted=n_acc.numpy())
    mla_check(o_sh, l_sh, ref_o, ref_l)


def test_sparse_mla_index_share_edges():
    # share map edges: a request with no accepted draft (its bonus row's list), one that
    # accepted every draft (its last verify row's list), and one whose map entry points past
    # the top-k rows (it selects nothing: out 0, lse -inf)
    _say("sparse_mla index share edges")
    w = W.replace(W.scaled(W.DRAFT_SHARE, ctx=3000, batch=5, topk=256), rows=6)
    lens = synth.context_lengths(w)
    qo0, ko = synth.q_row_offsets(w), synth.kv_row_offsets(lens)
    step0 = synth.random_topk(w, lens, qo0, w.topk, pad_frac=0.05)
    n_acc = synth.accepted_lengths(w).clone()
    n_acc[0], n_acc[1], n_acc[4] = 0, w.rows - 1, 10 ** 6
    qo1 = torch.arange(w.batch + 1, dtype=torch.int32)
    m = synth.mla_inputs(w, lens, rows=1, seed_offset=2)
    d = lambda x: x.to(DEV)
    out, lse = api.sparse_mla_decode(d(m["q"]), d(m["kv"]), d(step0), d(qo1), d(ko), 1, w.sm_scale,
                                     share_base=d(qo0), num_accepted=d(n_acc))
    assert torch.all(out[4] == 0) and torch.all(torch.isneginf(lse[4]))
    ok = n_acc.clone()
    ok[4] = 0  # the oracle is asked only about the requests with a valid map entry
    u16 = lambda x: x.view(torch.uint16).numpy()
    ref_o, ref_l = oracle.sparse_mla(u16(m["q"]), u16(m["kv"]), step0.numpy(), qo1.numpy(), ko.numpy(),
                                     w.sm_scale, share_base=qo0.numpy(), num_accepted=ok.numpy())
    mla_check(out[:4], lse[:4], ref_o[:4], ref_l[:4])


@pytest.mark.parametrize("heads", [64, 128])
def test_sparse_mla_many_rows_split_lists_and_workspace_reuse(heads):
    # 200 rows with k = 448 (ragged contexts, 20% padding): lists split over blocks whose
    # partial results are merged; a second call on the same workspace gives the same bits.
    _say(f"sparse_mla many rows heads={heads}")
    w = W.replace(W.scaled(W.MTP5_VERIFY, ctx=1200, batch=40, topk=448), rows=5, mla_heads=heads)
    lens = synth.context_lengths(w)
    qo, ko = synth.q_row_offsets(w), synth.kv_row_offsets(lens)
    m = synth.mla_inputs(w, lens)
    idx = synth.random_topk(w, lens, qo, w.topk, pad_frac=0.2)
    idx[7, :] = -1
    T = int(qo[-1])
    need = api.sparse_mla_workspace_size(T, heads, w.topk)
    ws = torch.zeros(max(need, 16), dtype=torch.uint8, device=DEV)
    u16 = lambda x: x.view(torch.uint16).numpy()
    ref_o, ref_l = oracle.sparse_mla(u16(m["q"]), u16(m["kv"]), idx.numpy(), qo.numpy(),
                                     ko.numpy(), w.sm_scale)
    outs = []
    for call in range(2):
        out, lse = api.sparse_mla_decode(m["q"].to(DEV), m["kv"].to(DEV), idx.to(DEV), qo.to(DEV),
                                         ko.to(DEV), w.rows, w.sm_scale, workspace=ws)
        _say(f"  call {call}: worst err/bound = {mla_check(out, lse, ref_o, ref_l):.3f}")
        outs.append((out.clone(), lse.clone()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("k", [1, 31, 33, 300, 2047])
def test_sparse_mla_list_lengths_off_the_chunk_grid(k):
    # top-k lists whose length is not a multiple of the 32-row chunk (one key, one short of
    # and one past a chunk, and a list that the small grid cuts into slices with a ragged
    # last chunk), on bf16 and FP8 rows
    _say(f"sparse_mla list length k={k}")
    w = W.replace(W.scaled(W.MTP5_VERIFY, ctx=3000, batch=2, topk=k), rows=3, mla_heads=64)
    lens = synth.context_lengths(w)
    qo, ko = synth.q_row_offsets(w), synth.kv_row_offsets(lens)
    m = synth.mla_inputs(w, lens)
    idx = synth.random_topk(w, lens, qo, k, pad_frac=0.1 if k > 1 else 0.0)
    d = lambda x: (torch.from_numpy(x) if isinstance(x, np.ndarray) else x).to(DEV)
    u16 = lambda x: x.view(torch.uint16).numpy()
    out, lse = api.sparse_mla_decode(d(m["q"]), d(m["kv"]), d(idx), d(qo), d(ko), w.rows, w.sm_scale)
    ref_o, ref_l = oracle.sparse_mla(u16(m["q"]), u16(m["kv"]), idx.numpy(), qo.numpy(), ko.numpy(),
                                     w.sm_scale)
    _say(f"  bf16 rows: worst err/bound = {mla_check(out, lse, ref_o, ref_l):.3f}")
    kv8 = oracle.mla_fp8_pack(u16(m["kv"]))
    out8, lse8 = api.sparse_mla_decode_fp8(d(m["q"]), d(kv8), d(idx), d(qo), d(ko), w.rows, w.sm_scale)
    ref_o8, ref_l8 = oracle.sparse_mla_fp8(u16(m["q"]), kv8, idx.numpy(), qo.numpy(), ko.numpy(),
                                           w.sm_scale)
    _say(f"  FP8 rows: worst err/bound = {mla_check(out8, lse8, ref_o8, ref_l8):.3f}")


@pytest.mark.parametrize("batch,rows,heads,ctx,topk,slices", [
    (8, 5, 128, 3000, 2048, 3), (4, 6, 128, 3000, 2048, 5), (6, 6, 64, 3000, 2048, 7),
    (1, 6, 16, 3000, 2048, 8), (1, 6, 16, 5000, 4096, 16)])
def test_sparse_mla_slice_counts(batch, rows, heads, ctx, topk, slices):
    # Small grids cut each row's list into as many slices as fit one block per CU (any
    # count up to 16): the slices' bf16 partials are merged by the combine kernel.
    _say(f"sparse_mla slices={slices} (T={batch * rows}, H={heads}, k={topk})")
    w = W.replace(W.scaled(W.MTP5_VERIFY, ctx=ctx, batch=batch, topk=topk), rows=rows,
                  mla_heads=heads)
    lens = synth.context_lengths(w)
    qo, ko = synth.q_row_offsets(w), synth.kv_row_offsets(lens)
    m = synth.mla_inputs(w, lens)
    idx = synth.random_topk(w, lens, qo, w.topk, pad_frac=0.1)
    idx[3, : topk // 2] = -1           # a row whose first slices hold nothing
    T = int(qo[-1])
    need = api.sparse_mla_workspace_size(T, heads, w.topk)
    assert need == T * slices * heads * (512 * 2 + 8), "the case does not take the slices it names"
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    u16 = lambda x: x.view(torch.uint16).numpy()
    ref_o, ref_l = oracle.sparse_mla(u16(m["q"]), u16(m["kv"]), idx.numpy(), qo.numpy(),
                                     ko.numpy(), w.sm_scale)
    outs = []
    for call in range(2):
        out, lse = api.sparse_mla_decode(m["q"].to(DEV), m["kv"].to(DEV), idx.to(DEV), qo.to(DEV),
                                         ko.to(DEV), w.rows, w.sm_scale, workspace=ws)
        _say(f"  call {call}: worst err/bound = {mla_check(out, lse, ref_o, ref_l):.3f}")
        outs.append((out.clone(), lse.clone()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_sparse_mla_dense_equals_full_visible_set():
    # k >= visible: sparse MLA over every visible position is dense causal attention
    _say("sparse_mla dense case")
    w = W.replace(W.scaled(W.MTP5_VERIFY, ctx=700, batch=2, topk=1024), mla_heads=32)
    lens = [700, 333]
    qo, ko = synth.q_row_offsets(w), synth.kv_row_offsets(lens)
    m = synth.mla_inputs(w, lens)
    idx = synth.random_topk(w, lens, qo, w.topk)
    out, lse = api.sparse_mla_decode(m["q"].to(DEV), m["kv"].to(DEV), idx.to(DEV), qo.to(DEV),
                                     ko.to(DEV), w.rows, w.sm_scale)
    u16 = lambda x: x.view(torch.uint16).numpy()
    ref_o, ref_l = oracle.sparse_mla(u16(m["q"]), u16(m["kv"]), idx.numpy(), qo.numpy(), ko.numpy(),
                                     w.sm_scale)
    mla_check(out, lse, ref_o, ref_l)


# ---------------------------------------------------------------- greedy accept
@pytest.mark.parametrize("name,batch,vocab,K", [("tiny", 1, 1024, 1), ("f32", 7, 5000, 4),
                                                ("bf16", 32, 151552, 5), ("ragged", 3, 8193, 0)])
def test_greedy_accept_bitexact(name, batch, vocab, K):
    _say(f"greedy_accept {name}")
    base = W.TINY if name in ("tiny", "f32") else W.MTP5_VERIFY
    w = W.replace(base, batch=batch, vocab=vocab, rows=K + 1)
    a = synth.accept_inputs(w)
    logits = a["logits"]
    if name == "bf16":
        logits[3, 100] = logits[3].max()   # planted exact tie: lower index must win
        logits[3, 7] = logits[3, 100]
    n, nxt, am = api.greedy_accept(logits.to(DEV), a["draft"].to(DEV), K)
    host = logits.view(torch.uint16).numpy() if logits.dtype == torch.bfloat16 else logits.numpy()
    rn, rnx, ram = oracle.greedy_accept(host, a["draft"].numpy(), K)
    assert np.array_equal(n.cpu().numpy(), rn) and np.array_equal(nxt.cpu().numpy(), rnx)
    assert np.array_equal(am.cpu().numpy(), ram)
    assert np.array_equal(rn, a["planted_n"].numpy())


@pytest.mark.parametrize("dtype,pad", [(torch.bfloat16, 5), (torch.bfloat16, 8), (torch.float32, 3)])
def test_greedy_accept_strided_rows_via_abi(dtype, pad):
    # logits rows `pad` entries longer than the vocabulary (logits_ld = V + pad, so with an
    # odd pad most bf16 rows start off a 16-byte boundary): the entries past V hold the
    # row's largest value and must never be taken
    _say(f"greedy_accept strided rows {dtype} pad={pad}")
    from dsa_sparse_attention_amd import _lib
    B, K, V = 5, 3, 5000
    w = W.replace(W.TINY, batch=B, vocab=V, rows=K + 1)
    a = synth.accept_inputs(w)
    base = a["logits"].float()
    wide = torch.empty((B * (K + 1), V + pad), dtype=torch.float32)
    wide[:, :V] = base
    wide[:, V:] = base.max() + 1.0
    wide = wide.to(dtype)
    host = wide[:, :V].contiguous()
    host = host.view(torch.uint16).numpy() if dtype == torch.bfloat16 else host.numpy()
    rn, rnx, ram = oracle.greedy_accept(host, a["draft"].numpy(), K)
    lib = _lib.load()
    dev = wide.to(DEV)
    draft = a["draft"].to(DEV)
    n = torch.empty(B, dtype=torch.int32, device=DEV)
    nxt = torch.empty(B, dtype=torch.int32, device=DEV)
    am = torch.empty((B, K + 1), dtype=torch.int32, device=DEV)
    need = lib.greedy_accept_workspace_size(B, K, V)
    ws = torch.empty(max(need, 4), dtype=torch.uint8, device=DEV)
    dt = api.DSA_BF16 if dtype == torch.bfloat16 else api.DSA_F32
    rc = lib.greedy_accept(dev.data_ptr(), dt, V + pad, draft.data_ptr(), B, K, V, n.data_ptr(),
                           nxt.data_ptr(), am.data_ptr(), ws.data_ptr(), ws.numel(),
                           torch.cuda.current_stream().cuda_stream)
    assert rc == 0, lib.dsa_last_error()
    torch.cuda.synchronize()
    assert np.array_equal(am.cpu().numpy(), ram)
    assert np.array_equal(n.cpu().numpy(), rn) and np.array_equal(nxt.cpu().numpy(), rnx)


@pytest.mark.parametrize("name,pad", [("bf16", 5), ("f32", 3)])
def test_rejection_accept_strided_rows_equal_contiguous(name, pad):
    # logits rows `pad` entries longer than the vocabulary, the extra entries huge: the
    # result must be the same as for the contiguous rows (which the oracle test covers)
    _say(f"rejection_accept strided rows {name} pad={pad}")
    from dsa_sparse_attention_amd import _lib
    B, K, V = 6, 3, 5000
    w = W.scaled(W.TINY, ctx=4096, batch=B, vocab=V, rows=K + 1,
                 logits_dtype="f32" if name == "f32" else "bf16")
    d = synth.rejection_inputs(w, draft_noise=0.3)
    g = {k: v.to(DEV) for k, v in d.items()}
    n0, x0 = api.rejection_accept(g["logits"], g["draft_probs"], g["draft"], g["u"], g["us"], K)
    lg = g["logits"]
    wide = torch.full((lg.shape[0], V + pad), 1.0e4, dtype=lg.dtype, device=DEV)
    wide[:, :V] = lg
    lib = _lib.load()
    n = torch.empty(B, dtype=torch.int32, device=DEV)
    nxt = torch.empty(B, dtype=torch.int32, device=DEV)
    need = lib.rejection_accept_workspace_size(B, K, V)
    ws = torch.empty(max(need, 8), dtype=torch.uint8, device=DEV)
    dt = api.DSA_F32 if name == "f32" else api.DSA_BF16
    rc = lib.rejection_accept(wide.data_ptr(), dt, V + pad, g["draft_probs"].data_ptr(),
                              g["draft"].data_ptr(), g["u"].data_ptr(), g["us"].data_ptr(), B, K, V,
                              n.data_ptr(), nxt.data_ptr(), ws.data_ptr(), ws.numel(),
                              torch.cuda.current_stream().cuda_stream)
    assert rc == 0, lib.dsa_last_error()
    torch.cuda.synchronize()
    assert torch.equal(n, n0) and torch.equal(nxt, x0)


def test_abi_rejects_bad_arguments_before_launch():
    _say("abi error paths")
    x = torch.zeros((4, 96), device=DEV)
    with pytest.raises(api.DsaError, match="UNSUPPORTED"):
        api.quantize_fp8(x)
    s = torch.zeros((2, 64), device=DEV)
    qo = torch.tensor([0, 2], dtype=torch.int32, device=DEV)
    ko = torch.tensor([0, 64], dtype=torch.int64, device=DEV)
    with pytest.raises(api.DsaError, match="INVALID_ARGUMENT"):
        api.topk(s, qo, ko, 2, 64, 0)
    q = torch.zeros((2, 20, 576), dtype=torch.bfloat16, device=DEV)
    kv = torch.zeros((64, 576), dtype=torch.bfloat16, device=DEV)
    idx = torch.zeros((2, 8), dtype=torch.int32, device=DEV)
    with pytest.raises(api.DsaError, match="UNSUPPORTED"):
        api.sparse_mla_decode(q, kv, idx, qo, ko, 2, 0.1)
    lg = torch.zeros((4, 10), device=DEV)
    with pytest.raises(api.DsaError, match="WORKSPACE"):
        api.greedy_accept(lg, torch.zeros((2, 1), dtype=torch.int32, device=DEV), 1,
                          workspace=torch.zeros(4, dtype=torch.uint8, device=DEV))


# ---------------------------------------------------------------- rejection-sampling accept
def _rejection_candidates(lg, dp, draft, u, us, K, eps_u=1e-5, eps_s=2e-6):
    """Oracle results under relative nudges of the uniforms: a decision or a draw that a
    nudge flips sits within float rounding of its boundary, where either side is right."""
    outs = []
    for su in (-1, 0, 1):
        for ss in (-1, 0, 1):
            uu = np.clip(u.astype(np.float64) * (1 + su * eps_u), 0, 1).astype(np.float32)
            sv = np.clip(us.astype(np.float64) * (1 + ss * eps_s), 0, 0.99999994).astype(np.float32)
            n, nxt, _, _ = oracle.rejection_accept(lg, dp, draft, uu, sv, K)
            outs.append((n, nxt))
    return outs


@pytest.mark.parametrize("name,batch,vocab,K,noise", [("f32", 7, 5000, 4, 1.0), ("bf16", 32, 151552, 5, 1.0),
                                                      ("bf16", 16, 151552, 5, 0.3),
                                                      ("f32", 5, 3001, 0, 1.0), ("bf16", 9, 40000, 1, 2.0)])
def test_rejection_accept_matches_oracle(name, batch, vocab, K, noise):
    _say(f"rejection_accept {name} B={batch} V={vocab} K={K}")
    w = W.scaled(W.MTP5_VERIFY if name == "bf16" else W.TINY, ctx=4096, batch=batch, vocab=vocab,
                 rows=K + 1, logits_dtype="f32" if name == "f32" else "bf16")
    d = synth.rejection_inputs(w, draft_noise=noise)
    g = {k: v.to(DEV) for k, v in d.items()}
    n, nxt = api.rejection_accept(g["logits"], g["draft_probs"], g["draft"], g["u"], g["us"], K)
    n, nxt = n.cpu().numpy(), nxt.cpu().numpy()
    lg = d["logits"].numpy() if name == "f32" else d["logits"].view(torch.int16).numpy().view(np.uint16)
    args = (d["draft_probs"].numpy(), d["draft"].numpy(), d["u"].numpy(), d["us"].numpy())
    rn, rnx, _, _ = oracle.rejection_accept(lg, *args, K)
    cands = _rejection_candidates(lg, *args, K)
    strict = 0
    for b in range(batch):
        options = {(int(cn[b]), int(cx[b])) for cn, cx in cands}
        assert (int(n[b]), int(nxt[b])) in options, f"request {b}: {n[b], nxt[b]} not in {options}"
        if len(options) == 1:
            strict += 1
            assert n[b] == rn[b] and nxt[b] == rnx[b]
    _say(f"  {strict}/{batch} requests away from every float boundary; mean accepted {n.mean():.2f}")
    assert strict >= batch // 2
