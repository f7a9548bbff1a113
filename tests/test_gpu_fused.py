"""Fused indexer score + refined top-k (dsa_index_topk) against the oracle, through the C ABI.

Bar: on every row, the set equals the oracle's top-k by the exact scores (bit-exact index
sets), with every row refined (status >= 0). Cases cover rows selected from their
candidates, rows whose candidates include every key (short contexts), and rows scored again
by their own block (exact-grid ties that swamp the candidate capacity).
"""
import numpy as np
import pytest
import torch

import oracle
from dsa_sparse_attention_amd import api, synth, workloads
from tests._pipeline import DEV, Case, gpu_indexer, oracle_quant

pytestmark = pytest.mark.gpu

W = workloads
SMALL = {
    "tiny": W.TINY,
    "decode_verify@4096": W.scaled(W.DECODE_VERIFY, ctx=4096, batch=3, topk=512),
    "mtp5_verify@6000": W.scaled(W.MTP5_VERIFY, ctx=6000, batch=3, topk=512),
    "mtp5_verify@24000": W.scaled(W.MTP5_VERIFY, ctx=24000, batch=2, topk=512),
    "long_ctx@12800": W.scaled(W.LONG_CTX, ctx=12800, batch=1, topk=64),
}


def _say(*a):
    print(*a, flush=True)


def _fused(gi, case, k, err_scale=0.0):
    T = case.T
    status = torch.full((T,), -9, dtype=torch.int32, device=DEV)
    path = torch.full((T,), -9, dtype=torch.int32, device=DEV)
    top = api.index_topk(gi["qc"], gi["qs"], case.w_f32, gi["kc"], gi["ks"], case.qo_d, case.ko_d,
                         case.w.rows, case.max_kv, k, status=status, path=path, err_scale=err_scale)
    return top.cpu().numpy(), status.cpu().numpy(), path.cpu().numpy()


@pytest.mark.parametrize("name", list(SMALL))
def test_fused_topk_equals_oracle(name):
    w = SMALL[name]
    _say(f"fused index_topk {name}")
    case = Case(w, with_mla=False, with_accept=False)
    gi = gpu_indexer(case)
    top, st, path = _fused(gi, case, w.topk)
    qc, qs, kc, ks, ko = oracle_quant(case)
    rows = np.arange(case.T)
    ref_s = oracle.index_score(qc, qs, case.host("w_f32"), kc, ks, case.qo.numpy(), ko,
                               rows=rows, width=case.max_kv)
    nvis = np.array([case.visible(int(t)) for t in rows])
    ref_k = oracle.topk(ref_s, nvis, w.topk)
    _say(f"  status min {st.min()}, band max {st.max()}, rows rescored {int((path == 1).sum())}")
    assert st.min() >= 0
    assert np.all((path == 0) | (path == 1))
    assert np.array_equal(top, ref_k)
    if w.spike_frac:
        for t in rows:
            assert list(top[t]) == list(case.spike_pos[0][:w.topk].numpy())


@pytest.mark.parametrize("ctx,k", [(2050, 2048), (8195, 2048), (65539, 2048), (300, 2048)])
def test_fused_row_lengths_around_k_and_path_sizes(ctx, k):
    # six verify rows of one request see ctx - 5 .. ctx keys: around k (n < k keeps every
    # visible key, n = k, n = k + 1), around the register path's size steps and its end, and
    # a context shorter than k; every row's set must be the oracle's, every row refined
    w = W.replace(W.scaled(W.MTP5_VERIFY, ctx=ctx, batch=1, topk=k), ctx_min=0)
    _say(f"fused index_topk at row lengths {ctx - 5}..{ctx}, k={k}")
    case = Case(w, with_mla=False, with_accept=False)
    gi = gpu_indexer(case)
    top, st, path = _fused(gi, case, k)
    qc, qs, kc, ks, ko = oracle_quant(case)
    rows = np.arange(case.T)
    ref_s = oracle.index_score(qc, qs, case.host("w_f32"), kc, ks, case.qo.numpy(), ko,
                               rows=rows, width=case.max_kv)
    nvis = np.array([case.visible(int(t)) for t in rows])
    assert list(nvis) == list(range(ctx - 5, ctx + 1))
    ref_k = oracle.topk(ref_s, nvis, k)
    _say(f"  status {list(st)}, path {list(path)}")
    assert st.min() >= 0
    assert np.array_equal(top, ref_k)


def test_fused_ragged_many_requests():
    # ragged requests, empty ones, rows before their request's first key: every row's set
    # equals the oracle's
    _say("fused index_topk ragged requests")
    rng = np.random.default_rng(31)
    B, H, D, k = 40, 16, 128, 48
    lens = rng.integers(0, 700, B)
    lens[rng.choice(B, 5, replace=False)] = 0
    lens[0] = 3
    R = rng.integers(1, 8, B)
    qo = np.concatenate([[0], np.cumsum(R)]).astype(np.int32)
    ko = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T, N, L = int(qo[-1]), int(ko[-1]), int(lens.max())
    q = rng.standard_normal((T, H, D)).astype(np.float32)
    kk = rng.standard_normal((N, D)).astype(np.float32)
    wt = rng.random((T, H)).astype(np.float32)
    qc, qs = oracle.quantize(q)
    kc, ks = oracle.quantize(kk)
    d = lambda a: torch.from_numpy(a).to(DEV)
    status = torch.zeros(T, dtype=torch.int32, device=DEV)
    top = api.index_topk(d(qc), d(qs), d(wt), d(kc), d(ks), d(qo), d(ko), int(R.max()), L, k,
                         status=status).cpu().numpy()
    ref_s = oracle.index_score(qc, qs, wt, kc, ks, qo, ko, width=max(L, 1))
    nvis = np.array([oracle.row_visible(qo, ko, t) for t in range(T)])
    ref_k = oracle.topk(ref_s, nvis, k)
    assert status.min().item() >= 0
    assert np.array_equal(top, ref_k)
    assert np.all(top[nvis == 0] == -1) and np.any(nvis == 0)


def _sample_count(max_kv_len):
    """Samples per request of dsa_index_topk (include/dsa.h: about one key in 32 of the
    longest request, 1024..8192)."""
    S = 1024
    while S < 8192 and S * 32 < max_kv_len:
        S *= 2
    return S


def test_fused_unsampled_spikes_take_the_row_fallback():
    # 7000 keys with large, distinct scores sit only at positions the threshold sample never
    # visits, so the sample's threshold admits far more candidates than a block holds: every
    # row is scored again by its own block, and its set must still be the oracle's
    _say("fused index_topk unsampled spikes (row fallback)")
    rng = np.random.default_rng(14)
    R, H, D, L, k = 2, 16, 128, 40000, 1024
    n0 = L - R + 1
    S = _sample_count(L)
    sampled = np.unique((np.arange(S, dtype=np.int64) * n0) // S)
    free = np.setdiff1d(np.arange(n0), sampled)
    spikes = np.sort(rng.choice(free, 7000, replace=False))
    q = rng.standard_normal((R, H, D)).astype(np.float32)
    wt = rng.random((R, H)).astype(np.float32)
    kk = rng.standard_normal((L, D)).astype(np.float32)
    direction = (wt[0][:, None] * q[0]).sum(0)
    direction /= np.linalg.norm(direction)
    kk[spikes] = direction[None, :] * rng.uniform(6.0, 9.0, (len(spikes), 1)) * np.sqrt(D)
    qc, qs = oracle.quantize(q)
    kc, ks = oracle.quantize(kk)
    qo = np.array([0, R], np.int32)
    ko = np.array([0, L], np.int64)
    d = lambda a: torch.from_numpy(a).to(DEV)
    status = torch.zeros(R, dtype=torch.int32, device=DEV)
    path = torch.zeros(R, dtype=torch.int32, device=DEV)
    top = api.index_topk(d(qc), d(qs), d(wt), d(kc), d(ks), d(qo), d(ko), R, L, k,
                         status=status, path=path).cpu().numpy()
    ref_s = oracle.index_score(qc, qs, wt, kc, ks, qo, ko)
    nvis = np.array([L - R + t + 1 for t in range(R)])
    ref_k = oracle.topk(ref_s, nvis, k)
    p = path.cpu().numpy()
    _say(f"  rows rescored {int((p == 1).sum())}/{R}, statuses {status.cpu().tolist()}")
    assert np.all(p == 1), "rows with unsampled spikes were expected to be scored again"
    assert status.min().item() >= 0
    assert np.array_equal(top, ref_k)
    assert np.all(np.isin(top[0], spikes))


def test_fused_exact_grid_ties():
    # integer codes on a small grid, unit scales, w = m/16: scores are exact and heavily
    # tied around the threshold; the sets must be the oracle's (ties to the lower position)
    _say("fused index_topk exact grid")
    rng = np.random.default_rng(12)
    T, H, D, L, k = 6, 64, 128, 30000, 512
    vals = np.array([-2, -1, 0, 1, 2], np.float32)
    q = oracle.fp8_encode(rng.choice(vals, (T, H, D)))
    kc = oracle.fp8_encode(rng.choice(vals, (L, D)))
    w = (rng.integers(0, 2, (T, H)) / 16).astype(np.float32)
    qs = np.ones((T, H), np.float32)
    ks = np.ones(L, np.float32)
    qo = np.array([0, T], np.int32)
    ko = np.array([0, L], np.int64)
    d = lambda a: torch.from_numpy(a).to(DEV)
    status = torch.zeros(T, dtype=torch.int32, device=DEV)
    path = torch.zeros(T, dtype=torch.int32, device=DEV)
    top = api.index_topk(d(q), d(qs), d(w), d(kc), d(ks), d(qo), d(ko), T, L, k, status=status,
                         path=path).cpu().numpy()
    ref_s = oracle.index_score(q, qs, w, kc, ks, qo, ko)
    nvis = np.array([L - T + t + 1 for t in range(T)])
    ref_k = oracle.topk(ref_s, nvis, k)
    p = path.cpu().numpy()
    _say(f"  rows rescored {int((p == 1).sum())}/{T}, statuses {sorted(set(status.cpu().tolist()))}")
    assert status.min().item() >= 0
    assert np.array_equal(top, ref_k)


def test_fused_rejects_bad_arguments():
    _say("fused index_topk error paths")
    q = torch.zeros((2, 8, 128), dtype=torch.uint8, device=DEV)
    ones = torch.ones((2, 8), device=DEV)
    kc = torch.zeros((64, 128), dtype=torch.uint8, device=DEV)
    ks = torch.ones(64, device=DEV)
    qo = torch.tensor([0, 2], dtype=torch.int32, device=DEV)
    ko = torch.tensor([0, 64], dtype=torch.int64, device=DEV)
    with pytest.raises(api.DsaError, match="INVALID_ARGUMENT"):
        api.index_topk(q, ones, ones, kc, ks, qo, ko, 2, 64, 4097)
    with pytest.raises(api.DsaError, match="WORKSPACE"):
        api.index_topk(q, ones, ones, kc, ks, qo, ko, 2, 64, 8,
                       workspace=torch.zeros(256, dtype=torch.uint8, device=DEV))
