"""Pins of the oracle's lightning-indexer score and top-k (CPU only).

Pinned against: exact integer arithmetic (every e4m3fn value is a multiple of
2^-9), torch float64 matmul for cases that reduce to one head, one-hot head
weights (which isolate each head and each scale), Python's sorted() as a brute
force for the selection, and the planted-spike closed form.
Score/selection semantics: "MAX Pipeline 中的 DeepSeek-V3.2 架构实现解析",
Indexer 的结构与计算流程 (top-k of shape (total_seq_len, index_topk)); chain
verify rows see a plain causal prefix ("GLM-5.3 推理全链路(十四)", 验证段).
"""
import numpy as np
import pytest
import torch

import oracle
from dsa_sparse_attention_amd import synth, workloads


def _rand_codes(rng, shape):
    c = rng.integers(0, 256, size=shape, dtype=np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x3F  # no NaN codes
    return c


def _case(rng, B=2, L=(37, 50), R=3, H=4, D=64):
    qo = np.arange(B + 1, dtype=np.int32) * R
    ko = np.concatenate([[0], np.cumsum(L)]).astype(np.int64)
    T, N = B * R, int(ko[-1])
    q = _rand_codes(rng, (T, H, D))
    k = _rand_codes(rng, (N, D))
    qs = rng.uniform(0.01, 2, (T, H)).astype(np.float32)
    ks = rng.uniform(0.01, 2, N).astype(np.float32)
    w = rng.uniform(0, 1, (T, H)).astype(np.float32)
    return q, qs, w, k, ks, qo, ko


def test_dot_products_are_exact_integers():
    rng = np.random.default_rng(1)
    q, qs, w, k, ks, qo, ko = _case(rng, B=1, L=(40,), R=1, H=1, D=128)
    ones = np.ones_like(qs)
    got = oracle.index_score(q, ones, np.ones_like(w), k, np.ones_like(ks), qo, ko)
    # exact: integer multiples of 2^-9 -> int64 dot, then ReLU
    qi = (oracle.fp8_decode(q) * 512).astype(np.int64)[0, 0]
    ki = (oracle.fp8_decode(k) * 512).astype(np.int64)
    exact = np.maximum(ki @ qi, 0).astype(np.float64) / 2.0 ** 18
    assert np.array_equal(got[0, :40], exact)


def test_single_head_reduces_to_matmul_relu_and_causal_rule():
    rng = np.random.default_rng(2)
    q, qs, w, k, ks, qo, ko = _case(rng, B=2, L=(37, 50), R=3, H=1, D=64)
    got = oracle.index_score(q, qs, w, k, ks, qo, ko)
    qd = torch.from_numpy(oracle.fp8_decode(q)[:, 0, :])
    kd = torch.from_numpy(oracle.fp8_decode(k))
    for b in range(2):
        L = int(ko[b + 1] - ko[b])
        kb = kd[ko[b]:ko[b + 1]]
        for r in range(3):
            t = b * 3 + r
            vis = L - 3 + r + 1                       # row r sits at position L-R+r
            ref = torch.relu(kb @ qd[t]).numpy() * float(w[t, 0]) * float(qs[t, 0])
            ref = ref * ks[ko[b]:ko[b + 1]].astype(np.float64)
            assert np.allclose(got[t, :vis], ref[:vis], rtol=1e-14, atol=0)
            assert np.all(np.isneginf(got[t, vis:]))
            assert oracle.row_visible(qo, ko, t) == vis


def test_one_hot_weights_isolate_each_head_and_scale():
    rng = np.random.default_rng(3)
    q, qs, w, k, ks, qo, ko = _case(rng, B=1, L=(30,), R=2, H=5, D=64)
    qd = torch.from_numpy(oracle.fp8_decode(q))
    kd = torch.from_numpy(oracle.fp8_decode(k))
    total = np.zeros((2, 30))
    for j in range(5):
        wj = np.zeros_like(w)
        wj[:, j] = w[:, j]
        got = oracle.index_score(q, qs, wj, k, ks, qo, ko)
        for t in range(2):
            ref = (torch.relu(kd @ qd[t, j]).numpy() * float(w[t, j]) * float(qs[t, j])
                   * ks.astype(np.float64))
            vis = 30 - 2 + t + 1
            assert np.allclose(got[t, :vis], ref[:vis], rtol=1e-14, atol=0)
            total[t, :vis] += got[t, :vis]
    full = oracle.index_score(q, qs, w, k, ks, qo, ko)
    assert np.allclose(full[0, :29], total[0, :29], rtol=1e-12)
    assert np.allclose(full[1, :30], total[1, :30], rtol=1e-12)


def test_exact_grid_scores_are_multiples_of_one_sixteenth():
    # integer codes in [-4, 4] are exact in e4m3fn; unit scales; w in {m/16}
    rng = np.random.default_rng(4)
    vals = np.array([-4, -3, -2, -1, 0, 1, 2, 3, 4], np.float32)
    q = oracle.fp8_encode(rng.choice(vals, (2, 8, 64)))
    k = oracle.fp8_encode(rng.choice(vals, (100, 64)))
    w = (rng.integers(0, 16, (2, 8)) / 16).astype(np.float32)
    qo = np.array([0, 2], np.int32)
    ko = np.array([0, 100], np.int64)
    s = oracle.index_score(q, np.ones((2, 8), np.float32), w, k, np.ones(100, np.float32), qo, ko)
    fin = s[np.isfinite(s)]
    assert np.array_equal(fin * 16, np.round(fin * 16)) and fin.max() < 2 ** 21
    qi = oracle.fp8_decode(q).astype(np.int64)
    ki = oracle.fp8_decode(k).astype(np.int64)
    wi = np.round(w * 16).astype(np.int64)
    ref = (np.maximum(np.einsum("thd,sd->ths", qi, ki), 0) * wi[:, :, None]).sum(1) / 16
    assert np.array_equal(s[0, :99], ref[0, :99]) and np.array_equal(s[1], ref[1])


def _brute_topk(row, n, k):
    order = sorted(range(n), key=lambda s: (-row[s], s))[:k]
    return sorted(order) + [-1] * (k - min(k, n))


@pytest.mark.parametrize("levels", [0, 3, 50])
def test_topk_matches_brute_force(levels):
    rng = np.random.default_rng(5 + levels)
    rows, width, k = 7, 300, 40
    if levels:
        s = rng.integers(0, levels, (rows, width)).astype(np.float64)
    else:
        s = rng.standard_normal((rows, width))
    nv = np.array([300, 299, 41, 40, 39, 1, 0], np.int64)
    got = oracle.topk(s, nv, k)
    for i in range(rows):
        assert list(got[i]) == _brute_topk(s[i], int(nv[i]), k)


def test_topk_ties_go_to_lower_position_and_pad():
    s = np.zeros((1, 10))
    got = oracle.topk(s, [10], 4)
    assert list(got[0]) == [0, 1, 2, 3]
    s = np.array([[1.0, 5.0, 5.0, 2.0, 5.0]])
    assert list(oracle.topk(s, [5], 2)[0]) == [1, 2]
    assert list(oracle.topk(s, [3], 5)[0]) == [0, 1, 2, -1, -1]
    # -0.0 and +0.0 are the same score: the lower position wins
    s = np.array([[0.0, -0.0, -1.0]])
    assert list(oracle.topk(s, [3], 1)[0]) == [0]
    s = np.array([[-0.0, 0.0, -1.0]])
    assert list(oracle.topk(s, [3], 1)[0]) == [0]


def test_planted_spikes_select_lowest_spike_positions():
    # long-context geometry at a CPU-sized context: spikes must own the top-k and,
    # tying exactly, be decided by position (closed form: the k lowest spike positions)
    w = workloads.scaled(workloads.LONG_CTX, ctx=12800, batch=1, topk=64)
    lens = synth.context_lengths(w)
    inp = synth.indexer_inputs(w, lens)
    qc, qs = oracle.quantize(inp["q"].numpy())
    kc, ks = oracle.quantize(inp["k"].numpy())
    qo = synth.q_row_offsets(w).numpy()
    ko = synth.kv_row_offsets(lens).numpy()
    s = oracle.index_score(qc, qs, inp["w"].numpy(), kc, ks, qo, ko)
    spikes = inp["spike_pos"][0].numpy()
    assert len(spikes) == 128 > w.topk
    nv = np.array([oracle.row_visible(qo, ko, t) for t in range(w.rows)])
    others = np.ones(w.ctx, bool)
    others[spikes] = False
    for t in range(w.rows):
        assert np.all(s[t, spikes] == s[t, spikes[0]])           # identical keys tie exactly
        assert s[t, spikes[0]] > s[t, :nv[t]][others[:nv[t]]].max()
    got = oracle.topk(s, nv, w.topk)
    for t in range(w.rows):
        assert list(got[t]) == list(spikes[:w.topk])
