"""Pins of the oracle's sparse MLA, index sharing and greedy acceptance (CPU only).

Sparse MLA ("MAX Pipeline 中的 DeepSeek-V3.2 架构实现解析", 稀疏 MLA 的前向路径; latent
512 + rope 64 from "GLM-5.3 推理全链路(十四)", 草稿层) is pinned to closed forms and
to torch's float64 scaled_dot_product_attention on the dense causal case.
Index sharing ("MAX 中 GLM-5.2 ... 统一 MTP 推测解码架构解析", 阶段 5) is pinned to a
physically compacted copy. Greedy acceptance ("GLM-5.3 推理全链路(十四)", 接受判定)
is pinned to the planted prefix lengths and torch.argmax's first-maximum rule.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from dsa_sparse_attention_amd import accounting, synth, workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16(x):
    return torch.as_tensor(x, dtype=torch.float32).to(torch.bfloat16).view(torch.uint16).numpy()


def _f(x_u16):
    return torch.from_numpy(np.ascontiguousarray(x_u16)).view(torch.bfloat16).double().numpy()


def _mla_case(rng, L=(40, 25), R=2, H=3):
    B = len(L)
    qo = np.arange(B + 1, dtype=np.int32) * R
    ko = np.concatenate([[0], np.cumsum(L)]).astype(np.int64)
    q = _bf16(rng.standard_normal((B * R, H, 576)))
    kv = _bf16(rng.standard_normal((int(ko[-1]), 576)))
    return q, kv, qo, ko


def test_identical_rows_give_that_row():
    rng = np.random.default_rng(1)
    q, kv, qo, ko = _mla_case(rng, L=(40,), R=1)
    kv[:] = kv[7]
    idx = np.array([[3, 9, 20, 33, -1, 0]], np.int32)
    out, lse = oracle.sparse_mla(q, kv, idx, qo, ko, 0.05)
    assert np.allclose(out[0], np.broadcast_to(_f(kv[7, :512]), (3, 512)), rtol=1e-14, atol=1e-14)
    z = float(np.float32(0.05)) * (_f(q[0]) @ _f(kv[7]))  # sm_scale is passed as float32
    assert np.allclose(lse[0], z + math.log(5), rtol=1e-13)


def test_zero_query_gives_mean_and_single_index_gives_row():
    rng = np.random.default_rng(2)
    q, kv, qo, ko = _mla_case(rng, L=(40,), R=1)
    q[:] = 0
    idx = np.array([[1, 4, 9, 16, 25, 36]], np.int32)
    out, lse = oracle.sparse_mla(q, kv, idx, qo, ko, 0.1)
    mean = _f(kv[idx[0], :512]).mean(axis=0)
    assert np.allclose(out[0], mean, rtol=1e-12, atol=1e-14)
    assert np.allclose(lse[0], math.log(6))
    idx1 = np.array([[-1, 17, -1, -1, -1, -1]], np.int32)
    out1, _ = oracle.sparse_mla(q, kv, idx1, qo, ko, 0.1)
    assert np.array_equal(out1[0], np.broadcast_to(_f(kv[17, :512]), (3, 512)))


def test_no_valid_index_gives_zero_and_neg_inf():
    rng = np.random.default_rng(3)
    q, kv, qo, ko = _mla_case(rng, L=(40,), R=1)
    idx = np.array([[-1, -1, 40, 99]], np.int32)   # -1 and positions past the request skipped
    out, lse = oracle.sparse_mla(q, kv, idx, qo, ko, 0.1)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def test_full_visible_set_equals_dense_causal_sdpa():
    rng = np.random.default_rng(4)
    L, R, H = (40, 25), 3, 4
    q, kv, qo, ko = _mla_case(rng, L=L, R=R, H=H)
    k = max(L)
    idx = np.full((len(L) * R, k), -1, np.int32)
    for b, Lb in enumerate(L):
        for r in range(R):
            vis = Lb - R + r + 1
            idx[b * R + r, :vis] = np.arange(vis)
    scale = float(np.float32(1 / math.sqrt(576)))   # sm_scale crosses the ABI as float32
    out, lse = oracle.sparse_mla(q, kv, idx, qo, ko, scale)
    for b, Lb in enumerate(L):
        C = torch.from_numpy(_f(kv[ko[b]:ko[b + 1]]))                       # [L, 576]
        Q = torch.from_numpy(_f(q[b * R:(b + 1) * R])).transpose(0, 1)     # [H, R, 576]
        mask = torch.zeros((R, Lb), dtype=torch.bool)
        for r in range(R):
            mask[r, :Lb - R + r + 1] = True
        ref = F.scaled_dot_product_attention(Q, C[None].expand(H, -1, -1),
                                             C[None, :, :512].expand(H, -1, -1),
                                             attn_mask=mask, scale=scale)
        got = torch.from_numpy(out[b * R:(b + 1) * R]).transpose(0, 1)
        assert torch.allclose(got, ref, rtol=1e-10, atol=1e-12)
        logits = (Q @ C.T) * scale
        ref_lse = torch.logsumexp(logits.masked_fill(~mask, -math.inf), dim=-1)
        assert torch.allclose(torch.from_numpy(lse[b * R:(b + 1) * R]).T, ref_lse, rtol=1e-12)


def test_permutation_invariance():
    rng = np.random.default_rng(5)
    q, kv, qo, ko = _mla_case(rng, L=(60,), R=1)
    idx = np.array([[5, 50, 12, 33, 7, 58, 21]], np.int32)
    a, la = oracle.sparse_mla(q, kv, idx, qo, ko, 0.07)
    b, lb = oracle.sparse_mla(q, kv, idx[:, ::-1].copy(), qo, ko, 0.07)
    assert np.allclose(a, b, rtol=1e-13, atol=1e-15) and np.allclose(la, lb, rtol=1e-14)


def test_index_share_equals_compacted_copy():
    # step-0 top-k rows of 3 requests x 4 rows; draft step reads row base[b] + n[b]
    rng = np.random.default_rng(6)
    L = (50, 60, 70)
    _, kv, _, ko = _mla_case(rng, L=L, R=1)
    q1 = _bf16(rng.standard_normal((3, 2, 576)))
    qo1 = np.arange(4, dtype=np.int32)
    step0 = np.stack([np.sort(rng.choice(45, 16, replace=False)) for _ in range(12)]).astype(np.int32)
    base = np.array([0, 4, 8, 12], np.int32)
    n_acc = np.array([2, 0, 3], np.int32)
    shared, lse_s = oracle.sparse_mla(q1, kv, step0, qo1, ko, 0.04, share_base=base,
                                      num_accepted=n_acc)
    compact = step0[base[:3] + n_acc]
    ref, lse_r = oracle.sparse_mla(q1, kv, compact, qo1, ko, 0.04)
    assert np.array_equal(shared, ref) and np.array_equal(lse_s, lse_r)


def test_greedy_accept_planted_prefix_and_first_max():
    w = workloads.replace(workloads.TINY, batch=64, rows=5, vocab=500)
    inp = synth.accept_inputs(w)
    n, nxt, am = oracle.greedy_accept(inp["logits"].numpy(), inp["draft"].numpy(), w.drafts)
    assert np.array_equal(n, inp["planted_n"].numpy())
    ref = torch.argmax(inp["logits"], dim=1).view(w.batch, w.rows).numpy()
    assert np.array_equal(am, ref)
    assert np.array_equal(nxt, am[np.arange(w.batch), n])


def test_greedy_accept_closed_forms_and_ties():
    V, K = 10, 3
    logits = np.zeros((2 * (K + 1), V), np.float32)
    # request 0: all drafts match; request 1: first draft misses
    for i, tok in enumerate([4, 5, 6, 7]):
        logits[i, tok] = 1.0
    logits[4 + 0, 2] = 3.0
    logits[4 + 0, 8] = 3.0              # tie: token 2 wins (first maximum)
    draft = np.array([[4, 5, 6], [8, 1, 1]], np.int32)
    n, nxt, am = oracle.greedy_accept(logits, draft, K)
    assert list(n) == [3, 0] and list(nxt) == [7, 2]
    assert am[1, 0] == int(torch.argmax(torch.from_numpy(logits[4])))
    # bf16 logits with -0.0 vs +0.0: equal values, lower index wins
    lb = np.zeros((1, 4), np.float32)
    lb[0, 0] = -0.0
    lb[0, 2] = -1.0
    n, nxt, _ = oracle.greedy_accept(_bf16(lb), np.zeros((1, 0), np.int32), 0)
    assert list(n) == [0] and list(nxt) == [0]


def test_planted_acceptance_reproduces_pages_mean_accept_length():
    gold = json.load(open(os.path.join(GOLDEN, "acceptance_lengths.json")))
    K = gold["draft_steps"]
    w = workloads.replace(workloads.TINY, batch=20000, rows=K + 1)
    n = synth.accepted_lengths(w).numpy()
    a = w.accept_rate
    closed = sum(a ** i for i in range(K + 1))            # E[n + 1] of the chain law
    assert abs(closed - gold["GLM-5"]) < 0.005
    sigma = np.std(n + 1) / math.sqrt(len(n))
    assert abs(np.mean(n + 1) - closed) < 4 * sigma


def test_indexer_read_ledger_matches_pages():
    gold = json.load(open(os.path.join(GOLDEN, "indexer_read_ledger.json")))
    assert accounting.index_key_bytes(1, gold["index_head_dim"]) == gold["bytes_per_token_per_layer"]
    assert accounting.index_key_bytes(1, 128, gold["full_indexer_layers"]) == \
        gold["bytes_per_token_all_full_layers"]
    for case in gold["cases"]:
        L = case["context"]
        ns = accounting.draft_round_index_bytes(L, 128, gold["full_indexer_layers"],
                                                gold["draft_forwards"], share=False) / 1e9
        sh = accounting.draft_round_index_bytes(L, 128, gold["full_indexer_layers"],
                                                gold["draft_forwards"], share=True) / 1e9
        assert abs(ns - case["no_share_GB"]) <= case["printed_precision_GB"]
        assert abs(sh - case["share_GB"]) <= case["printed_precision_GB"]
        assert ns / sh == gold["draft_forwards"]


def test_verify_layout_facts():
    gold = json.load(open(os.path.join(GOLDEN, "verify_layout.json")))
    assert gold["speculative_num_steps"] + 1 == gold["verify_rows_per_request"]
    assert workloads.MTP5_VERIFY.rows == gold["verify_rows_per_request"]
    assert workloads.MTP5_VERIFY.batch * workloads.MTP5_VERIFY.rows == \
        gold["batch_example"]["verify_tokens"]
    K = 5
    assert accounting.merged_offsets([0, 7, 9, 20], K) == [0, 7 + 5, 9 + 10, 20 + 15]


def test_verify_cache_rows_are_each_rows_own_position():
    # the cache row a verify row writes is its own position: one past it is exactly the
    # number of keys the row sees under the causal rule
    from dsa_sparse_attention_amd import synth
    lengths = [7, 300, 65, 1024]
    rows = [3, 1, 6, 2]
    qo = np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)
    ko = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    dst = synth.verify_cache_rows(lengths, rows).numpy()
    assert len(dst) == qo[-1] and len(set(dst.tolist())) == len(dst)
    for t in range(int(qo[-1])):
        b = int(np.searchsorted(qo, t, side="right") - 1)
        assert ko[b] <= dst[t] < ko[b + 1]
        assert dst[t] - ko[b] + 1 == oracle.row_visible(qo, ko, t)
