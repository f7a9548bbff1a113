"""Pins of the oracle's rejection-sampling acceptance ("GLM-5.3 推理全链路(十四)",
"接受判定:greedy 与 rejection sampling": keep draft i with probability min(1, p/q); at the
first refusal draw the step's token from the corrected distribution).

The defining property of the scheme is that the emitted tokens follow the target
distribution whatever the draft distribution is; the Monte Carlo test checks that law, and
the closed-form cases pin the accept test, the corrected distribution and the draw."""
import numpy as np
import pytest

import oracle



def _logits_of(p):
    return np.log(np.asarray(p, np.float64)).astype(np.float32)


def test_emitted_tokens_follow_the_target_law():
    # K = 1: the first emitted token (the draft if kept, else the corrected draw) follows
    # p_0, and the bonus after a kept draft follows p_1, for a draft law q_0 far from p_0
    rng = np.random.default_rng(1)
    V, N = 6, 200_000
    p0 = np.array([0.05, 0.30, 0.10, 0.25, 0.20, 0.10])
    p1 = np.array([0.40, 0.10, 0.10, 0.10, 0.20, 0.10])
    q0 = np.array([0.30, 0.05, 0.30, 0.05, 0.10, 0.20], np.float32)
    logits = np.tile(np.stack([_logits_of(p0), _logits_of(p1)]), (N, 1))
    cq = np.cumsum(q0.astype(np.float64))
    draft = np.minimum(np.searchsorted(cq, rng.random(N) * cq[-1], side="right"), V - 1)
    draft = draft.astype(np.int32).reshape(N, 1)
    dp = np.tile(q0, (N, 1, 1))
    u = rng.random((N, 1)).astype(np.float32)
    us = rng.random(N).astype(np.float32)
    n, nxt, _, _ = oracle.rejection_accept(logits, dp, draft, u, us, 1)
    first = np.where(n == 1, draft[:, 0], nxt)
    for law, tok in ((p0, first), (p1, nxt[n == 1])):
        freq = np.bincount(tok, minlength=V) / len(tok)
        sigma = np.sqrt(law * (1 - law) / len(tok))
        assert np.all(np.abs(freq - law) < 5 * sigma), (freq, law)


def test_identical_draft_and_target_keep_every_draft():
    rng = np.random.default_rng(2)
    B, K, V = 50, 4, 40
    logits = rng.normal(0, 2, (B * (K + 1), V)).astype(np.float32)
    p = np.exp(logits.astype(np.float64) - logits.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    dp = p.reshape(B, K + 1, V)[:, :K].astype(np.float32)
    draft = rng.integers(0, V, (B, K)).astype(np.int32)
    u = (0.999 * rng.random((B, K))).astype(np.float32)
    n, _, margin, _ = oracle.rejection_accept(logits, dp, draft, u, rng.random(B).astype(np.float32), K)
    assert np.all(n == K) and np.all(margin > 0)


def test_one_hot_draft_law_closed_form():
    # q = one-hot at x: the draft is kept iff u < p(x); the corrected law is p with x
    # removed, renormalised
    p = [0.1, 0.3, 0.6]
    logits = np.stack([_logits_of(p), _logits_of(p)])
    dp = np.array([[[0.0, 1.0, 0.0]]], np.float32)
    draft = np.array([[1]], np.int32)
    n, _, _, _ = oracle.rejection_accept(logits, dp, draft, np.array([[0.29]], np.float32),
                                         np.array([0.5], np.float32), 1)
    assert n[0] == 1
    for us, tok in ((0.1, 0), (0.14, 0), (0.2, 2), (0.99, 2)):
        n, nxt, _, _ = oracle.rejection_accept(logits, dp, draft, np.array([[0.31]], np.float32),
                                               np.array([us], np.float32), 1)
        assert n[0] == 0 and nxt[0] == tok, (us, nxt[0])


def test_draw_skips_zero_weight_entries_and_bonus_row():
    # every draft kept (q <= p at the drafts): the token comes from the last row; zero
    # probabilities are never drawn, u_s = 0 gives the first positive entry
    V = 5
    last = np.array([0.0, 0.0, 0.5, 0.0, 0.5])
    with np.errstate(divide="ignore"):
        rows = np.stack([np.log(np.full(V, 0.2)), np.log(last)]).astype(np.float32)
    dp = np.full((1, 1, V), 0.2, np.float32)
    for us, tok in ((0.0, 2), (0.49, 2), (0.51, 4), (0.999, 4)):
        n, nxt, _, _ = oracle.rejection_accept(rows, dp, np.array([[3]], np.int32),
                                               np.array([[0.5]], np.float32),
                                               np.array([us], np.float32), 1)
        assert n[0] == 1 and nxt[0] == tok


def test_bf16_logits_equal_their_float32_values():
    rng = np.random.default_rng(3)
    B, K, V = 8, 3, 64
    f = rng.normal(0, 3, (B * (K + 1), V)).astype(np.float32)
    bits = (f.view(np.uint32) >> 16).astype(np.uint16)
    f_round = (bits.astype(np.uint32) << 16).view(np.float32)
    dp = rng.dirichlet(np.ones(V), (B, K)).astype(np.float32)
    draft = rng.integers(0, V, (B, K)).astype(np.int32)
    u = rng.random((B, K)).astype(np.float32)
    us = rng.random(B).astype(np.float32)
    a = oracle.rejection_accept(bits, dp, draft, u, us, K)
    b = oracle.rejection_accept(f_round, dp, draft, u, us, K)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
