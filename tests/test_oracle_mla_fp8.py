"""Pins of the oracle's FP8 latent cache rows and its sparse MLA over them (no GPU).

The row layout is the pages' 656 bytes per token per layer ("GLM-5.3 推理全链路(十四)",
the draft layer's KV pool); the split 512 codes + 4 float32 scales + 64 bf16 rope is the
reading the oracle states. The sparse MLA over packed rows is pinned to the (separately
pinned) bf16 sparse MLA on rows whose FP8 values are exact in bf16, and to closed forms.
"""
import json
import os

import numpy as np
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bf16_bits(x: torch.Tensor) -> np.ndarray:
    return x.to(torch.bfloat16).view(torch.uint16).numpy()


def test_row_bytes_match_pages():
    gold = json.load(open(os.path.join(GOLDEN, "mla_fp8_row.json")))
    lat = bf16_bits(torch.randn(3, 576))
    p = oracle.mla_fp8_pack(lat)
    assert p.shape == (3, gold["bytes_per_token_per_layer"])
    # the reading: one byte per latent value, a float32 per 128-value block, bf16 rope
    assert gold["kv_lora_rank"] + 4 * (gold["kv_lora_rank"] // 128) + 2 * gold["qk_rope_head_dim"] == 656
    m = gold["accepted_move"]
    mb = m["batch"] * m["accept_length"] * m["layers"] * gold["bytes_per_token_per_layer"] / 1e6
    assert abs(mb - m["printed_MB"]) <= m["printed_precision_MB"]


def test_pack_against_torch_float8():
    g = torch.Generator().manual_seed(5)
    # per-block magnitudes over many binades, with zeros and an all-zero block
    x = torch.randn(16, 576, generator=g) * torch.exp2(torch.randint(-12, 12, (16, 1), generator=g).float())
    x[3, 128:256] = 0.0
    x[5, 7] = 0.0
    lat = bf16_bits(x)
    xb = torch.from_numpy(lat.astype(np.int16)).view(torch.bfloat16).float()
    p = oracle.mla_fp8_pack(lat)
    for b in range(4):
        blk = xb[:, 128 * b:128 * (b + 1)]
        amax = blk.abs().amax(dim=1)
        sc = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))  # float32 division
        assert np.array_equal(p[:, 512 + 4 * b:516 + 4 * b].copy().view(np.float32)[:, 0], sc.numpy())
        codes = (blk / sc[:, None]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(p[:, 128 * b:128 * (b + 1)], codes)
    assert np.array_equal(p[:, 528:].copy().view(np.uint16), lat[:, 512:])
    # the largest value of each non-zero block takes the top code
    mags = p[:, :512].reshape(16, 4, 128) & 0x7F
    assert np.all((mags.max(axis=2) == 0x7E) | (xb[:, :512].abs().reshape(16, 4, 128).amax(2).numpy() == 0))


def test_values_within_fp8_rounding():
    g = torch.Generator().manual_seed(6)
    x = torch.randn(32, 576, generator=g) * 2.0
    lat = bf16_bits(x)
    xf = torch.from_numpy(lat.astype(np.int16)).view(torch.bfloat16).double().numpy()
    v = oracle.mla_fp8_values(oracle.mla_fp8_pack(lat))
    sc = np.repeat(oracle.mla_fp8_pack(lat)[:, 512:528].copy().view(np.float32).astype(np.float64), 128, 1)
    err = np.abs(v[:, :512] - xf[:, :512])
    # RNE on e4m3: half a step, 2^-4 relative on the normal grid, 2^-10 * scale below 2^-6 * scale
    assert np.all(err <= np.maximum(2.0 ** -4 * np.abs(xf[:, :512]), 2.0 ** -10 * sc) * (1 + 1e-6))
    assert np.array_equal(v[:, 512:], xf[:, 512:])


def _exact_rows(n, g):
    """Rows whose FP8 values are exact in bf16: each block's largest magnitude is 448 * 2^e
    (scale exactly 2^e) and every value is an e4m3 grid point times 2^e."""
    grid = oracle.fp8_decode(np.arange(0x7F, dtype=np.uint8))  # non-negative finite codes
    codes = torch.randint(0, 0x7F, (n, 512), generator=g).numpy()
    sign = np.where(torch.rand(n, 512, generator=g).numpy() < 0.5, -1.0, 1.0)
    e = torch.randint(-8, 4, (n, 4), generator=g).numpy()
    vals = sign * grid[codes] * np.repeat(2.0 ** e, 128, axis=1)
    for b in range(4):
        vals[:, 128 * b] = 448.0 * 2.0 ** e[:, b]
    rope = torch.randn(n, 64, generator=g)
    x = torch.cat([torch.from_numpy(vals).float(), rope], dim=1)
    return bf16_bits(x)


def test_sparse_mla_fp8_equals_bf16_oracle_on_exact_rows():
    g = torch.Generator().manual_seed(7)
    lengths = [40, 25, 61]
    ko = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    rows = 3
    qo = np.arange(0, rows * len(lengths) + 1, rows, dtype=np.int32)
    kv = _exact_rows(int(ko[-1]), g)
    kv8 = oracle.mla_fp8_pack(kv)
    assert np.array_equal(oracle.mla_fp8_values(kv8),
                          torch.from_numpy(kv.astype(np.int16)).view(torch.bfloat16).double().numpy())
    H, k = 16, 24
    q = bf16_bits(torch.randn(int(qo[-1]), H, 576, generator=g))
    topk = np.full((int(qo[-1]), k), -1, np.int32)
    for b, L in enumerate(lengths):
        for r in range(rows):
            sel = torch.randperm(L, generator=g)[:20].sort().values.numpy()
            topk[b * rows + r, :len(sel)] = sel
    topk[1, 3] = 10_000  # out of range: skipped by both
    o8, l8 = oracle.sparse_mla_fp8(q, kv8, topk, qo, ko, 0.0417)
    ob, lb = oracle.sparse_mla(q, kv, topk, qo, ko, 0.0417)
    assert np.array_equal(o8, ob) and np.array_equal(l8, lb)


def test_sparse_mla_fp8_single_key_and_empty():
    g = torch.Generator().manual_seed(8)
    kv = bf16_bits(torch.randn(10, 576, generator=g))
    kv8 = oracle.mla_fp8_pack(kv)
    vals = oracle.mla_fp8_values(kv8)
    q = bf16_bits(torch.randn(2, 16, 576, generator=g))
    qf = torch.from_numpy(q.astype(np.int16)).view(torch.bfloat16).double().numpy()
    topk = np.array([[4, -1, -1], [-1, -1, -1]], np.int32)
    qo = np.array([0, 2], np.int32)
    ko = np.array([0, 10], np.int64)
    o, lse = oracle.sparse_mla_fp8(q, kv8, topk, qo, ko, 0.5)
    # one selected key: the output is that row's values, lse its logit
    assert np.allclose(o[0], np.broadcast_to(vals[4, :512], (16, 512)), rtol=0, atol=1e-12)
    assert np.allclose(lse[0], 0.5 * qf[0] @ vals[4], rtol=1e-12, atol=1e-12)
    # nothing selected: zeros and -inf
    assert np.all(o[1] == 0.0) and np.all(np.isneginf(lse[1]))
