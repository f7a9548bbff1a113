"""FP8 latent cache: the GPU row pack and sparse MLA over packed rows, against the oracle.

Bars: packed rows (codes, scales, rope) are bit-exact; the sparse MLA over FP8 rows meets
the sparse-MLA tolerance (max|d| <= 2e-2*max|o| + 1e-2*|o| per row and head, |d lse| <=
1e-3) against the float64 oracle over the values the codes stand for. The GPU decode is
fed the oracle's packed rows, so its inputs never come from the HIP path.
"""
import numpy as np
import pytest
import torch

import oracle
from dsa_sparse_attention_amd import api, synth, workloads
from tests._pipeline import DEV, mla_check

pytestmark = pytest.mark.gpu

W = workloads


def _say(*a):
    print(*a, flush=True)


def u16(x):
    return x.view(torch.uint16).numpy()


def _latent_rows(n, seed):
    """bf16 latent rows over many binades per block, with an all-zero block and zeros."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(n, 576, generator=g)
    x[:, :512] *= torch.exp2(torch.randint(-10, 10, (n, 4), generator=g).float()).repeat_interleave(128, 1)
    x[0, 128:256] = 0.0
    x[1, 3] = 0.0
    x[2, 0] = -1e30  # a block whose largest magnitude is huge: its small values underflow
    return x.to(torch.bfloat16)


def test_pack_bitexact_and_scatter():
    _say("mla_fp8_pack bit-exact")
    lat = _latent_rows(1003, 1)
    ref = oracle.mla_fp8_pack(u16(lat))
    got = api.mla_fp8_pack(lat.to(DEV)).cpu().numpy()
    assert np.array_equal(got, ref)
    # scatter into cache rows dst: only those rows change
    cache = torch.full((2000, api.FP8_ROW_BYTES), 0xAB, dtype=torch.uint8, device=DEV)
    dst = torch.randperm(2000, generator=torch.Generator().manual_seed(2))[:1003].to(DEV)
    api.mla_fp8_pack(lat.to(DEV), cache, dst_rows=dst)
    c = cache.cpu().numpy()
    d = dst.cpu().numpy()
    assert np.array_equal(c[d], ref)
    rest = np.setdiff1d(np.arange(2000), d)
    assert np.all(c[rest] == 0xAB)


def _fp8_case(w, pad=0.0, rows=None, seed_offset=0):
    lens = synth.context_lengths(w)
    qo, ko = synth.q_row_offsets(w, rows), synth.kv_row_offsets(lens)
    m = synth.mla_inputs(w, lens, rows=rows, seed_offset=seed_offset)
    kv8 = oracle.mla_fp8_pack(u16(m["kv"]))
    return lens, qo, ko, m["q"], kv8


@pytest.mark.parametrize("heads,pad", [(16, 0.0), (64, 0.1), (128, 0.0), (48, 0.5), (112, 0.1)])
def test_sparse_mla_fp8_matches_oracle(heads, pad):
    _say(f"sparse_mla_fp8 heads={heads} pad={pad}")
    w = W.replace(W.scaled(W.MTP5_VERIFY, ctx=3000, batch=3, topk=512), mla_heads=heads)
    lens, qo, ko, q, kv8 = _fp8_case(w)
    idx = synth.random_topk(w, lens, qo, w.topk, pad_frac=pad)
    idx[1, :] = -1                     # a row with nothing selected
    idx[2, 5] = 10 ** 6                # out-of-range entry is skipped
    out, lse = api.sparse_mla_decode_fp8(q.to(DEV), torch.from_numpy(kv8).to(DEV), idx.to(DEV),
                                         qo.to(DEV), ko.to(DEV), w.rows, w.sm_scale)
    ref_o, ref_l = oracle.sparse_mla_fp8(u16(q), kv8, idx.numpy(), qo.numpy(), ko.numpy(), w.sm_scale)
    worst = mla_check(out, lse, ref_o, ref_l)
    assert torch.all(out[1] == 0) and torch.all(torch.isneginf(lse[1]))
    _say(f"  worst err/bound = {worst:.3f}")


@pytest.mark.parametrize("heads", [64, 128])
def test_sparse_mla_fp8_split_lists_and_workspace_reuse(heads):
    _say(f"sparse_mla_fp8 many rows heads={heads}")
    # 20 rows of k = 1024: few enough blocks that each list is split over 4 blocks, whose
    # partial results the combine kernel merges
    w = W.replace(W.scaled(W.MTP5_VERIFY, ctx=3000, batch=4, topk=1024), rows=5, mla_heads=heads)
    lens, qo, ko, q, kv8 = _fp8_case(w)
    idx = synth.random_topk(w, lens, qo, w.topk, pad_frac=0.2)
    idx[7, :] = -1
    T = int(qo[-1])
    need = api.sparse_mla_workspace_size(T, heads, w.topk)
    assert need > 0, "this case must split its lists"
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    ref_o, ref_l = oracle.sparse_mla_fp8(u16(q), kv8, idx.numpy(), qo.numpy(), ko.numpy(), w.sm_scale)
    kvd = torch.from_numpy(kv8).to(DEV)
    outs = []
    for call in range(2):
        out, lse = api.sparse_mla_decode_fp8(q.to(DEV), kvd, idx.to(DEV), qo.to(DEV), ko.to(DEV),
                                             w.rows, w.sm_scale, workspace=ws)
        _say(f"  call {call}: worst err/bound = {mla_check(out, lse, ref_o, ref_l):.3f}")
        outs.append((out.clone(), lse.clone()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_sparse_mla_fp8_index_share_and_dense():
    _say("sparse_mla_fp8 index share + dense")
    w = W.replace(W.scaled(W.DRAFT_SHARE, ctx=3000, batch=5, topk=256), rows=6)
    lens = synth.context_lengths(w)
    qo0, ko = synth.q_row_offsets(w), synth.kv_row_offsets(lens)
    step0 = synth.random_topk(w, lens, qo0, w.topk, pad_frac=0.05)
    n_acc = synth.accepted_lengths(w)
    qo1 = torch.arange(w.batch + 1, dtype=torch.int32)
    m = synth.mla_inputs(w, lens, rows=1, seed_offset=1)
    kv8 = oracle.mla_fp8_pack(u16(m["kv"]))
    d = lambda x: (torch.from_numpy(x) if isinstance(x, np.ndarray) else x).to(DEV)
    o_sh, l_sh = api.sparse_mla_decode_fp8(d(m["q"]), d(kv8), d(step0), d(qo1), d(ko), 1, w.sm_scale,
                                           share_base=d(qo0), num_accepted=d(n_acc))
    compact = step0[qo0[:-1].long() + n_acc.long()].contiguous()
    o_cp, l_cp = api.sparse_mla_decode_fp8(d(m["q"]), d(kv8), d(compact), d(qo1), d(ko), 1, w.sm_scale)
    assert torch.equal(o_sh, o_cp) and torch.equal(l_sh, l_cp)
    ref_o, ref_l = oracle.sparse_mla_fp8(u16(m["q"]), kv8, step0.numpy(), qo1.numpy(), ko.numpy(),
                                         w.sm_scale, share_base=qo0.numpy(), num_accepted=n_acc.numpy())
    mla_check(o_sh, l_sh, ref_o, ref_l)
    # k >= visible: every visible position of both requests
    w2 = W.replace(W.scaled(W.MTP5_VERIFY, ctx=700, batch=2, topk=1024), mla_heads=32)
    lens2 = [700, 333]
    qo, ko2 = synth.q_row_offsets(w2), synth.kv_row_offsets(lens2)
    m2 = synth.mla_inputs(w2, lens2)
    kv82 = oracle.mla_fp8_pack(u16(m2["kv"]))
    idx = synth.random_topk(w2, lens2, qo, w2.topk)
    out, lse = api.sparse_mla_decode_fp8(d(m2["q"]), d(kv82), d(idx), d(qo), d(ko2), w2.rows, w2.sm_scale)
    ref_o, ref_l = oracle.sparse_mla_fp8(u16(m2["q"]), kv82, idx.numpy(), qo.numpy(), ko2.numpy(),
                                         w2.sm_scale)
    mla_check(out, lse, ref_o, ref_l)


def test_fp8_errors():
    q = torch.zeros((2, 16, 576), dtype=torch.bfloat16, device=DEV)
    kv8 = torch.zeros((10, 656), dtype=torch.uint8, device=DEV)
    idx = torch.zeros((2, 4), dtype=torch.int32, device=DEV)
    qo = torch.tensor([0, 2], dtype=torch.int32, device=DEV)
    ko = torch.tensor([0, 10], dtype=torch.int64, device=DEV)
    with pytest.raises(ValueError):
        api.sparse_mla_decode_fp8(q, kv8[:, :600], idx, qo, ko, 2, 0.1)
    with pytest.raises(api.DsaError, match="UNSUPPORTED"):
        api.sparse_mla_decode_fp8(q[:, :8].contiguous(), kv8, idx, qo, ko, 2, 0.1)  # H = 8
    with pytest.raises(ValueError):  # dst_rows must give one row per latent row
        api.mla_fp8_pack(torch.zeros((3, 576), dtype=torch.bfloat16, device=DEV), kv8,
                         dst_rows=torch.zeros(2, dtype=torch.int64, device=DEV))
    # the C entry point refuses a misaligned cache (checked before any launch)
    from dsa_sparse_attention_amd import _lib
    lat = torch.zeros((3, 576), dtype=torch.bfloat16, device=DEV)
    rc = _lib.load().dsa_mla_fp8_pack(lat.data_ptr(), None, 3, kv8.data_ptr() + 8, None)
    assert rc == 1 and b"aligned" in _lib.load().dsa_last_error()
