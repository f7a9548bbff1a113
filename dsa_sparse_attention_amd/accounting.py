"""Algorithmic work of each stage of the verify step (bytes and flops).

These are the bytes the method must move and the flops it must do, not what
a kernel happens to read: they are the numerators of the roofline fractions.

* Indexer keys: index_head_dim FP8 bytes per cached token per full indexer
  layer ("GLM-5.3 推理全链路(十四)", 附:长上下文下草稿段的索引器账, where one
  draft round without sharing reads 4*21*128*L bytes and with sharing
  21*128*L), plus the 4-byte per-token fp32 scale ("MAX Pipeline 中的
  DeepSeek-V3.2 架构实现解析", 配置体系: per-token fp32 scale cache).
* Sparse MLA: one 576-wide bf16 latent row gathered per selected position
  per query row ("GLM-5.3 推理全链路(十四)", 草稿前向的逐层算子: b queries
  against 2048 KV).
"""
from __future__ import annotations

from .workloads import DQK, LATENT


def index_key_bytes(context: int, index_dim: int = 128, full_layers: int = 1,
                    forwards: int = 1) -> int:
    """FP8 indexer-key bytes streamed by ``forwards`` forwards over ``full_layers`` layers."""
    return forwards * full_layers * index_dim * context


def draft_round_index_bytes(context: int, index_dim: int = 128, full_layers: int = 21,
                            draft_forwards: int = 4, share: bool = True) -> int:
    """Indexer reads of one draft round, with or without index_share_for_mtp_iteration."""
    return index_key_bytes(context, index_dim, full_layers, 1 if share else draft_forwards)


def merged_offsets(input_row_offsets, K: int) -> list[int]:
    """Ragged offsets after appending K drafts per request: off[i] + i*K.

    ("MAX 推测解码配置指南解读 max.pipelines.speculative", Token 合并.)
    """
    return [int(o) + i * K for i, o in enumerate(input_row_offsets)]


def index_score_work(lengths, rows: int, heads: int, dim: int) -> dict:
    """Bytes/flops of dsa_index_score for one batch.

    bytes: keys + scales once per request, q codes + q scale + w per row, and the
    fp32 score of every visible (row, key) written once.
    flops: 2*heads*dim per visible (row, key) pair (the FP8 contraction).
    """
    kbytes = sum(L * (dim + 4) for L in lengths)
    qbytes = len(lengths) * rows * heads * (dim + 8)
    pairs = sum(sum(L - rows + r + 1 for r in range(rows)) for L in lengths)
    return dict(bytes=kbytes + qbytes + 4 * pairs, flops=2 * heads * dim * pairs, pairs=pairs)


def topk_work(lengths, rows: int, k: int) -> dict:
    """Bytes of dsa_topk: each visible score read once, k indices written per row."""
    pairs = sum(sum(L - rows + r + 1 for r in range(rows)) for L in lengths)
    return dict(bytes=4 * pairs + 4 * k * rows * len(lengths), flops=0)


def index_topk_work(lengths, rows: int, heads: int, dim: int, k: int) -> dict:
    """Bytes/flops of dsa_index_topk for one batch: the index scoring's key, scale and query
    reads and its contraction, and the k indices written per row (no score rows)."""
    wi = index_score_work(lengths, rows, heads, dim)
    nrows = len(lengths) * rows
    return dict(bytes=wi["bytes"] - 4 * wi["pairs"] + 4 * k * nrows, flops=wi["flops"],
                pairs=wi["pairs"])


FP8_ROW_BYTES = 656  # FP8 latent cache row ("GLM-5.3 推理全链路(十四)": 656 B/token/layer)


def sparse_mla_work(n_rows: int, heads: int, k: int, selected_per_row=None,
                    row_bytes: int = DQK * 2) -> dict:
    """Bytes/flops of dsa_sparse_mla_decode (row_bytes 1152, bf16 rows) or of
    dsa_sparse_mla_decode_fp8 (row_bytes FP8_ROW_BYTES).

    bytes: one latent row per selected position, q and out per (row, head), 4-byte
    indices and the fp32 lse. flops: QK^T over 576 dims plus PV over 512.
    """
    sel = n_rows * k if selected_per_row is None else int(selected_per_row)
    bytes_ = sel * row_bytes + n_rows * heads * (DQK * 2 + LATENT * 2 + 4) + n_rows * k * 4
    flops = 2 * heads * sel * (DQK + LATENT)
    return dict(bytes=bytes_, flops=flops)


def greedy_accept_work(batch: int, drafts: int, vocab: int, elem_bytes: int) -> dict:
    rows = batch * (drafts + 1)
    return dict(bytes=rows * vocab * elem_bytes + batch * drafts * 4 + batch * 8, flops=0)


def rejection_accept_work(batch: int, drafts: int, vocab: int, elem_bytes: int) -> dict:
    """Every logits row once (softmax statistics), and the draft law of each request's
    drawing row once (the corrected weights); the drafts, uniforms and outputs."""
    rows = batch * (drafts + 1)
    return dict(bytes=rows * vocab * elem_bytes + batch * vocab * 4 + batch * drafts * 12 +
                batch * 12, flops=0)
