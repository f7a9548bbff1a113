"""Workload shapes of the DSA verify step (sizes only, no arithmetic).

Each workload fixes the ragged batch (requests, cached context per request,
verify rows per request), the indexer geometry (index heads x head dim,
top-k), the sparse-MLA head count (latent 512 + rope 64) and the vocabulary
for greedy acceptance. Page references:

* "MAX Pipeline 中的 DeepSeek-V3.2 架构实现解析", 配置体系: index_n_heads 64,
  index_head_dim 128, index_topk 2048.
* "GLM-5.3 推理全链路(十四)", 验证段: k+1 verify rows per request (6 rows for a
  5-step chain); 草稿层: kv_lora_rank 512, qk_rope_head_dim 64.
* "GLM-5.3 推理全链路(十四)", 索引器复用的收益与边界: draft steps reuse the
  step-0 top-k (index_share_for_mtp_iteration).
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

LATENT = 512
ROPE = 64
DQK = LATENT + ROPE


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    ctx: int                   # cached positions per request (includes its verify rows)
    rows: int                  # verify rows per request (bonus + drafts = k+1)
    index_heads: int
    index_dim: int
    topk: int
    mla_heads: int
    vocab: int
    seed: int
    ctx_min: int = 0           # >0: ragged contexts drawn uniformly in [ctx_min, ctx]
    logits_dtype: str = "bf16"  # "f32" or "bf16"
    logits_std: float = 2.0
    spike_frac: float = 0.0    # fraction of positions per request holding planted spike keys
    share_steps: int = 0       # draft steps reusing the step-0 top-k (one row per request each)
    accept_rate: float = 0.6975  # planted per-position draft match probability
    description: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def drafts(self) -> int:
        return self.rows - 1

    @property
    def sm_scale(self) -> float:
        return 1.0 / DQK ** 0.5


TINY = Workload(
    name="tiny", batch=1, ctx=4096, rows=2, index_heads=8, index_dim=64, topk=256,
    mla_heads=16, vocab=1024, seed=0, logits_dtype="f32", logits_std=1.0,
    description="1 request, context 4096, 2 verify rows, indexer 8x64, top-k 256, MLA 16 heads")

DECODE_VERIFY = Workload(
    name="decode_verify", batch=8, ctx=16384, rows=2, index_heads=64, index_dim=128,
    topk=2048, mla_heads=128, vocab=151552, seed=2,
    description="8 requests x 16384 context, 2 verify rows, indexer 64x128, MLA 128 heads")

MTP5_VERIFY = Workload(
    name="mtp5_verify", batch=32, ctx=65536, ctx_min=8192, rows=6, index_heads=64,
    index_dim=128, topk=2048, mla_heads=64, vocab=151552, seed=3,
    description="32 requests, ragged contexts U[8K,64K], 6 verify rows, MLA 64 heads, "
                "greedy accept over 151552 bf16 logits N(0,4)")

MTP5_VERIFY_64K = replace(
    MTP5_VERIFY, name="mtp5_verify_64k", ctx_min=0, seed=33,
    description="32 requests x 65536 context, 6 verify rows, indexer 64x128 FP8, top-k 2048, "
                "MLA 64 heads, greedy accept over 151552 bf16 logits N(0,4)")

DRAFT_SHARE = Workload(
    name="draft_share", batch=64, ctx=32768, rows=6, index_heads=64, index_dim=128,
    topk=2048, mla_heads=64, vocab=151552, seed=4, share_steps=4,
    description="64 requests x 32768 context; step 0 scores 6 rows/request, then 4 draft "
                "steps of 1 row/request reuse the step-0 top-k at the accepted position")

LONG_CTX = Workload(
    name="long_ctx", batch=4, ctx=262144, rows=6, index_heads=64, index_dim=128,
    topk=2048, mla_heads=128, vocab=151552, seed=5, spike_frac=0.01,
    description="4 requests x 262144 context, 6 verify rows, MLA 128 heads, 1% planted "
                "identical high-score spike keys per request")

ALL = {w.name: w for w in (TINY, DECODE_VERIFY, MTP5_VERIFY, MTP5_VERIFY_64K, DRAFT_SHARE,
                           LONG_CTX)}


def scaled(w: Workload, ctx: int, batch: int | None = None, name: str | None = None,
           **kw) -> Workload:
    """Same geometry at a smaller context (for CPU-sized parity cases)."""
    ctx_min = 0 if not w.ctx_min else max(w.rows, ctx // 8)
    return replace(w, ctx=ctx, ctx_min=ctx_min, batch=batch or w.batch,
                   name=name or f"{w.name}@{ctx}", **kw)
