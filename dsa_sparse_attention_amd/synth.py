"""Seeded synthetic inputs for the DSA verify step.

This module draws inputs only: it holds none of the method's arithmetic
(no Hadamard, no quantisation, no scoring, no selection, no attention).
Both the HIP path and the CPU oracle are fed from here; everything is a
pure function of (workload, seed, device).

Distributions (the pages publish no dataset; these stand in for live
activations): indexer q/k and MLA q/latent ~ N(0, 1) (bf16 for MLA),
index-head weights ~ U(0, 1), logits ~ N(0, logits_std^2). Planted
structure:

* drafts: each request's accepted prefix length n is drawn from the chain
  law (each position matches with probability ``accept_rate``, stopping at
  the first miss); the logits row of every matched draft is planted so the
  draft token is its unique maximum, and the row at the first miss is
  planted so the draft token is its minimum. With accept_rate 0.6975 and 4
  drafts the mean accept length sum_i rate^i is 2.76, the GLM-5 figure
  quoted in "GLM-5.3 推理全链路(十四)", 草稿层一节.
* spikes (long-context workload): a fraction of each request's visible
  positions hold one identical key vector of norm 8*sqrt(D) along the
  direction of that request's w-weighted query sum, so all spikes carry the
  same FP8 bytes and scale and tie exactly.
"""
from __future__ import annotations

import math

import torch

from .workloads import DQK, Workload


def generator(seed: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def context_lengths(w: Workload) -> list[int]:
    """Cached positions per request (ragged when ctx_min > 0)."""
    if not w.ctx_min:
        return [w.ctx] * w.batch
    g = generator(w.seed * 7919 + 1)
    lens = torch.randint(w.ctx_min, w.ctx + 1, (w.batch,), generator=g)
    return [int(x) for x in lens]


def prefix(lengths, dtype=torch.int64) -> torch.Tensor:
    out = [0]
    for n in lengths:
        out.append(out[-1] + int(n))
    return torch.tensor(out, dtype=dtype)


def q_row_offsets(w: Workload, rows: int | None = None) -> torch.Tensor:
    r = w.rows if rows is None else rows
    return prefix([r] * w.batch, torch.int32)


def kv_row_offsets(lengths) -> torch.Tensor:
    return prefix(lengths, torch.int64)


def verify_cache_rows(lengths, rows) -> torch.Tensor:
    """Cache row of each verify row (int64 [sum rows]): row r of request b holds position
    L_b - R_b + r, i.e. the last R_b positions of the request's cached range."""
    rs = [rows] * len(lengths) if isinstance(rows, int) else list(rows)
    out, base = [], 0
    for L, R in zip(lengths, rs):
        out.extend(base + L - R + r for r in range(R))
        base += L
    return torch.tensor(out, dtype=torch.int64)


def indexer_inputs(w: Workload, lengths, device="cpu", rows: int | None = None,
                   seed_offset: int = 0) -> dict:
    """Float32 indexer q [T,H_I,D_I], k [N,D_I] and head weights w [T,H_I]."""
    r = w.rows if rows is None else rows
    T = w.batch * r
    N = int(sum(lengths))
    g = generator(w.seed * 1000 + 11 + seed_offset, device)
    q = torch.randn((T, w.index_heads, w.index_dim), generator=g, device=device)
    k = torch.randn((N, w.index_dim), generator=g, device=device)
    wt = torch.rand((T, w.index_heads), generator=g, device=device)
    out = dict(q=q, k=k, w=wt, spike_pos=None)
    if w.spike_frac > 0:
        out["spike_pos"] = plant_spikes(w, lengths, q, k, wt, r)
    return out


def indexer_queries(w: Workload, rows: int, seed_offset: int = 0, device="cpu") -> dict:
    """Float32 indexer queries q [B*rows,H_I,D_I] and head weights w [B*rows,H_I] alone, for
    rows scored against an existing key cache (the draft rows of a step without index
    sharing)."""
    T = w.batch * rows
    g = generator(w.seed * 1000 + 13 + seed_offset, device)
    q = torch.randn((T, w.index_heads, w.index_dim), generator=g, device=device)
    wt = torch.rand((T, w.index_heads), generator=g, device=device)
    return dict(q=q, w=wt)


def plant_spikes(w: Workload, lengths, q, k, wt, rows) -> list[torch.Tensor]:
    """Overwrite a fraction of each request's keys with one identical spike vector."""
    gcpu = generator(w.seed * 1000 + 23)
    kv_off = prefix(lengths)
    spikes = []
    for b, L in enumerate(lengths):
        n = int(math.floor(w.spike_frac * L))
        hi = L - rows + 1  # positions 0..L-rows are visible to every row of the request
        pos = torch.randperm(hi, generator=gcpu)[:n].sort().values
        qs = q[b * rows:(b + 1) * rows].double()            # [R, H, D]
        ws = wt[b * rows:(b + 1) * rows].double()[..., None]  # [R, H, 1]
        direction = (ws * qs).sum(dim=(0, 1))
        direction = direction / direction.norm()
        vec = (8.0 * math.sqrt(w.index_dim) * direction).float()
        k[int(kv_off[b]) + pos.to(k.device)] = vec.to(k.device)
        spikes.append(pos)
    return spikes


def mla_inputs(w: Workload, lengths, device="cpu", rows: int | None = None,
               seed_offset: int = 0, kv: torch.Tensor | None = None) -> dict:
    """bf16 MLA queries [T,H,576] and latent cache rows [N,576] (512 latent + 64 rope)."""
    r = w.rows if rows is None else rows
    T = w.batch * r
    N = int(sum(lengths))
    g = generator(w.seed * 1000 + 37 + seed_offset, device)
    q = torch.randn((T, w.mla_heads, DQK), generator=g, device=device).to(torch.bfloat16)
    if kv is None:
        kv = torch.empty((N, DQK), dtype=torch.bfloat16, device=device)
        chunk = 1 << 18
        for s in range(0, N, chunk):
            e = min(N, s + chunk)
            kv[s:e] = torch.randn((e - s, DQK), generator=g, device=device).to(torch.bfloat16)
    return dict(q=q, kv=kv)


def accepted_lengths(w: Workload, seed_offset: int = 0) -> torch.Tensor:
    """Planted accepted-draft counts per request (chain law, at most rows-1)."""
    g = generator(w.seed * 1000 + 41 + seed_offset)
    K = w.drafts
    u = torch.rand((w.batch, max(K, 1)), generator=g)
    hit = (u < w.accept_rate)[:, :K]
    n = torch.zeros(w.batch, dtype=torch.int32)
    for b in range(w.batch):
        c = 0
        while c < K and bool(hit[b, c]):
            c += 1
        n[b] = c
    return n


def accept_inputs(w: Workload, device="cpu") -> dict:
    """Logits [B*(K+1), V] (f32 or bf16), drafts [B, K] and the planted accepted counts."""
    K = w.drafts
    rows = w.batch * (K + 1)
    g = generator(w.seed * 1000 + 53, device)
    dt = torch.float32 if w.logits_dtype == "f32" else torch.bfloat16
    logits = (w.logits_std * torch.randn((rows, w.vocab), generator=g, device=device)).to(dt)
    gcpu = generator(w.seed * 1000 + 59)
    draft = torch.randint(0, w.vocab, (w.batch, K), generator=gcpu, dtype=torch.int32)
    n = accepted_lengths(w)
    hi = logits.float().amax(dim=1).cpu()
    lo = logits.float().amin(dim=1).cpu()
    for b in range(w.batch):
        for i in range(K):
            row = b * (K + 1) + i
            tok = int(draft[b, i])
            if i < int(n[b]):
                logits[row, tok] = float(hi[row]) + 1.0   # draft is the unique maximum
            elif i == int(n[b]):
                logits[row, tok] = float(lo[row]) - 1.0   # draft cannot be the maximum
                break
    return dict(logits=logits, draft=draft.to(device), planted_n=n)


def rejection_inputs(w: Workload, device="cpu", draft_noise: float = 1.0,
                     seed_offset: int = 0) -> dict:
    """Inputs of rejection-sampling acceptance: target logits [B*(K+1), V] (f32 or bf16,
    ~N(0, logits_std^2)); the draft model's probabilities [B, K, V] float32, taken as the
    normalised exponential of the target row plus N(0, draft_noise^2) noise (a draft law
    close to the target's, as a trained draft layer gives); the draft tokens drawn from
    those probabilities; the uniforms u [B, K] and us [B]."""
    K, B, V = w.drafts, w.batch, w.vocab
    g = generator(w.seed * 1000 + 71 + seed_offset, device)
    dt = torch.float32 if w.logits_dtype == "f32" else torch.bfloat16
    logits = (w.logits_std * torch.randn((B * (K + 1), V), generator=g, device=device)).to(dt)
    tgt = logits.float().view(B, K + 1, V)[:, :K]
    z = tgt + draft_noise * torch.randn((B, K, V), generator=g, device=device)
    z = torch.exp(z - z.amax(dim=-1, keepdim=True))
    probs = (z / z.sum(dim=-1, keepdim=True)).float().contiguous()
    # draft tokens: inverse CDF of the draft law (float64 running sums)
    c = probs.double().cumsum(dim=-1)
    pick = torch.rand((B, K, 1), generator=g, device=device, dtype=torch.float64) * c[..., -1:]
    draft = torch.searchsorted(c, pick, right=True).clamp_(max=V - 1).view(B, K).to(torch.int32)
    u = torch.rand((B, K), generator=g, device=device)
    us = torch.rand(B, generator=g, device=device)
    return dict(logits=logits, draft_probs=probs, draft=draft.contiguous(), u=u, us=us)


def random_topk(w: Workload, lengths, q_off, k: int, device="cpu", pad_frac: float = 0.0,
                seed_offset: int = 0) -> torch.Tensor:
    """Random ascending sets of distinct visible positions per row, -1 padded."""
    g = generator(w.seed * 1000 + 67 + seed_offset)
    T = int(q_off[-1])
    out = torch.full((T, k), -1, dtype=torch.int32)
    for b, L in enumerate(lengths):
        R = int(q_off[b + 1] - q_off[b])
        for r in range(R):
            vis = L - R + r + 1
            m = min(k, vis)
            if pad_frac > 0:
                m = max(0, m - int(pad_frac * m))
            pos = torch.randperm(vis, generator=g)[:m].sort().values
            out[int(q_off[b]) + r, :m] = pos.to(torch.int32)
    return out.to(device)


def random_scores(rows: int, width: int, seed: int, tie_levels: int = 0,
                  device="cpu") -> torch.Tensor:
    """Float32 score rows for standalone top-k cases; tie_levels>0 draws from few values."""
    g = generator(seed)
    if tie_levels > 0:
        s = torch.randint(0, tie_levels, (rows, width), generator=g).float() * 0.25
    else:
        s = torch.randn((rows, width), generator=g) * 40.0 + 150.0
    return s.to(device)
