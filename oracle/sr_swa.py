"""SR-SWA block-sparse attention, step by step, on the CPU.

TEST INFRASTRUCTURE ONLY (see the package docstring): the plain reference the
HIP kernels are compared with.  Nothing here is blocked, fused or reordered
beyond what the method's own steps state.

The method ([rkmt] Sec. 5, steps 1-4; [lqnn] KV-cache section):

1. keys are grouped into blocks of ``block_size`` (32) consecutive tokens;
2. a one-head, 128-dim indexer scores every cached key against the query,
   and a block's score is the maximum over its keys;
3. the query keeps ``topk_blocks`` (16) blocks: its ``local_blocks`` (4) most
   recent blocks, and the highest-scoring remaining ("remote") blocks to fill
   the rest (12);
4. exact softmax attention runs over the tokens of the kept blocks only, for
   each of the 10 heads (128 dims, MHA, K already rotated).

Readings taken where the pages leave a point open:

* Score (open in [rkmt] Sec. 3/5): the plain dot product of the indexer query
  and indexer key, with no activation, weight or scale.  It is evaluated in
  float64 and rounded once to float32, the precision in which the kernels
  rank blocks.  bf16 x bf16 products are exact, so this is the correctly
  rounded float32 value of the dot product whenever the float64 sum is exact.
* Local window: block granular -- the block holding the query position p and
  the ``local_blocks - 1`` blocks before it.
* Remote blocks are chosen among the blocks before the local window only
  (the 16 kept blocks are distinct).
* Ranking: score descending, ties to the lower block index; a NaN score ranks
  below every number; -0.0 and +0.0 are equal.  If there are no more
  candidates than remote slots, all are kept.
* Causality: the query at position p sees keys 0..p, itself included.  Tokens
  of a kept block past p are not attended.
* Output order: kept block ids ascending.  Attention output in float64 with
  its log-sum-exp; over an empty token set the output is 0 and lse = -inf.
* Page-aware candidates (optional; [rkmt] Sec. 5 on the page-aware candidate
  constraint, [lehvn] Sec. 2 route A on the Page Gate): the candidate domain
  is the query's own page's image blocks plus the local window plus a global
  fallback.  Read as a two-tier ranking of the remote candidates: blocks that
  hold image tokens of the query's page come first (score descending, lower
  id first), and the other candidates fill the slots they leave, in the same
  order.  Block tags and the query's page are inputs.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Dict, List, Sequence

import numpy as np


@dataclass(frozen=True)
class SparseCfg:
    """Sparse-attention configuration; defaults are the released model's.

    block_size=32, topk_blocks=16, local_blocks=4 ([rkmt] Sec. 5 step 3;
    [lqnn] KV-cache section), 10 heads x 128 dims ([rkmt] Sec. 3), softmax
    scale 1/sqrt(128).
    """

    block_size: int = 32
    topk_blocks: int = 16
    local_blocks: int = 4
    num_heads: int = 10
    head_dim: int = 128
    index_dim: int = 128
    sm_scale: float = 1.0 / math.sqrt(128.0)

    @property
    def remote_slots(self) -> int:
        return self.topk_blocks - self.local_blocks


def widen(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def block_count(p: int, cfg: SparseCfg) -> int:
    """Number of blocks holding tokens 0..p ([rkmt] Sec. 5 step 1)."""
    return p // cfg.block_size + 1


def local_blocks(p: int, cfg: SparseCfg) -> List[int]:
    """The local window: the block holding p and the ones just before it."""
    nb = block_count(p, cfg)
    return list(range(max(0, nb - cfg.local_blocks), nb))


def candidate_count(p: int, cfg: SparseCfg) -> int:
    """Remote candidates are blocks 0 .. first local block - 1."""
    return max(0, block_count(p, cfg) - cfg.local_blocks)


def indexer_scores(q_idx_bits: np.ndarray, kidx_bits: np.ndarray) -> np.ndarray:
    """Indexer score of every key row ([rkmt] Sec. 5 step 2).

    q_idx_bits: [Di] bf16 bits; kidx_bits: [n, Di] bf16 bits -> float32 [n].
    """
    q = widen(q_idx_bits)
    k = widen(kidx_bits)
    return (k @ q).astype(np.float32)


def block_maxima(scores: np.ndarray, p: int, nblk: int, cfg: SparseCfg) -> np.ndarray:
    """Block score = max of the key scores in the block ([rkmt] Sec. 5 step 2).

    scores: float32 scores of tokens 0..(at least) the end of block nblk-1,
    index = token position.  Returns float32 [nblk]; tokens past p are not
    part of any block's maximum.
    """
    out = np.empty(nblk, dtype=np.float32)
    for j in range(nblk):
        lo = j * cfg.block_size
        hi = min(lo + cfg.block_size, p + 1)
        out[j] = np.max(scores[lo:hi])
    return out


def page_tiers(block_page: Sequence[int], query_page: int, ncand: int) -> np.ndarray:
    """Tier of each remote candidate under the page-aware constraint ([rkmt]
    Sec. 5; [lehvn] Sec. 2 route A): 1 for a block tagged with the query's
    page (it holds image tokens of that page), 0 for every other block."""
    tags = np.asarray(block_page, dtype=np.int64)[:ncand]
    return (tags == int(query_page)).astype(np.int64)


def rank_candidates(block_scores: np.ndarray, tiers=None) -> np.ndarray:
    """Candidate ids in rank order: score descending, lower id first on ties,
    NaN last ([rkmt] Sec. 5 step 3, with the tie rule stated above)."""
    s = np.asarray(block_scores, dtype=np.float64)
    ids = np.arange(s.size)
    is_nan = np.isnan(s)
    neg = np.where(is_nan, 0.0, -s)
    if tiers is None:
        # lexsort: last key is primary.
        return np.lexsort((ids, neg, is_nan)).astype(np.int64)
    # Page-aware: the tier (higher first) comes before everything else.
    neg_tier = -np.asarray(tiers, dtype=np.int64)[: s.size]
    return np.lexsort((ids, neg, is_nan, neg_tier)).astype(np.int64)


def select_blocks(block_scores: np.ndarray, p: int, cfg: SparseCfg, tiers=None) -> Dict[str, object]:
    """Kept blocks of the query at position p ([rkmt] Sec. 5 step 3).

    block_scores: float32 scores of the candidate blocks 0..ncand-1.
    tiers: optional page-aware tiers of the candidates (``page_tiers``).
    Returns a dict with ``selected`` (ascending ids), ``remote``, ``local``,
    ``ranked`` (candidates in rank order) and ``cutoff`` (score of the last
    remote block kept by ranking, or None when every candidate is kept; with
    tiers, ``cutoff_tier`` is that block's tier).
    """
    local = local_blocks(p, cfg)
    ncand = candidate_count(p, cfg)
    bs = np.asarray(block_scores, dtype=np.float32)[:ncand]
    ranked = rank_candidates(bs, tiers)
    cutoff_tier = None
    if ncand <= cfg.remote_slots:
        remote = list(range(ncand))
        cutoff = None
    else:
        remote = sorted(int(j) for j in ranked[: cfg.remote_slots])
        cutoff = float(bs[ranked[cfg.remote_slots - 1]])
        if tiers is not None:
            cutoff_tier = int(np.asarray(tiers)[ranked[cfg.remote_slots - 1]])
    return {
        "selected": sorted(remote + local),
        "remote": remote,
        "local": local,
        "ranked": ranked,
        "cutoff": cutoff,
        "block_scores": bs,
        "tiers": None if tiers is None else np.asarray(tiers, dtype=np.int64)[:ncand],
        "cutoff_tier": cutoff_tier,
    }


def attended_tokens(selected: Sequence[int], p: int, cfg: SparseCfg) -> np.ndarray:
    """Token positions of the kept blocks that the query at p may see."""
    toks: List[int] = []
    for j in sorted(selected):
        lo = j * cfg.block_size
        toks.extend(range(lo, min(lo + cfg.block_size, p + 1)))
    return np.asarray(toks, dtype=np.int64)


def attend(q_bits: np.ndarray, k_bits: np.ndarray, v_bits: np.ndarray,
           tokens: np.ndarray, scale: float):
    """Exact softmax attention over ``tokens`` in float64 ([rkmt] Sec. 5 step 4).

    q_bits [H, D]; k_bits, v_bits [H, n, D] (n >= max token + 1), bf16 bits.
    Returns (out [H, D] float64, lse [H] float64, natural log).
    """
    q = widen(q_bits)
    H, D = q.shape
    out = np.zeros((H, D), dtype=np.float64)
    lse = np.full(H, -np.inf, dtype=np.float64)
    if tokens.size == 0:
        return out, lse
    for h in range(H):
        k = widen(k_bits[h, tokens, :])
        v = widen(v_bits[h, tokens, :])
        z = (k @ q[h]) * scale
        m = np.max(z)
        w = np.exp(z - m)
        total = np.sum(w)
        out[h] = (w @ v) / total
        lse[h] = m + math.log(total)
    return out, lse


def decode_query(q_bits, q_idx_bits, k_bits, v_bits, kidx_bits, ctx_len: int,
                 cfg: SparseCfg = SparseCfg(), block_page=None, query_page=None):
    """One decode query of one sequence and layer, steps 1-4 in order.

    The query's own K/V are already in the cache, so it sits at
    p = ctx_len - 1.  k_bits/v_bits: [H, >=ctx_len, D]; kidx_bits:
    [>=ctx_len, Di]; q_bits [H, D]; q_idx_bits [Di].
    """
    return decode_query_fetch(q_bits, q_idx_bits, kidx_bits,
                              lambda toks: (k_bits[:, toks, :], v_bits[:, toks, :]), ctx_len, cfg,
                              block_page, query_page)


def decode_query_fetch(q_bits, q_idx_bits, kidx_bits, fetch_kv, ctx_len: int,
                       cfg: SparseCfg = SparseCfg(), block_page=None, query_page=None):
    """``decode_query`` with K/V supplied on demand.

    ``fetch_kv(tokens)`` returns (K, V) bf16 bits [H, len(tokens), D] of the
    given token positions; only the attended tokens are ever requested, so
    callers need not materialise a whole 128K-token cache.  With
    ``block_page`` (page tag per block, -1 for blocks without image tokens)
    and ``query_page`` the page-aware ranking is used.
    """
    H, D = np.asarray(q_bits).shape
    if ctx_len <= 0:
        return {"selected": [], "remote": [], "local": [], "out": np.zeros((H, D)), "lse": np.full(H, -np.inf),
                "block_scores": np.zeros(0, np.float32), "cutoff": None, "ranked": np.zeros(0, np.int64),
                "tokens": np.zeros(0, np.int64)}
    p = ctx_len - 1
    ncand = candidate_count(p, cfg)
    scores = indexer_scores(q_idx_bits, kidx_bits[: ncand * cfg.block_size])
    bscores = block_maxima(scores, p, ncand, cfg)
    tiers = None if block_page is None else page_tiers(block_page, query_page, ncand)
    sel = select_blocks(bscores, p, cfg, tiers)
    toks = attended_tokens(sel["selected"], p, cfg)
    k_rows, v_rows = fetch_kv(toks)
    out, lse = attend(q_bits, k_rows, v_rows, np.arange(toks.size), cfg.sm_scale)
    sel.update(out=out, lse=lse, tokens=toks)
    return sel


def prefill_rows(q_bits, q_idx_bits, k_bits, v_bits, kidx_bits, q_start: int,
                 rows: Sequence[int], cfg: SparseCfg = SparseCfg(), block_page=None, row_pages=None):
    """Chunked prefill: rows t of a chunk starting at q_start.

    Row t is the query at p = q_start + t; the chunk's own K/V are already in
    the cache and each row sees keys 0..p ([lehvn] Sec. 3 describes the
    chunked prefill; the per-row rule is the decode rule at that position).
    q_bits [T, H, D], q_idx_bits [T, Di].  ``row_pages[t]`` is row t's page
    when ``block_page`` turns the page-aware ranking on.  Returns one dict
    per row.
    """
    return prefill_rows_fetch(q_bits, q_idx_bits, kidx_bits,
                              lambda toks: (k_bits[:, toks, :], v_bits[:, toks, :]), q_start, rows, cfg,
                              block_page, row_pages)


def prefill_rows_fetch(q_bits, q_idx_bits, kidx_bits, fetch_kv, q_start: int,
                       rows: Sequence[int], cfg: SparseCfg = SparseCfg(), block_page=None, row_pages=None):
    """``prefill_rows`` with K/V supplied on demand (see decode_query_fetch)."""
    res = []
    for t in rows:
        qp = None if block_page is None else int(row_pages[t])
        r = decode_query_fetch(q_bits[t], q_idx_bits[t], kidx_bits, fetch_kv, q_start + t + 1, cfg,
                               block_page, qp)
        r["row"] = t
        res.append(r)
    return res
