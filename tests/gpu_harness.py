"""Shared GPU-test plumbing: run the HIP path through the C ABI, run the
oracle on the same seeded inputs (regenerated on the host), compare.

Tolerances (written here, used by every parity test):

* block scores: |gpu - oracle| <= gamma_127 * max over the block's keys of
  sum_d |q_d k_d| (+ the oracle's own float32 rounding of 1 ulp): the float32
  sum of 128 exact bf16 products in any order stays within this bound of the
  exact dot product (Higham, Accuracy and Stability of Numerical Algorithms,
  Sec. 3.1), and the block max is 1-Lipschitz.
* selection: equal sets, except blocks whose oracle score lies within 1e-4
  relative of the oracle's cutoff score (the ambiguity band), where either
  choice is accepted as long as both sets have the same size.  With page
  tiers the band holds only blocks of the cutoff block's tier.
* attention (given the same index set): max-abs <= 2e-3 and relative L2 <=
  1e-3 per query; lse within 1e-4 absolute.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional

import numpy as np
import torch

import block_sparse_long_sr_amd as U
import oracle
from synth import workloads as W

BAND = 1e-4
ATT_MAX_ABS = 2e-3
ATT_REL_L2 = 1e-3
LSE_ABS = 1e-4
GAMMA_127 = 127 * 2.0**-24 / (1 - 127 * 2.0**-24)


def cfg_for(wl: W.Workload, topk: int = 16, local: int = 4):
    return U.make_cfg(topk_blocks=topk, local_blocks=local, num_heads=wl.heads)


def ocfg(topk: int = 16, local: int = 4, heads: int = 10):
    return oracle.SparseCfg(topk_blocks=topk, local_blocks=local, num_heads=heads)


# ---------------------------------------------------------------- GPU side

def gpu_decode(dev, li: int, cfg, idx_override: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """Run the three decode entry points for resident layer li."""
    wl = dev.wl
    B, M, H, D = wl.batch, wl.max_blocks, wl.heads, wl.head_dim
    topk = cfg.topk_blocks
    kv = dev.kv(li)
    scores = torch.full((B, M), float("nan"), dtype=torch.float32, device="cuda")
    idx = torch.full((B, topk), -7, dtype=torch.int32, device="cuda")
    nsel = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    out = torch.full((B, H, D), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, H), float("nan"), dtype=torch.float32, device="cuda")
    U.indexer_score_decode(cfg, kv, dev.q_idx[li], scores)
    U.block_topk_decode(cfg, scores, dev.ctx_lens, B, M, idx, nsel)
    if idx_override is not None:
        idx_in = torch.from_numpy(np.ascontiguousarray(idx_override, dtype=np.int32)).cuda()
    else:
        idx_in = idx
    U.sparse_attn_decode(cfg, kv, dev.q[li], idx_in, out, lse)
    torch.cuda.synchronize()
    return {"scores": scores.cpu().numpy(), "idx": idx.cpu().numpy(), "nsel": nsel.cpu().numpy(),
            "out": out.cpu().numpy(), "lse": lse.cpu().numpy()}


def gpu_attn_decode(dev, li: int, cfg, idx_np: np.ndarray):
    wl = dev.wl
    out = torch.full((wl.batch, wl.heads, wl.head_dim), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((wl.batch, wl.heads), float("nan"), dtype=torch.float32, device="cuda")
    U.sparse_attn_decode(cfg, dev.kv(li), dev.q[li], torch.from_numpy(np.ascontiguousarray(idx_np, dtype=np.int32)).cuda(), out, lse)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def gpu_prefill(dev, cfg, idx_override: Optional[np.ndarray] = None, block_major: bool = True,
                fill=(0xA5, 0x5A)) -> Dict[str, np.ndarray]:
    """Scoring, merge and attention of a prefill chunk; the attention runs
    block-major (with its workspace) unless block_major is False.  The
    scoring and attention workspaces start filled with the bytes ``fill``
    (stale contents must not matter)."""
    wl = dev.wl
    T, M, H, D = wl.rows, wl.max_blocks, wl.heads, wl.head_dim
    topk = cfg.topk_blocks
    kv = dev.kv(0)
    ws_bytes = U.workspace_size(cfg, U.OP_INDEXER_PREFILL, T, M)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
    ws.fill_(fill[0])
    idx = torch.full((T, topk), -7, dtype=torch.int32, device="cuda")
    nsel = torch.full((T,), -7, dtype=torch.int32, device="cuda")
    out = torch.full((T, H, D), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    wsarg = (ws.data_ptr(), ws_bytes)
    U.indexer_score_prefill(cfg, kv, dev.q_idx, wl.q_start, T, wsarg)
    U.block_topk_prefill(cfg, wsarg, wl.q_start, T, M, idx, nsel)
    idx_in = idx if idx_override is None else torch.from_numpy(np.ascontiguousarray(idx_override, dtype=np.int32)).cuda()
    aws = None
    if block_major:
        ab = U.workspace_size(cfg, U.OP_ATTN_PREFILL, T, M)
        assert ab > 0
        aws = torch.empty(ab, dtype=torch.uint8, device="cuda")
        aws.fill_(fill[1])
    U.sparse_attn_prefill(cfg, kv, dev.q, wl.q_start, T, idx_in, out, lse, ws=aws)
    torch.cuda.synchronize()
    return {"idx": idx.cpu().numpy(), "nsel": nsel.cpu().numpy(), "out": out.cpu().numpy(),
            "lse": lse.cpu().numpy()}


# ------------------------------------------------------------- oracle side

def fetcher(wl: W.Workload, layer: int, seq: int):
    """K/V rows of given token positions, regenerated on the host."""
    def fetch(toks: np.ndarray):
        toks = np.asarray(toks, np.int64)
        return wl.kv_tokens(W.ROLE_K, layer, seq, toks), wl.kv_tokens(W.ROLE_V, layer, seq, toks)

    return fetch


def oracle_decode(wl: W.Workload, layer: int, seq: int, cfg=None, kidx=None):
    cfg = cfg or ocfg(heads=wl.heads)
    L = int(wl.ctx_lens[seq])
    if kidx is None:
        kidx = wl.kidx(layer, seq, 0, L)
    return oracle.decode_query_fetch(wl.q(layer, seq), wl.q_idx(layer, seq), kidx, fetcher(wl, layer, seq), L, cfg)


def oracle_attend_with(wl: W.Workload, layer: int, seq: int, q_bits, selected: List[int], p: int, cfg=None):
    cfg = cfg or ocfg(heads=wl.heads)
    toks = oracle.attended_tokens(selected, p, cfg)
    k, v = fetcher(wl, layer, seq)(toks)
    return oracle.attend(q_bits, k, v, np.arange(toks.size), cfg.sm_scale)


# ---------------------------------------------------------------- checks

def score_bound(q_idx_bits, kidx_bits, ncand: int) -> np.ndarray:
    """Per-block bound on |float32 dot - exact dot| (see module docstring)."""
    q = np.abs(oracle.widen(q_idx_bits))
    k = np.abs(oracle.widen(kidx_bits[: 32 * ncand]))
    per_key = k @ q
    per_blk = per_key.reshape(ncand, 32).max(axis=1) if ncand else np.zeros(0)
    return GAMMA_127 * per_blk


def check_scores(gpu_scores_row: np.ndarray, ref: Dict, q_idx_bits, kidx_bits, max_blocks: int):
    ncand = ref["block_scores"].size
    o = ref["block_scores"].astype(np.float64)
    g = gpu_scores_row[:ncand].astype(np.float64)
    tol = score_bound(q_idx_bits, kidx_bits, ncand) + np.abs(o) * 2.0**-23
    assert np.array_equal(np.isnan(g), np.isnan(o)), \
        f"NaN block scores differ: gpu {np.nonzero(np.isnan(g))[0][:8]} oracle {np.nonzero(np.isnan(o))[0][:8]}"
    bad = np.abs(g - o) > tol
    assert not bad.any(), f"{bad.sum()} block scores out of bound, first at {np.argmax(bad)}: gpu {g[bad][0]} oracle {o[bad][0]}"
    assert np.all(np.isneginf(gpu_scores_row[ncand:max_blocks])), "non-candidate entries must be -inf"


def check_selection(gpu_idx_row: np.ndarray, ref: Dict, topk: int):
    """Band rule; returns the set of blocks in the ambiguity band."""
    got = [int(x) for x in gpu_idx_row if x >= 0]
    assert list(gpu_idx_row[len(got):]) == [-1] * (topk - len(got)), f"padding: {gpu_idx_row}"
    assert got == sorted(got), f"not ascending: {got}"
    want = ref["selected"]
    band = set()
    if ref["cutoff"] is not None:
        c = ref["cutoff"]
        bs = ref["block_scores"].astype(np.float64)
        near = np.abs(bs - c) <= BAND * abs(c)
        if ref.get("tiers") is not None:   # page-aware: only the cutoff's own tier is ambiguous
            near &= ref["tiers"] == ref["cutoff_tier"]
        band = set(np.nonzero(near)[0].tolist())
    assert len(got) == len(want), f"size {len(got)} != {len(want)}"
    assert set(got) - band == set(want) - band, f"gpu {got} oracle {want} band {sorted(band)}"
    for j in ref["local"]:
        assert j in got
    return band


def check_attention(gpu_out: np.ndarray, gpu_lse: np.ndarray, ref_out: np.ndarray, ref_lse: np.ndarray):
    g = gpu_out.astype(np.float64)
    err = np.abs(g - ref_out).max() if g.size else 0.0
    nrm = np.linalg.norm(ref_out)
    rel = np.linalg.norm(g - ref_out) / nrm if nrm > 0 else np.linalg.norm(g)
    assert np.all(np.isfinite(g)), "non-finite attention output"
    assert err <= ATT_MAX_ABS, f"max-abs {err:.3e}"
    assert rel <= ATT_REL_L2, f"rel-L2 {rel:.3e}"
    fin = np.isfinite(ref_lse)
    assert np.all(np.isneginf(gpu_lse[~fin])), "lse of an empty set must be -inf"
    if fin.any():
        assert np.abs(gpu_lse[fin] - ref_lse[fin]).max() <= LSE_ABS
    return err, rel


def pad_idx(selected: List[int], topk: int) -> np.ndarray:
    a = np.full(topk, -1, np.int32)
    a[: len(selected)] = selected
    return a


def full_decode_check(dev, wl: W.Workload, li: int, layer: int, seqs, cfg_u, cfg_o, res=None):
    """Scores, selection, attention (oracle indices) and end-to-end checks for
    the given sequences of one layer.  Returns per-seq stats."""
    if res is None:
        res = gpu_decode(dev, li, cfg_u)
    topk = cfg_u.topk_blocks
    idx_oracle = np.full((wl.batch, topk), -1, np.int32)
    refs = {}
    for b in seqs:
        L = int(wl.ctx_lens[b])
        kidx = wl.kidx(layer, b, 0, L)
        ref = oracle.decode_query_fetch(wl.q(layer, b), wl.q_idx(layer, b), kidx, fetcher(wl, layer, b), L, cfg_o)
        refs[b] = ref
        check_scores(res["scores"][b], ref, wl.q_idx(layer, b), kidx, wl.max_blocks)
        check_selection(res["idx"][b], ref, topk)
        assert res["nsel"][b] == min(topk, -(-L // 32))
        idx_oracle[b] = pad_idx(ref["selected"], topk)
    out_o, lse_o = gpu_attn_decode(dev, li, cfg_u, idx_oracle)
    stats = {}
    for b in seqs:
        ref = refs[b]
        stats[b] = check_attention(out_o[b], lse_o[b], ref["out"], ref["lse"])
        got = [int(x) for x in res["idx"][b] if x >= 0]
        if got == ref["selected"]:
            check_attention(res["out"][b], res["lse"][b], ref["out"], ref["lse"])
        else:  # differs inside the band: the oracle recomputes with the GPU's set
            L = int(wl.ctx_lens[b])
            o2, l2 = oracle_attend_with(wl, layer, b, wl.q(layer, b), got, L - 1, cfg_o)
            check_attention(res["out"][b], res["lse"][b], o2, l2)
    return stats


# ------------------------------------------- full-size checks (D2H inputs)
# At the measured sizes the oracle takes the device inputs themselves, copied
# to the host (DeviceWorkload.host_*), instead of regenerating 135 GB of
# caches on the host; the device generator is pinned to the host generator
# bit for bit in test_synth / test_gpu_decode.

def oracle_decode_d2h(dev, li: int, b: int, cfg_o, block_page=None, query_page=None):
    """Oracle result of decode query (resident layer li, sequence b) on the
    device inputs; returns (ref, q, q_idx, kidx, fetch)."""
    L = int(dev.wl.ctx_lens[b])
    kidx = dev.host_kidx(li, b, L)
    q, qi = dev.host_decode_queries(li, b)
    fetch = dev.host_kv_fetch(li, b)
    ref = oracle.decode_query_fetch(q, qi, kidx, fetch, L, cfg_o, block_page, query_page)
    return ref, q, qi, kidx, fetch


def check_query_end_to_end(ref, q, fetch, p: int, cfg_o, idx_row, out, lse):
    """Selection under the band rule, then the GPU's attention output against
    the oracle's on the GPU's own set (the oracle's when they are equal)."""
    check_selection(idx_row, ref, cfg_o.topk_blocks)
    got = [int(x) for x in idx_row if x >= 0]
    if got == ref["selected"]:
        return check_attention(out, lse, ref["out"], ref["lse"]), got != ref["selected"]
    toks = oracle.attended_tokens(got, p, cfg_o)
    k, v = fetch(toks)
    o2, l2 = oracle.attend(q, k, v, np.arange(toks.size), cfg_o.sm_scale)
    return check_attention(out, lse, o2, l2), True


def check_decode_full(dev, res, queries, cfg_u, cfg_o, tags=None, qpages=None, scores=True):
    """Every (resident layer, sequence) in ``queries`` against the oracle on
    the device inputs: block scores (within the summation-order bound),
    selection (band rule), the GPU's attention on the GPU's selection and,
    per layer, the GPU's attention on the oracle's own index set.
    ``res``: host arrays idx [nl][B][topk], out [nl][B][H][D], lse
    [nl][B][H] and (with scores) scores [nl][B][M].  Returns a summary."""
    wl = dev.wl
    topk = cfg_u.topk_blocks
    by_layer: Dict[int, Dict[int, Dict]] = {}
    band_diffs = 0
    worst = [0.0, 0.0]
    for li, b in queries:
        bp = None if tags is None else tags[b]
        qp = None if qpages is None else int(qpages[b])
        ref, q, qi, kidx, fetch = oracle_decode_d2h(dev, li, b, cfg_o, bp, qp)
        L = int(wl.ctx_lens[b])
        if scores and L > 0:
            check_scores(res["scores"][li][b], ref, qi, kidx, wl.max_blocks)
        (err, rel), differs = check_query_end_to_end(ref, q, fetch, L - 1, cfg_o, res["idx"][li][b],
                                                     res["out"][li][b], res["lse"][li][b])
        band_diffs += int(differs)
        worst = [max(worst[0], err), max(worst[1], rel)]
        by_layer.setdefault(li, {})[b] = ref
    # the attention itself, measured with the oracle's index set
    for li, refs in by_layer.items():
        idx_o = np.full((wl.batch, topk), -1, np.int32)
        for b, ref in refs.items():
            idx_o[b] = pad_idx(ref["selected"], topk)
        out_o, lse_o = gpu_attn_decode(dev, li, cfg_u, idx_o)
        for b, ref in refs.items():
            err, rel = check_attention(out_o[b], lse_o[b], ref["out"], ref["lse"])
            worst = [max(worst[0], err), max(worst[1], rel)]
    return {"queries": len(queries), "band_differences": band_diffs, "max_abs": worst[0], "rel_l2": worst[1]}


def gpu_decode_step(dev, cfg, schedule, tags=None, qpages=None) -> Dict[str, np.ndarray]:
    """uocr_sparse_decode_step over every resident layer of dev (layer-major
    outputs, host copies); ``err`` is the workspace's error word after a
    one-launch call (the other schedules leave the workspace alone)."""
    wl = dev.wl
    nl, B, M, H, D = dev.q.shape[0], wl.batch, wl.max_blocks, wl.heads, wl.head_dim
    topk = cfg.topk_blocks
    bp = None if tags is None else torch.from_numpy(np.ascontiguousarray(tags, dtype=np.int32)).cuda()
    qp = None if qpages is None else torch.from_numpy(np.ascontiguousarray(qpages, dtype=np.int32)).cuda()
    kv = U.make_kv(dev.k[0], dev.v[0], dev.kidx[0], dev.block_table, dev.ctx_lens, wl.pool_blocks, B, M, bp, qp)
    scores = torch.full((nl, B, M), float("nan"), dtype=torch.float32, device="cuda")
    idx = torch.full((nl, B, topk), -7, dtype=torch.int32, device="cuda")
    nsel = torch.full((nl, B), -7, dtype=torch.int32, device="cuda")
    out = torch.full((nl, B, H, D), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((nl, B, H), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.zeros(U.workspace_size(cfg, U.OP_DECODE_STEP, nl * B, M), dtype=torch.uint8, device="cuda")
    U.sparse_decode_step(cfg, kv, nl, dev.q_idx, dev.q, scores, idx, out, lse, n_sel=nsel, ws=ws,
                         schedule=schedule)
    torch.cuda.synchronize()
    return {"scores": scores.cpu().numpy(), "idx": idx.cpu().numpy(), "nsel": nsel.cpu().numpy(),
            "out": out.cpu().numpy(), "lse": lse.cpu().numpy(),
            "err": int(ws[4:8].cpu().numpy().view(np.uint32)[0])}
