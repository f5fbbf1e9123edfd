"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each check reaches the oracle's result by a different route than the oracle
itself: printed constants, hand-worked fixtures (tests/golden), brute-force
subset enumeration, exact integer arithmetic, the textbook dense causal
softmax attention, closed forms and invariants.  A plausible mistake in the
oracle (a dropped term, an off-by-one block or token bound, a reversed tie
rule, a wrong scale, a transposed operand) fails at least one of them; the
mutation tests at the end check that claim on planted mistakes.
"""
from __future__ import annotations

import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import logsumexp, softmax

import oracle
from oracle import SparseCfg
from synth import rng

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
CFG = SparseCfg()


def _bits(x):
    return rng.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def _read_pairs(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                k, *v = line.split()
                out[k] = v
    return out


def _read_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                rows.append([int(x) for x in line.split()])
    return rows


# --------------------------------------------------------------------------
# Printed constants and hand-worked bookkeeping
# --------------------------------------------------------------------------

def test_constants_match_pages():
    g = {k: int(v[0]) for k, v in _read_pairs("constants.txt").items()}
    assert CFG.block_size == g["block_size"]
    assert CFG.topk_blocks == g["topk_blocks"]
    assert CFG.local_blocks == g["local_blocks"]
    assert CFG.remote_slots == g["remote_blocks"]
    assert CFG.local_blocks * CFG.block_size == g["local_window_tokens"]
    assert CFG.topk_blocks * CFG.block_size == g["read_set_tokens"]
    assert CFG.num_heads == g["num_heads"] == g["num_kv_heads"]
    assert CFG.head_dim == g["head_dim"]
    assert CFG.index_dim == g["index_dim"]
    assert math.isclose(CFG.sm_scale, 1.0 / math.sqrt(g["head_dim"]))


@pytest.mark.parametrize("row", _read_rows("block_windows.txt"))
def test_block_windows_golden(row):
    p, nb, lo, hi, ncand, nkept = row
    assert oracle.block_count(p, CFG) == nb
    assert oracle.local_blocks(p, CFG) == list(range(lo, hi + 1))
    assert oracle.candidate_count(p, CFG) == ncand
    scores = np.random.default_rng(p).standard_normal(ncand).astype(np.float32)
    sel = oracle.select_blocks(scores, p, CFG)
    assert len(sel["selected"]) == nkept
    assert sel["selected"] == sorted(set(sel["selected"]))


def test_tie_break_golden():
    g = _read_pairs("tie_break.txt")
    p = int(g["p"][0])
    scores = np.array([float(x) for x in g["scores"]], np.float32)
    sel = oracle.select_blocks(scores, p, CFG)
    assert sel["remote"] == [int(x) for x in g["remote"]]
    assert sel["selected"] == [int(x) for x in g["selected"]]
    assert sel["cutoff"] == float(g["cutoff"][0])


# --------------------------------------------------------------------------
# Selection: brute force, invariants, special cases
# --------------------------------------------------------------------------

def _exact(x):
    return Fraction(float(x))


def brute_force_remote(scores, n_remote):
    """Subset of size n_remote with the largest exact sum; among equal sums the
    lexicographically smallest sorted id tuple.  Independent of sorting."""
    best, best_sum = None, None
    ex = [_exact(s) for s in scores]
    for comb in itertools.combinations(range(len(scores)), n_remote):
        s = sum(ex[i] for i in comb)
        if best_sum is None or s > best_sum or (s == best_sum and comb < best):
            best, best_sum = comb, s
    return list(best)


@pytest.mark.parametrize("seed", range(12))
def test_selection_brute_force(seed):
    g = np.random.default_rng(1000 + seed)
    ncand = int(g.integers(13, 19))          # C(18,12) = 18564 subsets
    p = (ncand + CFG.local_blocks) * CFG.block_size - 1 - int(g.integers(0, 32))
    assert oracle.candidate_count(p, CFG) == ncand
    if seed % 2:
        scores = g.integers(-3, 4, ncand).astype(np.float32)   # many exact ties
    else:
        scores = g.standard_normal(ncand).astype(np.float32)
    sel = oracle.select_blocks(scores, p, CFG)
    assert sel["remote"] == brute_force_remote(scores, CFG.remote_slots)
    assert sel["selected"] == sorted(sel["remote"] + oracle.local_blocks(p, CFG))


@pytest.mark.parametrize("p", [0, 5, 31, 100, 127, 128, 300, 511, 512, 777, 2047, 5000])
def test_local_always_kept_and_sizes(p):
    g = np.random.default_rng(p)
    ncand = oracle.candidate_count(p, CFG)
    scores = g.standard_normal(ncand).astype(np.float32) * 100
    sel = oracle.select_blocks(scores, p, CFG)
    nb = oracle.block_count(p, CFG)
    for j in range(max(0, nb - 4), nb):
        assert j in sel["selected"]
    assert len(sel["selected"]) == min(16, nb)
    assert all(0 <= j < nb for j in sel["selected"])


def test_small_context_keeps_everything():
    for p in range(0, 16 * 32):
        ncand = oracle.candidate_count(p, CFG)
        sel = oracle.select_blocks(np.zeros(ncand, np.float32), p, CFG)
        assert sel["selected"] == list(range(oracle.block_count(p, CFG)))
        assert sel["cutoff"] is None


def test_remote_are_the_highest():
    g = np.random.default_rng(7)
    p = 4096 * 32 - 1
    ncand = oracle.candidate_count(p, CFG)
    scores = g.standard_normal(ncand).astype(np.float32)
    sel = oracle.select_blocks(scores, p, CFG)
    kept = np.zeros(ncand, bool)
    kept[sel["remote"]] = True
    assert kept.sum() == 12
    assert scores[kept].min() > scores[~kept].max()


def test_nan_ranks_last_and_signed_zero_ties():
    p = 20 * 32 - 1    # 16 candidates
    s = np.full(16, -5.0, np.float32)
    s[3] = np.nan
    s[0] = -0.0
    s[1] = 0.0
    s[2] = -0.0
    sel = oracle.select_blocks(s, p, CFG)
    # 0, 1, 2 tie at zero; the NaN (id 3) is the only candidate left out
    # besides the highest ids among the -5 ties.
    assert 3 not in sel["remote"]
    assert sel["remote"][:3] == [0, 1, 2]
    assert sel["remote"] == [0, 1, 2] + list(range(4, 13))


# --------------------------------------------------------------------------
# Page-aware candidate ranking (optional tiers)
# --------------------------------------------------------------------------

def test_page_gate_golden():
    g = _read_pairs("page_gate.txt")
    for suf in ("", "2"):
        p = int(g["p" + suf][0])
        qpage = int(g["query_page" + suf][0])
        tags = [int(x) for x in g["tags" + suf]]
        scores = np.array([float(x) for x in g["scores" + suf]], np.float32)
        ncand = oracle.candidate_count(p, CFG)
        sel = oracle.select_blocks(scores, p, CFG, oracle.page_tiers(tags, qpage, ncand))
        assert sel["remote"] == [int(x) for x in g["remote" + suf]]
        if "selected" + suf in g:
            assert sel["selected"] == [int(x) for x in g["selected" + suf]]
        assert sel["cutoff"] == float(g["cutoff" + suf][0])
        assert sel["cutoff_tier"] == int(g["cutoff_tier" + suf][0])


def brute_force_remote_tiered(scores, tags, qpage, n_remote):
    """Subset of size n_remote maximising sum(score + M * [tag == qpage]) with a
    weight M larger than any difference of score sums, exact; among equal
    sums the lexicographically smallest sorted id tuple.  Independent of
    sorting and of the oracle's tier helper."""
    ex = [_exact(s) for s in scores]
    big = 2 * sum(abs(e) for e in ex) + 1
    w = [ex[i] + (big if tags[i] == qpage else 0) for i in range(len(scores))]
    best, best_sum = None, None
    for comb in itertools.combinations(range(len(scores)), n_remote):
        s = sum(w[i] for i in comb)
        if best_sum is None or s > best_sum or (s == best_sum and comb < best):
            best, best_sum = comb, s
    return list(best)


@pytest.mark.parametrize("seed", range(10))
def test_page_gate_brute_force(seed):
    g = np.random.default_rng(3000 + seed)
    ncand = int(g.integers(13, 18))
    p = (ncand + CFG.local_blocks) * CFG.block_size - 1 - int(g.integers(0, 32))
    assert oracle.candidate_count(p, CFG) == ncand
    # page tags: a few pages, -1 for blocks without image tokens; the query's
    # page tags fewer or more candidates than the 12 remote slots
    npages = int(g.integers(1, 4))
    tags = g.integers(-1, npages, ncand).tolist()
    qpage = int(g.integers(0, npages))
    if seed % 3 == 0:
        tags = [qpage if g.random() < 0.85 else -1 for _ in range(ncand)]
    if seed % 2:
        scores = g.integers(-3, 4, ncand).astype(np.float32)
    else:
        scores = g.standard_normal(ncand).astype(np.float32)
    sel = oracle.select_blocks(scores, p, CFG, oracle.page_tiers(tags, qpage, ncand))
    assert sel["remote"] == brute_force_remote_tiered(scores, tags, qpage, CFG.remote_slots)
    assert sel["selected"] == sorted(sel["remote"] + oracle.local_blocks(p, CFG))


@pytest.mark.parametrize("p", [700, 5000, 131071])
def test_page_gate_uniform_tiers_reduce_to_plain_ranking(p):
    g = np.random.default_rng(p)
    ncand = oracle.candidate_count(p, CFG)
    scores = g.standard_normal(ncand).astype(np.float32)
    plain = oracle.select_blocks(scores, p, CFG)
    for tags, qpage in (([3] * ncand, 3), ([-1] * ncand, 0), ([1] * ncand, 2)):
        gated = oracle.select_blocks(scores, p, CFG, oracle.page_tiers(tags, qpage, ncand))
        assert gated["selected"] == plain["selected"]
        assert gated["cutoff"] == plain["cutoff"]


def test_page_gate_in_page_blocks_first():
    g = np.random.default_rng(11)
    p = 4096 * 32 - 1
    ncand = oracle.candidate_count(p, CFG)
    scores = g.standard_normal(ncand).astype(np.float32)
    for n_in in (0, 5, 12, 40):
        tags = np.full(ncand, -1)
        tags[g.choice(ncand, n_in, replace=False)] = 4
        sel = oracle.select_blocks(scores, p, CFG, oracle.page_tiers(tags, 4, ncand))
        inpage = set(np.nonzero(tags == 4)[0].tolist())
        remote = set(sel["remote"])
        if n_in <= 12:
            assert inpage <= remote                       # all of the page's blocks kept
            rest = sorted(set(range(ncand)) - inpage, key=lambda j: (-scores[j], j))
            assert remote - inpage == set(rest[: 12 - n_in])   # fallback: best of the rest
        else:
            assert remote <= inpage                       # only the page's blocks
            best = sorted(inpage, key=lambda j: (-scores[j], j))[:12]
            assert remote == set(best)


def test_page_gate_prefill_rows_use_their_own_page():
    g = np.random.default_rng(21)
    S, T, q_start = 3000, 64, 2936
    ki = g.integers(-2, 3, (S, 128)).astype(np.float32)
    kib = (ki.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    qi = g.integers(-2, 3, (T, 128)).astype(np.float32)
    qib = (qi.view(np.uint32) >> 16).astype(np.uint16)
    q = np.zeros((T, 10, 128), np.uint16)
    k = np.zeros((10, S, 128), np.uint16)
    nblk = (S + 31) // 32
    tags = [(j * 32) // 1000 if (j * 32) % 1000 < 400 else -1 for j in range(nblk)]
    row_pages = [(q_start + t) // 1000 for t in range(T)]
    res = oracle.prefill_rows(q, qib, k, k, kib, q_start, [0, 63], CFG, tags, row_pages)
    for r in res:
        p = q_start + r["row"]
        ncand = oracle.candidate_count(p, CFG)
        one = oracle.decode_query(q[r["row"]], qib[r["row"]], k, k, kib, p + 1, CFG, tags, row_pages[r["row"]])
        assert r["selected"] == one["selected"]
        tiers = oracle.page_tiers(tags, row_pages[r["row"]], ncand)
        assert r["tiers"].tolist() == tiers.tolist()


# --------------------------------------------------------------------------
# Indexer scores and block maxima
# --------------------------------------------------------------------------

def test_indexer_scores_exact_integers():
    g = np.random.default_rng(3)
    q = g.choice([-2, -1, 1, 2], 128)          # no zero term can hide a dropped one
    k = g.choice([-2, -1, 1, 2], (97, 128))
    s = oracle.indexer_scores(_bits(q), _bits(k))
    for i in range(k.shape[0]):
        exact = sum(int(q[d]) * int(k[i, d]) for d in range(128))
        assert s[i] == np.float32(exact)
    assert s.dtype == np.float32


def test_indexer_scores_correctly_rounded():
    key = rng.stream_key(99, 1)
    q = rng.normal_bf16(key, np.arange(128))
    k = rng.normal_bf16(key, np.arange(128, 128 + 64 * 128)).reshape(64, 128)
    s = oracle.indexer_scores(q, k)
    qf = rng.bf16_bits_to_f32(q)
    kf = rng.bf16_bits_to_f32(k)
    for i in range(64):
        exact = sum(Fraction(float(qf[d])) * Fraction(float(kf[i, d])) for d in range(128))
        assert s[i] == np.float32(float(exact))


def test_block_maxima_loops():
    g = np.random.default_rng(11)
    p = 32 * 9 + 13
    scores = g.standard_normal(p + 40).astype(np.float32)
    scores[p + 1:] = 1e9          # past p: must not leak into any maximum
    bm = oracle.block_maxima(scores, p, 10, CFG)
    for j in range(10):
        m = -math.inf
        for t in range(32 * j, 32 * j + 32):
            if t <= p:
                m = max(m, float(scores[t]))
        assert bm[j] == np.float32(m)


def test_block_maxima_boundary_tokens():
    scores = np.zeros(32 * 6, np.float32)
    scores[31] = 5.0     # last token of block 0
    scores[32] = 7.0     # first token of block 1
    scores[95] = 3.0     # last token of block 2
    bm = oracle.block_maxima(scores, 32 * 6 - 1, 6, CFG)
    assert list(bm[:3]) == [5.0, 7.0, 3.0]


# --------------------------------------------------------------------------
# Attention: closed forms, dense equivalence, invariants
# --------------------------------------------------------------------------

def _rand_seq(seed, S, H=10, D=128, Di=128, values="normal"):
    key = rng.stream_key(seed, 77)
    f = rng.normal_bf16 if values == "normal" else rng.small_int_bf16
    n = 0

    def take(count):
        nonlocal n
        out = f(key, np.arange(n, n + count))
        n += count
        return out

    q = take(H * D).reshape(H, D)
    qi = take(Di)
    k = take(H * S * D).reshape(H, S, D)
    v = take(H * S * D).reshape(H, S, D)
    ki = take(S * Di).reshape(S, Di)
    return q, qi, k, v, ki


def dense_causal(q_bits, k_bits, v_bits, p):
    """Textbook causal attention of one query row at position p:
    softmax(q K^T / sqrt(d) + mask) V with the mask -inf on keys > p."""
    q = oracle.widen(q_bits)
    H, D = q.shape
    S = k_bits.shape[1]
    out = np.zeros((H, D))
    lse = np.zeros(H)
    mask = np.where(np.arange(S) <= p, 0.0, -np.inf)
    for h in range(H):
        logits = oracle.widen(k_bits[h]) @ q[h] / math.sqrt(D) + mask
        out[h] = softmax(logits) @ oracle.widen(v_bits[h])
        lse[h] = logsumexp(logits)
    return out, lse


def test_attention_closed_form():
    # one head, D=2, unit scale: logits 0, 1, 2 over three keys
    q = _bits([[1.0, 0.0]])
    k = _bits([[[0.0, 3.0], [1.0, -1.0], [2.0, 0.5]]])
    v = _bits([[[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]]])
    out, lse = oracle.attend(q, k, v, np.array([0, 1, 2]), 1.0)
    e = math.e
    z = 1 + e + e * e
    assert out[0, 0] == pytest.approx((1 + e * e) / z, rel=1e-15)
    assert out[0, 1] == pytest.approx((e + e * e) / z, rel=1e-15)
    assert lse[0] == pytest.approx(math.log(z), rel=1e-15)


def test_attention_equal_logits_lse():
    q = _bits(np.zeros((2, 8)))
    k = _bits(np.ones((2, 40, 8)))
    v = _bits(np.arange(2 * 40 * 8).reshape(2, 40, 8) % 7)
    toks = np.arange(0, 40, 3)
    out, lse = oracle.attend(q, k, v, toks, 0.25)
    assert np.allclose(lse, math.log(toks.size), rtol=0, atol=1e-14)
    want = oracle.widen(v)[:, toks, :].mean(axis=1)
    assert np.allclose(out, want, rtol=0, atol=1e-13)


@pytest.mark.parametrize("ctx", [1, 2, 31, 32, 33, 100, 200, 511, 512])
def test_dense_equivalence_small_context(ctx):
    """At most 16 blocks: the sparse result is dense causal attention."""
    q, qi, k, v, ki = _rand_seq(ctx, 512)
    r = oracle.decode_query(q, qi, k, v, ki, ctx, CFG)
    out, lse = dense_causal(q, k, v, ctx - 1)
    np.testing.assert_allclose(r["out"], out, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(r["lse"], lse, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("ctx", [2048, 1500, 1057])
def test_topk_all_equals_dense(ctx):
    q, qi, k, v, ki = _rand_seq(ctx + 5, 2048)
    nb = -(-ctx // 32)
    cfg = SparseCfg(topk_blocks=nb)
    r = oracle.decode_query(q, qi, k, v, ki, ctx, cfg)
    assert r["selected"] == list(range(nb))
    out, lse = dense_causal(q, k, v, ctx - 1)
    np.testing.assert_allclose(r["out"], out, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(r["lse"], lse, rtol=1e-12, atol=1e-12)


def test_sparse_equals_dense_over_kept_tokens():
    """Beyond 16 blocks: the result is the dense formula with every key outside
    the kept blocks masked, and differs from full dense attention."""
    ctx = 2048
    q, qi, k, v, ki = _rand_seq(5, ctx)
    r = oracle.decode_query(q, qi, k, v, ki, ctx, CFG)
    keep = np.zeros(ctx, bool)
    for j in r["selected"]:
        keep[32 * j: 32 * j + 32] = True
    qf = oracle.widen(q)
    for h in range(10):
        logits = oracle.widen(k[h]) @ qf[h] / math.sqrt(128) + np.where(keep, 0.0, -np.inf)
        want = softmax(logits) @ oracle.widen(v[h])
        np.testing.assert_allclose(r["out"][h], want, rtol=1e-12, atol=1e-12)
        assert r["lse"][h] == pytest.approx(logsumexp(logits), rel=1e-13)
    full, _ = dense_causal(q, k, v, ctx - 1)
    assert np.abs(full - r["out"]).max() > 1e-3


def test_token_count_invariant():
    for p in [511, 512, 600, 2047, 5000, 131071]:
        nb = p // 32 + 1
        ncand = max(0, nb - 4)
        sel = oracle.select_blocks(np.arange(ncand, dtype=np.float32), p, CFG)
        toks = oracle.attended_tokens(sel["selected"], p, CFG)
        if nb >= 16:
            assert toks.size == 15 * 32 + (p % 32) + 1
        assert toks.max() == p
        assert len(set(toks.tolist())) == toks.size


def test_constant_values_and_dominant_key():
    ctx = 3000
    q, qi, k, v, ki = _rand_seq(9, ctx)
    vc = np.full_like(v, _bits([1.5])[0])
    r = oracle.decode_query(q, qi, k, vc, ki, ctx, CFG)
    np.testing.assert_allclose(r["out"], 1.5, rtol=0, atol=1e-14)
    # a key of a kept block aligned with q and huge: output is that key's value
    sel = r["selected"]
    t = 32 * sel[3] + 7
    k2 = k.copy()
    k2[:, t, :] = _bits(oracle.widen(q) * 64.0)
    r2 = oracle.decode_query(q, qi, k2, v, ki, ctx, CFG)
    np.testing.assert_allclose(r2["out"], oracle.widen(v[:, t, :]), rtol=0, atol=1e-12)


def test_block_order_permutation_invariance():
    ctx = 2500
    q, qi, k, v, ki = _rand_seq(13, ctx)
    r = oracle.decode_query(q, qi, k, v, ki, ctx, CFG)
    p = ctx - 1
    sel = list(r["selected"])
    g = np.random.default_rng(1)
    perm = [sel[i] for i in g.permutation(len(sel))]
    toks = np.concatenate([np.arange(32 * j, min(32 * j + 32, p + 1)) for j in perm])
    out, lse = oracle.attend(q, k, v, toks, CFG.sm_scale)
    np.testing.assert_allclose(out, r["out"], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, r["lse"], rtol=1e-13, atol=1e-14)


def test_empty_context():
    q, qi, k, v, ki = _rand_seq(1, 64)
    r = oracle.decode_query(q, qi, k, v, ki, 0, CFG)
    assert r["selected"] == []
    assert np.all(r["out"] == 0) and np.all(np.isneginf(r["lse"]))


# --------------------------------------------------------------------------
# Prefill rows
# --------------------------------------------------------------------------

def test_prefill_rows_causal_and_dense():
    S, q_start, T = 640, 500, 140
    key = rng.stream_key(5, 9)
    qT = rng.normal_bf16(key, np.arange(T * 10 * 128)).reshape(T, 10, 128)
    qiT = rng.normal_bf16(key, np.arange(10**6, 10**6 + T * 128)).reshape(T, 128)
    _, _, k, v, ki = _rand_seq(21, S)
    rows = [0, 1, 11, 12, 13, 44, 139]
    res = oracle.prefill_rows(qT, qiT, k, v, ki, q_start, rows, CFG)
    for r in res:
        p = q_start + r["row"]
        assert r["tokens"].max() == p
        if p < 512:
            out, lse = dense_causal(qT[r["row"]], k, v, p)
            np.testing.assert_allclose(r["out"], out, rtol=1e-12, atol=1e-12)
    # keys after a row's position do not change that row
    k2, v2, ki2 = k.copy(), v.copy(), ki.copy()
    cut = q_start + 44 + 1
    k2[:, cut:, :] = 0x4000
    v2[:, cut:, :] = 0x4000
    ki2[cut:, :] = 0x4000
    a = oracle.prefill_rows(qT, qiT, k, v, ki, q_start, [44], CFG)[0]
    b = oracle.prefill_rows(qT, qiT, k2, v2, ki2, q_start, [44], CFG)[0]
    assert a["selected"] == b["selected"]
    np.testing.assert_array_equal(a["out"], b["out"])


# --------------------------------------------------------------------------
# Mutation checks: planted mistakes in a copy of the oracle's steps are caught
# --------------------------------------------------------------------------

def _mutants():
    import oracle.sr_swa as m

    def wrong_tie(scores, tiers=None):
        s = np.asarray(scores, np.float64)
        ids = np.arange(s.size)
        return np.lexsort((-ids, -np.nan_to_num(s), np.isnan(s)))

    def reversed_tiers(block_page, query_page, ncand):
        tags = np.asarray(block_page, dtype=np.int64)[:ncand]
        return (tags != int(query_page)).astype(np.int64)

    def off_by_one_tokens(selected, p, cfg):
        toks = []
        for j in sorted(selected):
            toks.extend(range(32 * j, min(32 * j + 32, p)))     # drops p itself
        return np.asarray(toks, np.int64)

    def no_scale_attend(q, k, v, tokens, scale):
        return ORIG["attend"](q, k, v, tokens, 1.0)

    def dropped_dim_scores(qb, kb):
        qf = m.widen(qb)
        kf = m.widen(kb)
        return (kf[:, :-1] @ qf[:-1]).astype(np.float32)

    def local_three(p, cfg):
        nb = m.block_count(p, cfg)
        return list(range(max(0, nb - 3), nb))

    return {
        "rank_candidates": wrong_tie,
        "attended_tokens": off_by_one_tokens,
        "attend": no_scale_attend,
        "indexer_scores": dropped_dim_scores,
        "local_blocks": local_three,
        "page_tiers": reversed_tiers,
    }


ORIG = {}


def _pins_pass():
    checks = [
        test_tie_break_golden,
        lambda: [test_block_windows_golden(r) for r in _read_rows("block_windows.txt")],
        lambda: test_dense_equivalence_small_context(100),
        lambda: test_selection_brute_force(1),
        test_indexer_scores_exact_integers,
        lambda: test_local_always_kept_and_sizes(2047),
        test_page_gate_golden,
        lambda: test_page_gate_brute_force(1),
    ]
    try:
        for c in checks:
            c()
    except AssertionError:
        return False
    return True


@pytest.mark.parametrize("name", sorted(_mutants().keys()))
def test_planted_mistake_is_caught(name, monkeypatch):
    import oracle.sr_swa as m
    ORIG["attend"] = m.attend
    mut = _mutants()[name]
    monkeypatch.setattr(m, name, mut)
    monkeypatch.setattr(oracle, name, mut)
    assert not _pins_pass(), f"a planted mistake in {name} went unnoticed"


def test_unmutated_oracle_passes_the_same_checks():
    assert _pins_pass()
