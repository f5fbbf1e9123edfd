"""Property-based checks (hypothesis, tiny shapes, no GPU) of the oracle's
selection, attention, page2d coordinates and page-window schedule, and of the
C library's block pool against the oracle's schedule.

Each property follows from the method's definition (news.rkmt.cn/news/25027
Sec. 4-5; leheavengame.com OCR 2 release article, Sec. 2) independently of
the oracle's code: brute-force subset enumeration for the selection, textbook
softmax identities for the attention, stream concatenation for the
coordinates, membership and order invariants for the schedule."""
import itertools
import math
import os

import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle
from oracle import page_window as pw

SETTINGS = settings(max_examples=60, deadline=None, suppress_health_check=[HealthCheck.too_slow])


def _bf16(x):
    return (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


# ---------------------------------------------------------------- selection

@SETTINGS
@given(st.integers(0, 12), st.integers(1, 4), st.lists(st.integers(-4, 4), min_size=0, max_size=12),
       st.integers(0, 31))
def test_selection_is_the_best_subset(n_remote, local, score_ints, p_off):
    """The remote set is the size-R subset with the largest score sum, the
    lexicographically smallest ids among equal sums (scores with many exact
    ties); the local window is always kept; the output is ascending."""
    cfg = oracle.SparseCfg(topk_blocks=n_remote + local, local_blocks=local)
    ncand = len(score_ints)
    p = (ncand + local) * 32 - 1 - p_off if ncand + local > 0 else 0
    p = max(p, 0)
    ncand = oracle.candidate_count(p, cfg)
    scores = np.asarray(score_ints[:ncand], np.float32)
    sel = oracle.select_blocks(scores, p, cfg)
    local_ids = oracle.local_blocks(p, cfg)
    assert set(local_ids) <= set(sel["selected"])
    assert sel["selected"] == sorted(sel["selected"])
    assert len(sel["selected"]) == min(cfg.topk_blocks, p // 32 + 1)
    if ncand <= n_remote:
        assert sel["remote"] == list(range(ncand))
    else:
        best = None
        for comb in itertools.combinations(range(ncand), n_remote):
            key = (sum(int(score_ints[i]) for i in comb), [-i for i in comb])
            if best is None or key > best[0]:
                best = (key, list(comb))
        assert sel["remote"] == best[1]


# ---------------------------------------------------------------- attention

@SETTINGS
@given(st.integers(1, 3), st.integers(1, 40), st.integers(0, 2**31 - 1))
def test_attention_identities(heads, ntok, seed):
    """Constant V gives that constant; a permutation of the attended tokens
    changes nothing; one dominant logit gives that token's V; lse is the
    log-sum-exp of the scaled logits."""
    g = np.random.default_rng(seed)
    D = 8
    q = _bf16(g.standard_normal((heads, D)))
    k = _bf16(g.standard_normal((heads, ntok, D)))
    v = _bf16(g.standard_normal((heads, ntok, D)))
    toks = np.arange(ntok)
    out, lse = oracle.attend(q, k, v, toks, 0.5)
    perm = g.permutation(ntok)
    out_p, lse_p = oracle.attend(q, k[:, perm], v[:, perm], toks, 0.5)
    np.testing.assert_allclose(out_p, out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse_p, lse, rtol=0, atol=1e-12)
    qf = oracle.widen(q)
    kf = oracle.widen(k)
    for h in range(heads):
        z = 0.5 * (kf[h] @ qf[h])
        assert abs(lse[h] - (z.max() + math.log(np.exp(z - z.max()).sum()))) <= 1e-12
    cv = np.broadcast_to(_bf16(np.full(D, 1.5)), (heads, ntok, D)).copy()
    out_c, _ = oracle.attend(q, k, cv, toks, 0.5)
    np.testing.assert_allclose(out_c, 1.5, rtol=0, atol=1e-12)
    # token 0's key equals the query scaled up: its logit dominates
    kd = k.copy()
    kd[:, 0] = _bf16(oracle.widen(q) * 64.0)
    out_d, _ = oracle.attend(q, kd, v, toks, 1.0)
    vd = oracle.widen(v[:, 0])
    for h in range(heads):
        qq = float(qf[h] @ qf[h])
        if qq > 1.0:  # a margin of at least 63 in the logit
            np.testing.assert_allclose(out_d[h], vd[h], rtol=0, atol=1e-9 * max(1.0, np.abs(vd[h]).max()) +
                                       ntok * math.exp(-63 * qq / 2) * 10)


# ------------------------------------------------------ page2d coordinates

@SETTINGS
@given(st.lists(st.integers(0, 3), max_size=60), st.integers(0, 60), st.integers(0, 5), st.integers(-1, 9))
def test_page_coords_compose(stream, cut, page0, tok0):
    """Coordinates of a stream equal those of two chunks, the second started
    from the state the first ends in (marker id 3)."""
    marker = 3
    cut = min(cut, len(stream))
    t_all, p_all, s_all = oracle.page_coords(stream, marker, (page0, tok0))
    t1, p1, s1 = oracle.page_coords(stream[:cut], marker, (page0, tok0))
    t2, p2, s2 = oracle.page_coords(stream[cut:], marker, s1)
    assert list(t_all) == list(t1) + list(t2)
    assert list(p_all) == list(p1) + list(p2)
    assert tuple(s_all) == tuple(s2)
    # closed form: page = start page + markers so far; tok = distance to the last marker
    for i in range(len(stream)):
        n_mark = sum(1 for x in stream[:i + 1] if x == marker)
        assert p_all[i] == page0 + n_mark
        last = max([j for j in range(i + 1) if stream[j] == marker], default=None)
        assert t_all[i] == (i - last if last is not None else tok0 + i + 1)


# ----------------------------------------------------- page-window schedule

doc = st.integers(1, 9).flatmap(lambda n: st.tuples(
    st.lists(st.integers(0, 70), min_size=n, max_size=n), st.lists(st.integers(0, 70), min_size=n, max_size=n),
    st.integers(2, 5), st.sampled_from([0, 1, 31, 32, 33, 64])))


@SETTINGS
@given(doc)
def test_schedule_invariants(d):
    img, txt, W, tail = d
    r = oracle.page_window_schedule(img, txt, W, tail)
    final = r["final"]
    assert len(set(final)) == len(final)
    wins = pw.windows(len(img), W)
    assert len(r["window_peaks"]) == len(wins) and r["peak"] == max(r["window_peaks"])
    # the last window's pages are complete, images then text, at the end
    first, last = wins[-1]
    pages = pw.new_pages(len(wins) - 1, first, last)
    want = [("img", k, i) for k in pages for i in range(img[k])] + [("txt", k, i) for k in pages for i in range(txt[k])]
    assert final[len(final) - len(want):] == want
    # no window holds more blocks than everything appended so far
    seen = 0
    for w, (f, l) in enumerate(wins):
        for k in pw.new_pages(w, f, l):
            seen += img[k] + txt[k]
        assert r["window_peaks"][w] <= -(-seen // 32)


@pytest.fixture(scope="module")
def U():
    import block_sparse_long_sr_amd as U
    return U


@SETTINGS
@given(doc)
def test_c_pool_schedule_matches_oracle(U, d):
    img, txt, W, tail = d
    ref = oracle.page_window_schedule(img, txt, W, tail)
    pool = U.BlockPool(1024)
    assert pool.page_window_run(0, img, txt, W, tail) == ref["window_peaks"]
    row, length = pool.table(0, 1024)
    assert length == len(ref["final"]) and pool.peak == ref["peak"]
    live = [b for b in row if b >= 0]
    assert len(live) == -(-length // 32) == len(set(live))
