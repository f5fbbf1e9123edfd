"""The page-window schedule of continuous decoding on the GPU caches
(leheavengame.com OCR 2 release article, Sec. 2 route A, storage half): a
document streams through the cache write window by window, the block pool
releases and compacts at each window boundary (a rewrite of the block-table
row, no cache data moves), and the sparse decode path then runs on the
compacted cache.  Checked against the oracle's schedule and the oracle's
decode query over the kept tokens, rotated on the host."""
from __future__ import annotations

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import block_sparse_long_sr_amd as U  # noqa: E402
import oracle  # noqa: E402
import gpu_harness as G  # noqa: E402

H, D = 10, 128


def _bf16(g, shape):
    return (g.standard_normal(shape).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _dev(a):
    a = np.ascontiguousarray(a)
    return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).cuda()


def test_decode_on_caches_compacted_by_the_page_window_schedule():
    g = np.random.default_rng(0x5E)
    n_pages, Wp, tail = 11, 4, 48
    img = g.integers(20, 140, n_pages).tolist()
    txt = g.integers(10, 120, n_pages).tolist()
    img[5] = 0                                          # a page without image tokens
    # one K/V/indexer-K row per token of the document, in first-append order
    labels = [("img", k, i) for k in range(n_pages) for i in range(img[k])]
    labels += [("txt", k, i) for k in range(n_pages) for i in range(txt[k])]
    row_of = {lab: r for r, lab in enumerate(labels)}
    kn, vn, ixn = _bf16(g, (len(labels), H, D)), _bf16(g, (len(labels), H, D)), _bf16(g, (len(labels), D))

    def coords(lab):  # page2d: page number, offset inside the page (its image, then its text)
        kind, k, i = lab
        return (i if kind == "img" else img[k] + i), k

    full = oracle.page_window_schedule(img, txt, Wp, tail)
    P = M = full["peak"] + 3
    pool = U.BlockPool(P)
    dk = torch.zeros((P, H, 32, D), dtype=torch.int16, device="cuda")
    dv = torch.zeros_like(dk)
    di = torch.zeros((P, 32, D), dtype=torch.int16, device="cuda")
    dtab = torch.full((1, M), -1, dtype=torch.int32, device="cuda")
    dctx = torch.zeros(1, dtype=torch.int32, device="cuda")
    kv = U.make_kv(dk, dv, di, dtab, dctx, P, 1, M)
    cfg = U.make_cfg()
    held = []

    def upload_table():
        row, length = pool.table(0, M)
        dtab.copy_(torch.tensor(row, dtype=torch.int32).view(1, M))
        dctx.fill_(length)
        return length

    def append(labs):
        before = pool.table(0, M)[1]
        pool.append(0, len(labs))
        after = upload_table()
        if not labs:
            return
        rows = [row_of[lab] for lab in labs]
        tp, pp = zip(*[coords(lab) for lab in labs])
        args = [_dev(np.asarray(a, np.int32)) for a in (np.zeros(len(labs)), np.arange(before, after), tp, pp)]
        args += [_dev(kn[rows]), _dev(vn[rows]), _dev(ixn[rows])]
        held.extend(args)
        U.rope_cache_write(cfg, kv, len(labs), *args)

    def decode_and_check(window_last):
        L = upload_table()
        # the oracle's token list at this point: the schedule run on the pages seen so far
        seq = oracle.page_window_schedule(img[:window_last], txt[:window_last], Wp, tail)["final"]
        assert len(seq) == L
        q, qi = _bf16(g, (1, H, D)), _bf16(g, (1, D))
        qt, qp = coords(seq[-1])
        dq, dqi = _dev(q), _dev(qi)
        U.rope_queries(cfg, 1, _dev(np.array([qt], np.int32)), _dev(np.array([qp], np.int32)), q=dq, q_idx=dqi)
        scores = torch.empty((1, M), dtype=torch.float32, device="cuda")
        idx = torch.empty((1, 16), dtype=torch.int32, device="cuda")
        out = torch.empty((1, H, D), dtype=torch.float32, device="cuda")
        lse = torch.empty((1, H), dtype=torch.float32, device="cuda")
        U.indexer_score_decode(cfg, kv, dqi, scores)
        U.topk_attn_decode(cfg, kv, dq, scores, idx, out, lse)
        torch.cuda.synchronize()
        rows = [row_of[lab] for lab in seq]
        k_rot = np.stack([oracle.rope_page2d(kn[r], *coords(lab)) for r, lab in zip(rows, seq)], axis=1)
        v_all = np.transpose(vn[rows], (1, 0, 2))
        ix_rot = np.stack([oracle.rope_page2d(ixn[r], *coords(lab)) for r, lab in zip(rows, seq)])
        ref = oracle.decode_query(oracle.rope_page2d(q[0], qt, qp), oracle.rope_page2d(qi[0], qt, qp),
                                  k_rot, v_all, ix_rot, L)
        G.check_scores(scores.cpu().numpy()[0], ref, oracle.rope_page2d(qi[0], qt, qp), ix_rot, M)
        G.check_selection(idx.cpu().numpy()[0], ref, 16)
        got = sorted(int(x) for x in idx.cpu().numpy()[0] if x >= 0)
        toks = oracle.attended_tokens(got, L - 1, G.ocfg())
        want_o, want_l = oracle.attend(oracle.rope_page2d(q[0], qt, qp), k_rot, v_all, toks, G.ocfg().sm_scale)
        G.check_attention(out.cpu().numpy()[0], lse.cpu().numpy()[0], want_o, want_l)

    wins = oracle.page_window.windows(n_pages, Wp)
    assert len(wins) >= 3
    for w, (first, last) in enumerate(wins):
        print(f"case: page window {w} pages [{first}, {last})", flush=True)
        pages = oracle.page_window.new_pages(w, first, last)
        shared_lo = shared_hi = None
        for k in pages:
            if k == last - 1:
                shared_lo = pool.table(0, M)[1]
            append([("img", k, i) for i in range(img[k])])
            if k == last - 1:
                shared_hi = pool.table(0, M)[1]
        for k in pages:
            append([("txt", k, i) for i in range(txt[k])])
        decode_and_check(last)
        if w + 1 < len(wins):
            end = pool.table(0, M)[1]
            pool.keep(0, [(shared_lo, shared_hi), (max(shared_hi, end - tail), end)])
    assert pool.peak == full["peak"] and pool.table(0, M)[1] == len(full["final"])
