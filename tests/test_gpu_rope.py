"""GPU parity of the page2d rotary encoding and the KV-cache write
(news.rkmt.cn/news/25027 Sec. 4 and Sec. 6) against the CPU oracle, through
the C ABI: bit-exact pools and queries, out-of-range tokens skipped, and the
sparse decode path run on caches the cache write produced."""
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


def _dev(a, dtype=None):
    a = np.ascontiguousarray(a)
    t = torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a)
    return t.cuda()


def test_cache_write_and_queries_bit_exact():
    g = np.random.default_rng(11)
    P, B, M = 48, 4, 12
    table = g.permutation(P)[: B * M].reshape(B, M).astype(np.int32)
    table[2, 5] = -1                                      # an unmapped block: its tokens are skipped
    n = 300
    seq = g.integers(0, B, n).astype(np.int32)
    pos = g.integers(0, M * 32, n).astype(np.int32)
    # one writer per (seq, pos) slot
    _, first = np.unique(seq.astype(np.int64) * 100000 + pos, return_index=True)
    keep = np.zeros(n, bool)
    keep[first] = True
    seq, pos = seq[keep], pos[keep]
    n = seq.size
    seq[:3] = [-1, B, 1]                                  # out-of-range sequence ids
    pos[2] = M * 32                                       # out-of-range position
    tok = g.integers(0, 3000, n).astype(np.int32)
    tok[:8] = [0, 1, 2, 63, 64, 999, 131071, 5]
    page = g.integers(0, 200, n).astype(np.int32)
    kn, vn, ixn = _bf16(g, (n, H, D)), _bf16(g, (n, H, D)), _bf16(g, (n, D))
    kp = np.zeros((P, H, 32, D), np.uint16)
    vp = np.zeros_like(kp)
    ip = np.zeros((P, 32, D), np.uint16)
    for t in range(n):
        if not (0 <= seq[t] < B and 0 <= pos[t] < M * 32) or table[seq[t], pos[t] // 32] < 0:
            continue
        oracle.cache_write(kp, vp, ip, table, int(seq[t]), int(pos[t]), kn[t], vn[t], ixn[t], int(tok[t]),
                           int(page[t]))
    print("case: cache write", n, "tokens", flush=True)
    dk, dv, di = (torch.zeros(x.shape, dtype=torch.int16, device="cuda") for x in (kp, vp, ip))
    # the descriptor holds raw pointers: every tensor stays referenced until the kernels ran
    dtab, dctx = _dev(table), _dev(np.full(B, M * 32, np.int32))
    args = [_dev(a) for a in (seq, pos, tok, page, kn, vn, ixn)]
    kv = U.make_kv(dk, dv, di, dtab, dctx, P, B, M)
    U.rope_cache_write(U.make_cfg(), kv, n, *args)
    torch.cuda.synchronize()
    for got, want in ((dk, kp), (dv, vp), (di, ip)):
        np.testing.assert_array_equal(got.cpu().numpy().view(np.uint16), want)

    q, qi = _bf16(g, (n, H, D)), _bf16(g, (n, D))
    dq, dqi = _dev(q), _dev(qi)
    U.rope_queries(U.make_cfg(), n, args[2], args[3], q=dq, q_idx=dqi)
    torch.cuda.synchronize()
    want_q = np.stack([oracle.rope_page2d(q[t], int(tok[t]), int(page[t])) for t in range(n)])
    want_qi = np.stack([oracle.rope_page2d(qi[t], int(tok[t]), int(page[t])) for t in range(n)])
    np.testing.assert_array_equal(dq.cpu().numpy().view(np.uint16), want_q)
    np.testing.assert_array_equal(dqi.cpu().numpy().view(np.uint16), want_qi)


def test_decode_on_caches_written_by_the_rope_kernel():
    """A 3-page document written token by token through the cache write
    (coordinates: in-page offset, page number), a rotated decode query, then
    the sparse decode path, against the oracle on oracle-rotated inputs."""
    g = np.random.default_rng(12)
    L, page_len = 2900, 1000
    M = -(-L // 32)
    P = M + 7
    table = g.permutation(P)[:M].reshape(1, M).astype(np.int32)
    kn, vn, ixn = _bf16(g, (L, H, D)), _bf16(g, (L, H, D)), _bf16(g, (L, D))
    tok = (np.arange(L) % page_len).astype(np.int32)
    page = (np.arange(L) // page_len).astype(np.int32)
    dk = torch.zeros((P, H, 32, D), dtype=torch.int16, device="cuda")
    dv = torch.zeros_like(dk)
    di = torch.zeros((P, 32, D), dtype=torch.int16, device="cuda")
    ctx, dtab = _dev(np.array([L], np.int32)), _dev(table)
    kv = U.make_kv(dk, dv, di, dtab, ctx, P, 1, M)
    cfg = U.make_cfg()
    args = [_dev(a) for a in (np.zeros(L, np.int32), np.arange(L, dtype=np.int32), tok, page, kn, vn, ixn)]
    U.rope_cache_write(cfg, kv, L, *args)
    q, qi = _bf16(g, (1, H, D)), _bf16(g, (1, D))
    qtok, qpage = np.array([(L - 1) % page_len], np.int32), np.array([(L - 1) // page_len], np.int32)
    dq, dqi, dqt, dqp = _dev(q), _dev(qi), _dev(qtok), _dev(qpage)
    U.rope_queries(cfg, 1, dqt, dqp, q=dq, q_idx=dqi)
    scores = torch.empty((1, M), dtype=torch.float32, device="cuda")
    idx = torch.empty((1, 16), dtype=torch.int32, device="cuda")
    out = torch.empty((1, H, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((1, H), dtype=torch.float32, device="cuda")
    U.indexer_score_decode(cfg, kv, dqi, scores)
    U.topk_attn_decode(cfg, kv, dq, scores, idx, out, lse)
    torch.cuda.synchronize()
    # oracle: rotate on the host, then the sparse decode query
    k_rot = np.stack([oracle.rope_page2d(kn[t], int(tok[t]), int(page[t])) for t in range(L)], axis=1)
    v_all = np.transpose(vn, (1, 0, 2))
    ix_rot = np.stack([oracle.rope_page2d(ixn[t], int(tok[t]), int(page[t])) for t in range(L)])
    q_rot = oracle.rope_page2d(q[0], int(qtok[0]), int(qpage[0]))
    qi_rot = oracle.rope_page2d(qi[0], int(qtok[0]), int(qpage[0]))
    ref = oracle.decode_query(q_rot, qi_rot, k_rot, v_all, ix_rot, L)
    G.check_selection(idx.cpu().numpy()[0], ref, 16)
    got = [int(x) for x in idx.cpu().numpy()[0] if x >= 0]
    if got == ref["selected"]:
        G.check_attention(out.cpu().numpy()[0], lse.cpu().numpy()[0], ref["out"], ref["lse"])


def test_page_coords_prefill_chunks_and_decode_steps_bit_exact():
    """uocr_page_coords against the oracle's coordinate rule: several
    streams over several 1024-token tiles with ragged tails, chunked calls
    carrying the state, and one-token decode steps of a batch."""
    g = np.random.default_rng(0xC0)
    marker = 151
    B, n = 5, 2600
    dens = [0.0, 0.002, 0.05, 0.5, 1.0]
    toks = np.stack([np.where(g.random(n) < d, marker, g.integers(0, 150, n)) for d in dens]).astype(np.int32)
    start = np.stack([g.integers(0, 20, B), g.integers(-1, 500, B)], axis=1).astype(np.int32)
    keep = []

    def run(tk, st):
        tk = np.ascontiguousarray(tk, dtype=np.int32)
        bb, nn = tk.shape
        d_tok, d_st = _dev(tk), _dev(st.astype(np.int32))
        d_tp = torch.full((bb, nn), -7, dtype=torch.int32, device="cuda")
        d_pp = torch.full((bb, nn), -7, dtype=torch.int32, device="cuda")
        keep.extend([d_tok, d_st, d_tp, d_pp])
        U.page_coords(bb, nn, d_tok, marker, d_st, d_tp, d_pp)
        torch.cuda.synchronize()
        return d_tp.cpu().numpy(), d_pp.cpu().numpy(), d_st.cpu().numpy()

    tp, pp, st = run(toks, start)
    for b in range(B):
        ot, op, os_ = oracle.page_coords(toks[b], marker, tuple(start[b]))
        np.testing.assert_array_equal(tp[b], ot)
        np.testing.assert_array_equal(pp[b], op)
        assert tuple(st[b]) == os_
    # one stream in chunks of 1, 255, 1024, 1025 and the rest, state carried on the device
    s = start[3:4].copy()
    out_t, out_p = [], []
    a = 0
    for c in [1, 255, 1024, 1025, n - 2305]:
        t_, p_, s = run(toks[3:4, a:a + c], s)
        out_t.append(t_[0])
        out_p.append(p_[0])
        a += c
    np.testing.assert_array_equal(np.concatenate(out_t), tp[3])
    np.testing.assert_array_equal(np.concatenate(out_p), pp[3])
    # decode: 16 sequences, 300 steps of one token each
    D, steps = 16, 300
    dt = np.where(g.random((D, steps)) < 0.03, marker, g.integers(0, 150, (D, steps))).astype(np.int32)
    ds = np.stack([np.zeros(D), np.full(D, -1)], axis=1).astype(np.int32)
    d_st = _dev(ds)
    got_t = np.empty((D, steps), np.int64)
    got_p = np.empty((D, steps), np.int64)
    d_tp = torch.empty((D, 1), dtype=torch.int32, device="cuda")
    d_pp = torch.empty((D, 1), dtype=torch.int32, device="cuda")
    d_all = _dev(np.ascontiguousarray(dt.T))          # [steps][D]
    for k in range(steps):
        U.page_coords(D, 1, d_all[k], marker, d_st, d_tp, d_pp)
        if k % 50 == 49 or k == steps - 1:
            torch.cuda.synchronize()
        got_t[:, k] = d_tp[:, 0].cpu().numpy()
        got_p[:, k] = d_pp[:, 0].cpu().numpy()
    for b in range(D):
        ot, op, os_ = oracle.page_coords(dt[b], marker, (0, -1))
        np.testing.assert_array_equal(got_t[b], ot)
        np.testing.assert_array_equal(got_p[b], op)
        assert tuple(d_st.cpu().numpy()[b]) == os_
