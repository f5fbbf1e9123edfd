"""GPU parity of the page-aware candidate ranking (news.rkmt.cn/news/25027
Sec. 5, the page-aware candidate constraint; leheavengame.com OCR 2 release
article Sec. 2 route A, Page Gate) against the CPU oracle, through the C ABI:
the fused decode selection + attention and the chunked-prefill scoring +
merge with block page tags and query pages."""
from __future__ import annotations

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import block_sparse_long_sr_amd as U  # noqa: E402
import oracle  # noqa: E402
from synth import device as SD  # noqa: E402
from synth import workloads as W  # noqa: E402
import gpu_harness as G  # noqa: E402


def _wl(name, seed, lens, values="normal"):
    lens = np.asarray(lens, np.int64)
    return W.Workload(name=name, seed=seed, batch=len(lens), layers=1, ctx_lens=lens,
                      max_blocks=int(max(1, -(-int(lens.max()) // 32))), values=values)


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def gated_decode(dev, cfg, tags, qpages):
    """Indexer scoring, then the fused selection + attention with page tags."""
    wl = dev.wl
    B, M, H, D = wl.batch, wl.max_blocks, wl.heads, wl.head_dim
    topk = cfg.topk_blocks
    bp, qp = _i32(tags), _i32(qpages)
    kv = U.make_kv(dev.k[0], dev.v[0], dev.kidx[0], dev.block_table, dev.ctx_lens, wl.pool_blocks, B, M, bp, qp)
    scores = torch.full((B, M), float("nan"), dtype=torch.float32, device="cuda")
    idx = torch.full((B, topk), -7, dtype=torch.int32, device="cuda")
    nsel = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    out = torch.full((B, H, D), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, H), float("nan"), dtype=torch.float32, device="cuda")
    U.indexer_score_decode(cfg, kv, dev.q_idx[0], scores)
    U.topk_attn_decode(cfg, kv, dev.q[0], scores, idx, out, lse, n_sel=nsel)
    torch.cuda.synchronize()
    return {"scores": scores.cpu().numpy(), "idx": idx.cpu().numpy(), "nsel": nsel.cpu().numpy(),
            "out": out.cpu().numpy(), "lse": lse.cpu().numpy()}


def check_gated_decode(wl, seqs, tags, qpages, topk=16, local=4):
    cfg_u, cfg_o = G.cfg_for(wl, topk, local), G.ocfg(topk, local, wl.heads)
    dev = SD.generate(wl)
    res = gated_decode(dev, cfg_u, tags, qpages)
    refs = {}
    for b in seqs:
        L = int(wl.ctx_lens[b])
        kidx = wl.kidx(0, b, 0, L)
        ref = oracle.decode_query_fetch(wl.q(0, b), wl.q_idx(0, b), kidx, G.fetcher(wl, 0, b), L, cfg_o,
                                        tags[b], int(qpages[b]))
        refs[b] = ref
        if L > 0:
            G.check_scores(res["scores"][b], ref, wl.q_idx(0, b), kidx, wl.max_blocks)
        G.check_selection(res["idx"][b], ref, topk)
        assert res["nsel"][b] == min(topk, -(-L // 32))
        got = [int(x) for x in res["idx"][b] if x >= 0]
        if got == ref["selected"]:
            G.check_attention(res["out"][b], res["lse"][b], ref["out"], ref["lse"])
        else:
            o2, l2 = G.oracle_attend_with(wl, 0, b, wl.q(0, b), got, L - 1, cfg_o)
            G.check_attention(res["out"][b], res["lse"][b], o2, l2)
    return res, refs


def test_page_gate_decode_document_pages():
    """Ragged multi-page documents (400 image + 600 text tokens per page, the
    query on the last page): every remote block comes from the query's page,
    although 1-3 earlier pages carry keys correlated with the query."""
    wl = W.config4()
    print("case: page-aware decode,", wl.name, flush=True)
    tags = np.tile(W.page_tags(wl.max_blocks), (wl.batch, 1))
    qpages = np.array([W.page_of(L - 1) for L in wl.ctx_lens], np.int32)
    seqs = list(range(0, wl.batch, 4))
    res, refs = check_gated_decode(wl, seqs, tags, qpages)
    for b in seqs:
        ref = refs[b]
        assert all(tags[b, j] == qpages[b] for j in ref["remote"]), b
        got = [int(x) for x in res["idx"][b] if x >= 0]
        assert sum(tags[b, j] == qpages[b] for j in got) >= 12


def test_page_gate_decode_fallback_fills_slots():
    """Pages with 200 image tokens (7 tagged blocks): all of the query's
    page's candidate blocks are kept and the other slots fall back to the
    best blocks of the rest of the context."""
    lens = [12000, 30000, 7000, 64000, 2500, 1000]
    wl = _wl("page gate fallback", 0xD1, lens)
    print("case: page-aware decode fallback", lens, flush=True)
    tags = np.tile(W.page_tags(wl.max_blocks, 1000, 200), (wl.batch, 1))
    qpages = np.array([W.page_of(L - 1) for L in lens], np.int32)
    # the query sits on its page's text, so its page's image blocks are candidates
    res, refs = check_gated_decode(wl, range(wl.batch), tags, qpages)
    for b in range(wl.batch):
        ref = refs[b]
        if ref["tiers"] is None or ref["cutoff"] is None:
            continue
        inpage = set(np.nonzero(ref["tiers"])[0].tolist())
        assert inpage <= set(ref["remote"])


def test_page_gate_decode_random_tags():
    """Random tags over a few pages (the query's page tags from none to more
    than twelve candidates), including lengths below 16 blocks."""
    lens = [32768, 20000, 5000, 900, 480, 4097, 16384, 100]
    wl = _wl("page gate random", 0xD2, lens)
    print("case: page-aware decode random tags", lens, flush=True)
    g = np.random.default_rng(5)
    tags = np.full((wl.batch, wl.max_blocks), -1, np.int32)
    qpages = np.zeros(wl.batch, np.int32)
    for b in range(wl.batch):
        frac = [0.0, 0.002, 0.01, 0.3, 1.0, 0.5, 0.05, 0.2][b]
        tags[b] = np.where(g.random(wl.max_blocks) < frac, 3, g.integers(-1, 3, wl.max_blocks))
        qpages[b] = 3
    check_gated_decode(wl, range(wl.batch), tags, qpages)


def test_page_gate_decode_small_int_exact():
    """Integer-valued inputs: scores are exact, the tier bit costs no ranking
    precision, so the selection matches the oracle exactly (with ties)."""
    lens = [3000, 7777, 2049]
    wl = _wl("page gate small ints", 0xD3, lens, values="small_int")
    print("case: page-aware decode small-int exact", flush=True)
    tags = np.tile(W.page_tags(wl.max_blocks, 1000, 300), (wl.batch, 1))
    qpages = np.array([W.page_of(L - 1) for L in lens], np.int32)
    res, refs = check_gated_decode(wl, range(wl.batch), tags, qpages)
    for b in range(wl.batch):
        got = [int(x) for x in res["idx"][b] if x >= 0]
        assert got == refs[b]["selected"]


def gated_prefill(dev, cfg, tags_row, row_pages):
    wl = dev.wl
    T, M, H, D = wl.rows, wl.max_blocks, wl.heads, wl.head_dim
    topk = cfg.topk_blocks
    bp, qp = _i32(tags_row[None, :]), _i32(row_pages)
    kv = U.make_kv(dev.k[0], dev.v[0], dev.kidx[0], dev.block_table, dev.ctx_lens, wl.pool_blocks, 1, M, bp, qp)
    ws_bytes = U.workspace_size(cfg, U.OP_INDEXER_PREFILL, T, M)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
    idx = torch.full((T, topk), -7, dtype=torch.int32, device="cuda")
    nsel = torch.full((T,), -7, dtype=torch.int32, device="cuda")
    out = torch.full((T, H, D), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    wsarg = (ws.data_ptr(), ws_bytes)
    U.indexer_score_prefill(cfg, kv, dev.q_idx, wl.q_start, T, wsarg)
    U.block_topk_prefill(cfg, wsarg, wl.q_start, T, M, idx, nsel)
    U.sparse_attn_prefill(cfg, kv, dev.q, wl.q_start, T, idx, out, lse)
    torch.cuda.synchronize()
    return {"idx": idx.cpu().numpy(), "nsel": nsel.cpu().numpy(), "out": out.cpu().numpy(),
            "lse": lse.cpu().numpy()}


@pytest.mark.parametrize("values", ["normal", "small_int"])
def test_page_gate_prefill_rows_on_two_pages(values):
    """A chunk whose rows lie on two pages: each row ranks its own page's
    image blocks first (rows on the second page's image tokens see part of
    their page's blocks inside the local window)."""
    wl = W.prefill_case(f"page gate prefill {values}", 0xD4, 6000, 3800, 600, values=values)
    print("case:", wl.name, flush=True)
    cfg_u, cfg_o = G.cfg_for(wl), G.ocfg()
    dev = SD.generate(wl)
    tags = W.page_tags(wl.max_blocks, 1000, 350)
    row_pages = np.array([W.page_of(wl.q_start + t) for t in range(wl.rows)], np.int32)
    res = gated_prefill(dev, cfg_u, tags, row_pages)
    S = int(wl.ctx_lens[0])
    kidx = wl.kidx(0, 0, 0, S)
    allrows = np.arange(wl.rows)
    q = wl.q_rows(allrows)
    qi = wl.q_idx_rows(allrows)
    rows = sorted(set([0, 1, 199, 200, 201, 399, 400, 599] + list(range(3, wl.rows, 23))))
    refs = oracle.prefill_rows_fetch(q, qi, kidx, G.fetcher(wl, 0, 0), wl.q_start, rows, cfg_o, tags, row_pages)
    for r in refs:
        t = r["row"]
        got = [int(x) for x in res["idx"][t] if x >= 0]
        if values == "small_int":
            assert got == r["selected"], (t, got, r["selected"])
        else:
            G.check_selection(res["idx"][t], r, 16)
        assert res["nsel"][t] == min(16, (wl.q_start + t) // 32 + 1)
        if got == r["selected"]:
            G.check_attention(res["out"][t], res["lse"][t], r["out"], r["lse"])
        else:
            o2, l2 = G.oracle_attend_with(wl, 0, 0, q[t], got, wl.q_start + t, cfg_o)
            G.check_attention(res["out"][t], res["lse"][t], o2, l2)


def test_page_gate_prefill_long_chunk_8bit_split_ids():
    """A 8704-row chunk at 128K with page tags: 17 row tiles would ask for
    splits of 272 blocks (9-bit in-split ids); the plan holds splits to 256
    blocks (8-bit ids), so with the tier bit a score still ranks to 2^-14
    relative, inside the 1e-4 band.  Sampled rows on every row tile against
    the oracle on the device inputs."""
    S, T = 131072, 8704
    wl = W.prefill_case("page gate prefill T=8704 at 122368 of 131072", 0xD5, S, S - T, T)
    print("case:", wl.name, flush=True)
    cfg_u, cfg_o = G.cfg_for(wl), G.ocfg()
    M = wl.max_blocks
    assert U.workspace_size(cfg_u, U.OP_INDEXER_PREFILL, T, M) == T * (M // 256) * 12 * 4
    dev = SD.generate(wl)
    tags = W.page_tags(M)
    row_pages = np.array([W.page_of(wl.q_start + t) for t in range(T)], np.int32)
    res = gated_prefill(dev, cfg_u, tags, row_pages)
    kidx = dev.host_kidx(0, 0, S)
    q, qi = dev.host_prefill_queries()
    fetch = dev.host_kv_fetch(0, 0)
    rows = sorted(set([0, 1, 31, 511, 512, 4095, 4096, 8191, 8192, T - 1] + list(range(7, T, 613))))
    refs = oracle.prefill_rows_fetch(q, qi, kidx, fetch, wl.q_start, rows, cfg_o, tags, row_pages)
    for r in refs:
        t = r["row"]
        assert res["nsel"][t] == min(16, (wl.q_start + t) // 32 + 1)
        G.check_query_end_to_end(r, q[t], fetch, wl.q_start + t, cfg_o, res["idx"][t], res["out"][t], res["lse"][t])
