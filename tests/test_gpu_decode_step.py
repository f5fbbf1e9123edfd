"""GPU parity of the one-launch decode step (uocr_sparse_decode_step: every
layer's scoring, selection and attention as ticket-ordered work items)
through the C ABI: block scores and selections bit for bit equal to the
separate entry points, attention against the oracle (news.rkmt.cn/news/25027
Sec. 5 steps 2-4) and within float32 summation-order noise of the separate
attention kernel."""
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


def _wl(name, seed, lens, layers, values="normal"):
    lens = np.asarray(lens, np.int64)
    return W.Workload(name=name, seed=seed, batch=len(lens), layers=layers, ctx_lens=lens,
                      max_blocks=int(max(1, -(-int(lens.max()) // 32))), values=values)


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def run_step(dev, cfg, tags=None, qpages=None, fill=0xA7, schedule=U.STEP_ONE_LAUNCH, optional=True):
    """One call over every resident layer (by default forced to the one
    launch, whatever the automatic choice); returns host copies and the
    workspace's error word."""
    wl = dev.wl
    nl, B, M, H, D = dev.q.shape[0], wl.batch, wl.max_blocks, wl.heads, wl.head_dim
    topk = cfg.topk_blocks
    bp = _i32(tags) if tags is not None else None
    qp = _i32(qpages) if qpages is not None else None
    kv = U.make_kv(dev.k[0], dev.v[0], dev.kidx[0], dev.block_table, dev.ctx_lens, wl.pool_blocks, B, M, bp, qp)
    scores = torch.full((nl, B, M), float("nan"), dtype=torch.float32, device="cuda")
    idx = torch.full((nl, B, topk), -7, dtype=torch.int32, device="cuda")
    nsel = torch.full((nl, B), -7, dtype=torch.int32, device="cuda")
    out = torch.full((nl, B, H, D), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((nl, B, H), float("nan"), dtype=torch.float32, device="cuda")
    wsb = U.workspace_size(cfg, U.OP_DECODE_STEP, nl * B, M)
    assert wsb > 0
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    ws.fill_(fill)  # stale counters must not matter: the call clears them
    U.sparse_decode_step(cfg, kv, nl, dev.q_idx, dev.q, scores, idx, out, lse if optional else None,
                         n_sel=nsel if optional else None, ws=ws, schedule=schedule)
    torch.cuda.synchronize()
    err = int(ws[4:8].cpu().numpy().view(np.uint32)[0])
    return {"scores": scores.cpu().numpy(), "idx": idx.cpu().numpy(), "nsel": nsel.cpu().numpy(),
            "out": out.cpu().numpy(), "lse": lse.cpu().numpy(), "err": err}


def separate(dev, cfg, li, tags=None, qpages=None):
    """Layer li through the separate scoring launch and the fused
    selection + attention launch."""
    wl = dev.wl
    B, M, H, D = wl.batch, wl.max_blocks, wl.heads, wl.head_dim
    bp = _i32(tags) if tags is not None else None
    qp = _i32(qpages) if qpages is not None else None
    kv = U.make_kv(dev.k[li], dev.v[li], dev.kidx[li], dev.block_table, dev.ctx_lens, wl.pool_blocks, B, M, bp, qp)
    scores = torch.full((B, M), float("nan"), dtype=torch.float32, device="cuda")
    idx = torch.full((B, cfg.topk_blocks), -7, dtype=torch.int32, device="cuda")
    nsel = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    out = torch.full((B, H, D), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, H), float("nan"), dtype=torch.float32, device="cuda")
    U.indexer_score_decode(cfg, kv, dev.q_idx[li], scores)
    U.topk_attn_decode(cfg, kv, dev.q[li], scores, idx, out, lse, n_sel=nsel)
    torch.cuda.synchronize()
    return {"scores": scores.cpu().numpy(), "idx": idx.cpu().numpy(), "nsel": nsel.cpu().numpy(),
            "out": out.cpu().numpy(), "lse": lse.cpu().numpy()}


def compare_with_separate(dev, cfg, res, tags=None, qpages=None, atol=1e-5):
    for li in range(dev.q.shape[0]):
        ref = separate(dev, cfg, li, tags, qpages)
        np.testing.assert_array_equal(res["scores"][li].view(np.uint32), ref["scores"].view(np.uint32),
                                      err_msg=f"layer {li} block scores")
        np.testing.assert_array_equal(res["idx"][li], ref["idx"], err_msg=f"layer {li} selection")
        np.testing.assert_array_equal(res["nsel"][li], ref["nsel"])
        fin = np.isfinite(ref["lse"])
        assert np.array_equal(fin, np.isfinite(res["lse"][li]))
        assert np.all(np.isneginf(res["lse"][li][~fin]))
        np.testing.assert_allclose(res["lse"][li][fin], ref["lse"][fin], rtol=0, atol=atol)
        np.testing.assert_allclose(res["out"][li], ref["out"], rtol=0, atol=atol)


def oracle_check(wl, res, layer, b, cfg_o, tags=None, qpage=None):
    L = int(wl.ctx_lens[b])
    kidx = wl.kidx(layer, b, 0, L)
    if tags is None:
        ref = oracle.decode_query_fetch(wl.q(layer, b), wl.q_idx(layer, b), kidx, G.fetcher(wl, layer, b), L, cfg_o)
    else:
        ref = oracle.decode_query_fetch(wl.q(layer, b), wl.q_idx(layer, b), kidx, G.fetcher(wl, layer, b), L, cfg_o,
                                        tags[b], int(qpage))
    G.check_scores(res["scores"][layer, b], ref, wl.q_idx(layer, b), kidx, wl.max_blocks)
    G.check_selection(res["idx"][layer, b], ref, cfg_o.topk_blocks)
    got = [int(x) for x in res["idx"][layer, b] if x >= 0]
    if got == ref["selected"]:
        G.check_attention(res["out"][layer, b], res["lse"][layer, b], ref["out"], ref["lse"])
    else:
        o2, l2 = G.oracle_attend_with(wl, layer, b, wl.q(layer, b), got, L - 1, cfg_o)
        G.check_attention(res["out"][layer, b], res["lse"][layer, b], o2, l2)


def test_ragged_batch_three_layers():
    lens = [0, 1, 31, 33, 127, 129, 513, 4097, 9999, 20001]
    wl = _wl("step ragged", 0x5701, lens, layers=3)
    print("case: decode step ragged", lens, "3 layers", flush=True)
    dev = SD.generate(wl)
    cfg = G.cfg_for(wl)
    res = run_step(dev, cfg)
    assert res["err"] == 0
    compare_with_separate(dev, cfg, res)
    for layer, b in ((0, 9), (2, 7), (1, 2), (2, 0)):
        oracle_check(wl, res, layer, b, G.ocfg())
    # the per-layer schedule runs the separate kernels themselves: identical,
    # attention included; the automatic choice takes it for this small batch
    for sched in (U.STEP_PER_LAYER, U.STEP_AUTO):
        r2 = run_step(dev, cfg, schedule=sched)
        compare_with_separate(dev, cfg, r2, atol=0)
    # lse and n_sel are optional outputs: left NULL, nothing else changes
    r3 = run_step(dev, cfg, optional=False)
    for k in ("scores", "idx", "out"):
        np.testing.assert_array_equal(r3[k].view(np.uint32), res[k].view(np.uint32), err_msg=k)
    assert np.all(np.isnan(r3["lse"])) and np.all(r3["nsel"] == -7)


def test_batch_of_one_is_layer_serial_and_repeatable():
    # batch 1: no overlap across sequences; layer l + 1 waits for layer l
    wl = _wl("step one sequence", 0x5702, [12345], layers=4)
    print("case: decode step B=1, 4 layers, twice", flush=True)
    dev = SD.generate(wl)
    cfg = G.cfg_for(wl)
    r1 = run_step(dev, cfg, fill=0x00)
    r2 = run_step(dev, cfg, fill=0xFF)
    assert r1["err"] == 0 and r2["err"] == 0
    for k in ("scores", "out", "lse"):
        np.testing.assert_array_equal(r1[k].view(np.uint32), r2[k].view(np.uint32), err_msg=k)
    np.testing.assert_array_equal(r1["idx"], r2["idx"])
    compare_with_separate(dev, cfg, r1)
    oracle_check(wl, r1, 3, 0, G.ocfg())


@pytest.mark.parametrize("topk,local", [(16, 4), (8, 1), (64, 2)])
def test_topk_variants(topk, local):
    lens = [3000, 65, 7777, 600, 2049]
    wl = _wl(f"step topk {topk}", 0x5703 + topk, lens, layers=2, values="small_int")
    print("case: decode step topk", topk, "local", local, flush=True)
    dev = SD.generate(wl)
    cfg = G.cfg_for(wl, topk, local)
    res = run_step(dev, cfg)
    assert res["err"] == 0
    compare_with_separate(dev, cfg, res)
    oracle_check(wl, res, 1, 2, G.ocfg(topk, local))


def test_page_tags():
    g = np.random.default_rng(0x5704)
    lens = [8000, 3000, 12000, 500, 5000, 9000]
    wl = _wl("step page tags", 0x5704, lens, layers=2)
    print("case: decode step with page tags", flush=True)
    dev = SD.generate(wl)
    M = wl.max_blocks
    tags = (np.arange(M)[None, :] // g.integers(20, 60, (wl.batch, 1))).astype(np.int32)
    qpages = np.array([g.integers(0, max(1, int(tags[b, max(0, -(-lens[b] // 32) - 1)]) + 1))
                       for b in range(wl.batch)], np.int32)
    cfg = G.cfg_for(wl)
    res = run_step(dev, cfg, tags, qpages)
    assert res["err"] == 0
    compare_with_separate(dev, cfg, res, tags, qpages)
    oracle_check(wl, res, 1, 2, G.ocfg(), tags, qpages[2])
    r2 = run_step(dev, cfg, tags, qpages, schedule=U.STEP_PER_LAYER)
    compare_with_separate(dev, cfg, r2, tags, qpages, atol=0)


def test_full_headline_workload_sampled():
    """16 sequences x 12 layers at 131072 tokens, the measured configuration:
    every layer bitwise against the separate launches, sampled queries
    against the oracle."""
    torch.cuda.empty_cache()
    wl = W.config3()
    print("case: decode step", wl.name, flush=True)
    dev = SD.generate(wl)
    cfg = G.cfg_for(wl)
    res = run_step(dev, cfg)
    assert res["err"] == 0
    compare_with_separate(dev, cfg, res)
    for layer, b in ((0, 0), (11, 15)):
        oracle_check(wl, res, layer, b, G.ocfg())
    # the automatic choice takes the one launch here: the same results bit for bit
    r_auto = run_step(dev, cfg, schedule=U.STEP_AUTO)
    for k in ("scores", "idx", "out", "lse"):
        np.testing.assert_array_equal(r_auto[k].view(np.uint32), res[k].view(np.uint32), err_msg=k)
    del dev
    torch.cuda.empty_cache()


def test_ragged_multi_page_workload_with_page_tags():
    """64 documents of 1000-token pages (400 image + 600 text tokens), one
    layer, with and without the page tags of their image blocks."""
    wl = W.config4()
    print("case: decode step", wl.name, flush=True)
    dev = SD.generate(wl)
    M = wl.max_blocks
    tags = np.tile(W.page_tags(M), (wl.batch, 1)).astype(np.int32)
    qpages = np.array([W.page_of(int(L) - 1) for L in wl.ctx_lens], np.int32)
    cfg = G.cfg_for(wl)
    for t, q in ((None, None), (tags, qpages)):
        res = run_step(dev, cfg, t, q)
        assert res["err"] == 0
        compare_with_separate(dev, cfg, res, t, q)
        b = int(np.argmax(wl.ctx_lens))
        oracle_check(wl, res, 0, b, G.ocfg(), t, None if q is None else q[b])


def test_context_above_4096_candidate_blocks():
    # 5000 blocks: more candidates than the 8-keys-per-thread selection holds
    # (the 32-keys-per-thread instantiation)
    lens = [160000, 1000, 131105]
    wl = _wl("step long context", 0x5705, lens, layers=2)
    print("case: decode step max_blocks", wl.max_blocks, flush=True)
    dev = SD.generate(wl)
    cfg = G.cfg_for(wl)
    res = run_step(dev, cfg)
    assert res["err"] == 0
    compare_with_separate(dev, cfg, res)
    oracle_check(wl, res, 1, 0, G.ocfg())


@pytest.mark.parametrize("batch,layers", [(200, 3), (3, 5)])
def test_batch_shapes(batch, layers):
    """Ticket order at other batch sizes: 200 sequences (lag 100, 600 slots)
    and 3 sequences (lag 1), ragged contexts of 1 to 6000 tokens, forced to
    the one launch: no wait gives up, scores and selections equal the
    separate launches bit for bit, sampled queries match the oracle."""
    g = np.random.default_rng(0x5709 + batch)
    lens = g.integers(1, 6000, size=batch)
    wl = _wl(f"step batch {batch} x {layers} layers", 0x5709 + batch, lens, layers=layers)
    print(f"case: decode step batch {batch} x {layers} layers", flush=True)
    dev = SD.generate(wl)
    cfg = G.cfg_for(wl)
    res = run_step(dev, cfg)
    assert res["err"] == 0
    compare_with_separate(dev, cfg, res)
    for layer, b in ((0, 0), (layers - 1, batch - 1), (layers // 2, batch // 2)):
        oracle_check(wl, res, layer, b, G.ocfg())


def test_maximum_candidate_count():
    """The largest context the step accepts: max_blocks - local = 16384
    candidate blocks (a 524,416-token sequence, where every thread of the
    selection holds its full share of keys) beside a short sequence.  The one
    launch, the per-layer launches and the separate entry points agree bit
    for bit on scores and selections, and both sequences match the oracle."""
    lens = [16388 * 32, 3000]
    wl = _wl("step maximum candidates", 0x5708, lens, layers=1)
    print("case: decode step at the candidate limit, max_blocks", wl.max_blocks, flush=True)
    dev = SD.generate(wl)
    cfg = G.cfg_for(wl)
    assert wl.max_blocks - cfg.local_blocks == 16384
    res = run_step(dev, cfg)
    assert res["err"] == 0
    compare_with_separate(dev, cfg, res)
    compare_with_separate(dev, cfg, run_step(dev, cfg, schedule=U.STEP_PER_LAYER), atol=0)
    for b in range(wl.batch):
        oracle_check(wl, res, 0, b, G.ocfg())


def test_out_of_range_pool_blocks():
    """Block-table entries outside the pool (-1, >= num_blocks): their blocks
    score NaN, rank last and are never attended, exactly as in the separate
    launches."""
    lens = [9000, 3000, 12345, 700]
    wl = _wl("step bad table", 0x5706, lens, layers=2)
    print("case: decode step with out-of-range table entries", flush=True)
    dev = SD.generate(wl)
    tab = dev.block_table.cpu().numpy().copy()
    g = np.random.default_rng(0x5706)
    for b, L in enumerate(lens):
        nb = -(-L // 32)
        for j in g.choice(nb, size=min(nb, 7), replace=False):
            tab[b, j] = -1 if g.random() < 0.5 else wl.pool_blocks + int(g.integers(0, 1000))
    dev.block_table.copy_(torch.from_numpy(tab))
    cfg = G.cfg_for(wl)
    res = run_step(dev, cfg)
    assert res["err"] == 0
    compare_with_separate(dev, cfg, res)
    assert np.isnan(res["scores"]).any()


def test_concurrent_calls_on_two_streams():
    """Two one-launch calls with their own workspaces running at the same
    time on two streams give the results of the calls run one after the
    other."""
    wl = _wl("step concurrent", 0x5707, [20000, 7000, 15000, 30000, 1000, 25000], layers=3)
    print("case: decode step, two concurrent calls", flush=True)
    dev = SD.generate(wl)
    cfg = G.cfg_for(wl)
    ref = run_step(dev, cfg)
    nl, B, M, H, D = dev.q.shape[0], wl.batch, wl.max_blocks, wl.heads, wl.head_dim
    halves = [(0, 3), (3, 6)]
    outs = []
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    keep = []
    torch.cuda.synchronize()
    for (b0, b1), st in zip(halves, streams):
        nb = b1 - b0
        kv = U.make_kv(dev.k[0], dev.v[0], dev.kidx[0], dev.block_table[b0:b1], dev.ctx_lens[b0:b1],
                       wl.pool_blocks, nb, M)
        qi = dev.q_idx[:, b0:b1].contiguous()
        q = dev.q[:, b0:b1].contiguous()
        sc = torch.full((nl, nb, M), float("nan"), dtype=torch.float32, device="cuda")
        ix = torch.full((nl, nb, 16), -7, dtype=torch.int32, device="cuda")
        o = torch.full((nl, nb, H, D), float("nan"), dtype=torch.float32, device="cuda")
        ls = torch.full((nl, nb, H), float("nan"), dtype=torch.float32, device="cuda")
        ws = torch.full((U.workspace_size(cfg, U.OP_DECODE_STEP, nl * nb, M),), 0x33, dtype=torch.uint8,
                        device="cuda")
        torch.cuda.synchronize()
        keep.append((kv, qi, q, ws))
        U.sparse_decode_step(cfg, kv, nl, qi, q, sc, ix, o, ls, ws=ws, stream=st, schedule=U.STEP_ONE_LAUNCH)
        outs.append((b0, b1, sc, ix, o, ls, ws))
    torch.cuda.synchronize()
    for b0, b1, sc, ix, o, ls, ws in outs:
        assert int(ws[4:8].cpu().numpy().view(np.uint32)[0]) == 0
        np.testing.assert_array_equal(sc.cpu().numpy().view(np.uint32), ref["scores"][:, b0:b1].view(np.uint32))
        np.testing.assert_array_equal(ix.cpu().numpy(), ref["idx"][:, b0:b1])
        np.testing.assert_array_equal(o.cpu().numpy().view(np.uint32), ref["out"][:, b0:b1].view(np.uint32))
        np.testing.assert_array_equal(ls.cpu().numpy().view(np.uint32), ref["lse"][:, b0:b1].view(np.uint32))


def test_graph_capture_and_replays():
    """The one-launch step captured in a HIP graph (its counters are cleared
    by a kernel, not a memset) and replayed several times with eager work in
    between: every replay equals the eager call bit for bit."""
    wl = _wl("step graph", 0x5708, [9000, 30000, 4097, 12345], layers=3)
    print("case: decode step in a HIP graph", flush=True)
    dev = SD.generate(wl)
    cfg = G.cfg_for(wl)
    ref = run_step(dev, cfg)
    nl, B, M, H, D = dev.q.shape[0], wl.batch, wl.max_blocks, wl.heads, wl.head_dim
    kv = U.make_kv(dev.k[0], dev.v[0], dev.kidx[0], dev.block_table, dev.ctx_lens, wl.pool_blocks, B, M)
    scores = torch.zeros((nl, B, M), dtype=torch.float32, device="cuda")
    idx = torch.zeros((nl, B, 16), dtype=torch.int32, device="cuda")
    out = torch.zeros((nl, B, H, D), dtype=torch.float32, device="cuda")
    lse = torch.zeros((nl, B, H), dtype=torch.float32, device="cuda")
    ws = torch.zeros(U.workspace_size(cfg, U.OP_DECODE_STEP, nl * B, M), dtype=torch.uint8, device="cuda")
    cap = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=cap):
        U.sparse_decode_step(cfg, kv, nl, dev.q_idx, dev.q, scores, idx, out, lse, ws=ws,
                             stream=cap.cuda_stream, schedule=U.STEP_ONE_LAUNCH)
    torch.cuda.synchronize()
    for rep in range(3):
        for x in (scores, out, lse):
            x.fill_(float("nan"))
        idx.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert int(ws[4:8].cpu().numpy().view(np.uint32)[0]) == 0
        np.testing.assert_array_equal(scores.cpu().numpy().view(np.uint32), ref["scores"].view(np.uint32))
        np.testing.assert_array_equal(idx.cpu().numpy(), ref["idx"])
        np.testing.assert_array_equal(out.cpu().numpy().view(np.uint32), ref["out"].view(np.uint32))
        np.testing.assert_array_equal(lse.cpu().numpy().view(np.uint32), ref["lse"].view(np.uint32))
        run_step(dev, cfg)  # eager work between replays


def test_contiguous_block_layout():
    """The workload generator's contiguous placement (each sequence's blocks
    consecutive in the pool): same parity as the random placement."""
    wl = _wl("step contiguous layout", 0x5709, [20000, 9000, 33000], layers=2)
    wl.layout = "contiguous"
    print("case: decode step, contiguous block layout", flush=True)
    dev = SD.generate(wl)
    tab = dev.block_table.cpu().numpy()
    assert np.array_equal(tab[0, :10], np.arange(10))
    cfg = G.cfg_for(wl)
    res = run_step(dev, cfg)
    assert res["err"] == 0
    compare_with_separate(dev, cfg, res)
    oracle_check(wl, res, 1, 2, G.ocfg())
