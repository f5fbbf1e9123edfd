"""GPU parity of the chunked-prefill path (MFMA indexer scoring with fused
block max and per-split selection, merge, sparse attention) against the CPU
oracle, through the C ABI."""
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


def check_prefill(wl, rows, topk=16, local=4, exact=False, block_major=True):
    cfg_u, cfg_o = G.cfg_for(wl, topk, local), G.ocfg(topk, local)
    dev = SD.generate(wl)
    res = G.gpu_prefill(dev, cfg_u, block_major=block_major)
    S = int(wl.ctx_lens[0])
    kidx = wl.kidx(0, 0, 0, S)
    allrows = np.arange(wl.rows)
    q = wl.q_rows(allrows)
    qi = wl.q_idx_rows(allrows)
    refs = oracle.prefill_rows_fetch(q, qi, kidx, G.fetcher(wl, 0, 0), wl.q_start, list(rows), cfg_o)
    idx_oracle = res["idx"].copy()
    for r in refs:
        t = r["row"]
        if exact:
            got = [int(x) for x in res["idx"][t] if x >= 0]
            assert got == r["selected"], (t, got, r["selected"])
        else:
            G.check_selection(res["idx"][t], r, topk)
        assert res["nsel"][t] == min(topk, (wl.q_start + t) // 32 + 1)
        idx_oracle[t] = G.pad_idx(r["selected"], topk)
    res_o = G.gpu_prefill(dev, cfg_u, idx_override=idx_oracle, block_major=block_major)
    for r in refs:
        t = r["row"]
        G.check_attention(res_o["out"][t], res_o["lse"][t], r["out"], r["lse"])
        got = [int(x) for x in res["idx"][t] if x >= 0]
        if got == r["selected"]:
            G.check_attention(res["out"][t], res["lse"][t], r["out"], r["lse"])
        else:
            o2, l2 = G.oracle_attend_with(wl, 0, 0, q[t], got, wl.q_start + t, cfg_o)
            G.check_attention(res["out"][t], res["lse"][t], o2, l2)
    return res


def test_prefill_three_tiles_ragged():
    wl = W.prefill_case("prefill S=1700 q_start=1000 T=700", 0xF1, 1700, 1000, 700)
    print("case:", wl.name, flush=True)
    check_prefill(wl, range(wl.rows))


def test_prefill_unaligned_start_dense_rows():
    wl = W.prefill_case("prefill S=377 q_start=77 T=300", 0xF2, 377, 77, 300)
    print("case:", wl.name, flush=True)
    check_prefill(wl, range(wl.rows))


def test_prefill_small_integer_inputs_exact():
    wl = W.prefill_case("prefill small-int", 0xF3, 2260, 2000, 260, values="small_int")
    print("case:", wl.name, flush=True)
    check_prefill(wl, range(wl.rows), exact=True)


@pytest.mark.parametrize("topk,local", [(8, 2), (20, 4), (5, 4), (4, 4), (16, 1), (24, 8)])
def test_prefill_remote_slot_variants(topk, local):
    """Selection sizes and local windows: topk above 16 or not a multiple of 4
    takes the window pass's general path for the row's block ids; local 1
    and 8 change the window the pass covers per 32-row block."""
    wl = W.prefill_case(f"prefill topk {topk} local {local}", 0xF4 + topk, 2500, 2200, 300)
    print("case:", wl.name, flush=True)
    check_prefill(wl, range(0, wl.rows, 3), topk, local)


def test_prefill_64_splits_sampled():
    wl = W.prefill_case("prefill S=32768 q_start=30720 T=2048", 0xF5, 32768, 30720, 2048)
    print("case:", wl.name, flush=True)
    rows = sorted(set([0, 1, 31, 32, 255, 256, 511, 1023, 1024, 2047] + list(range(5, 2048, 97))))
    check_prefill(wl, rows)


def test_prefill_full_chunk_sampled():
    """The measured chunk: T=2048 rows at q_start=129024 of a 131072-token
    context (64 splits of 64 blocks), in the bench's launch configuration
    (block-major attention), sampled rows against the oracle."""
    wl = W.config5()
    print("case:", wl.name, flush=True)
    rows = [0, 1, 31, 32, 511, 512, 1024, 2047] + list(range(7, 2048, 331))
    check_prefill(wl, sorted(set(rows)))


def test_prefill_attention_hot_blocks():
    """Every row of a 2048-row chunk keeps the same 16 blocks: each bucket
    holds 2048 pairs (64 full 32-row chunks of one block), the staged
    bucketing's LDS counters take 2048 atomics each, and most blocks get no
    pair at all.  Block-major against row-major and sampled rows against the
    oracle."""
    wl = W.prefill_case("prefill hot blocks S=8192 q_start=6144 T=2048", 0xFB, 8192, 6144, 2048)
    print("case:", wl.name, flush=True)
    cfg_u, cfg_o = G.cfg_for(wl), G.ocfg()
    dev = SD.generate(wl)
    T = wl.rows
    hot = np.array([0, 3, 17, 40, 41, 42, 99, 100, 150, 151, 152, 160, 170, 180, 190, 191], np.int32)
    idx = np.tile(hot, (T, 1))
    res_b = G.gpu_prefill(dev, cfg_u, idx_override=idx)
    res_r = G.gpu_prefill(dev, cfg_u, idx_override=idx, block_major=False)
    assert np.abs(res_b["out"] - res_r["out"]).max() <= 1e-5
    assert np.abs(res_b["lse"] - res_r["lse"]).max() <= 1e-5
    q = wl.q_rows(np.arange(T))
    toks = np.concatenate([oracle.attended_tokens([int(j)], wl.q_start, cfg_o) for j in hot])
    k_, v_ = G.fetcher(wl, 0, 0)(toks)
    for t in [0, 1, 31, 32, 1000, 2047]:
        o2, l2 = oracle.attend(q[t], k_, v_, np.arange(toks.size), cfg_o.sm_scale)
        G.check_attention(res_b["out"][t], res_b["lse"][t], o2, l2)


def test_prefill_block_major_unstaged_bucketing():
    """A chunk past the bucketing's LDS staging (more than 4096 blocks and
    more than 32768 (row, slot) pairs): the pairs are scattered straight to
    the workspace, and those past the first 32768 are loaded in later rounds
    (rows 2048 and up).  Sampled rows, both sides of that split, against the
    oracle."""
    wl = W.prefill_case("prefill S=140000 q_start=137900 T=2100", 0xFA, 140000, 137900, 2100)
    print("case:", wl.name, flush=True)
    assert wl.max_blocks > 4096 and wl.rows * 16 > 32768
    check_prefill(wl, sorted(set([0, 1, 31, 2047, 2048, 2049, 2080, 2099] + list(range(5, 2100, 233)))))


def test_prefill_maximum_context():
    """The longest context the prefill scoring accepts: 32768 blocks (a
    1,048,576-token context) in 64 splits of 512 blocks, so list entries carry
    the widest (9-bit) in-split block ids; a ragged 600-row chunk ending at
    the context's last token.  The attention takes the row-major gather (the
    block-major workspace covers at most 16384 blocks)."""
    S = 32768 * 32
    wl = W.prefill_case("prefill S=1048576 q_start=1047976 T=600", 0xF9, S, S - 600, 600)
    print("case:", wl.name, flush=True)
    cfg = G.cfg_for(wl)
    assert U.workspace_size(cfg, U.OP_ATTN_PREFILL, wl.rows, wl.max_blocks) == 0
    check_prefill(wl, [0, 1, 31, 32, 299, 511, 512, 599], block_major=False)


def test_prefill_nan_key_in_candidate_block_ranks_last():
    """As the decode case: a NaN indexer key makes its block's score NaN in
    the MFMA scoring too, and that block ranks last for every row."""
    wl = W.prefill_case("prefill NaN key", 0xF7, 3000, 2200, 300)
    print("case:", wl.name, flush=True)
    cfg_u, cfg_o = G.cfg_for(wl), G.ocfg()
    dev = SD.generate(wl)
    tab = dev.block_table.cpu().numpy()
    S = int(wl.ctx_lens[0])
    kid = wl.kidx(0, 0, 0, S).copy()
    nan_blocks = [3, 50]
    for j, i in zip(nan_blocks, [9, 0]):
        kid[32 * j + i, 100] = 0x7FC0
        dev.kidx[0][int(tab[0, j]), i, 100] = 0x7FC0
    torch.cuda.synchronize()
    res = G.gpu_prefill(dev, cfg_u)
    rows = list(range(0, wl.rows, 7)) + [wl.rows - 1]
    allrows = np.arange(wl.rows)
    refs = oracle.prefill_rows_fetch(wl.q_rows(allrows), wl.q_idx_rows(allrows), kid, G.fetcher(wl, 0, 0),
                                     wl.q_start, rows, cfg_o)
    for r in refs:
        t = r["row"]
        G.check_selection(res["idx"][t], r, cfg_u.topk_blocks)
        for j in nan_blocks:
            assert np.isnan(r["block_scores"][j])
            assert j not in r["selected"] and j not in res["idx"][t]


def test_prefill_attention_block_major_matches_row_major_and_oracle():
    """The block-major prefill attention (pairs bucketed by block, per-slot
    partials, merge) against the row-major gather and the oracle, on index
    sets that stress the bucketing: the rows' own selections, then random
    sets with duplicates, -1 padding, out-of-range ids and blocks past p."""
    wl = W.prefill_case("prefill attention paths S=4700 q_start=3000 T=1700", 0xF8, 4700, 3000, 1700)
    print("case:", wl.name, flush=True)
    cfg_u, cfg_o = G.cfg_for(wl), G.ocfg()
    topk = cfg_u.topk_blocks
    dev = SD.generate(wl)
    res_b = G.gpu_prefill(dev, cfg_u)
    res_r = G.gpu_prefill(dev, cfg_u, idx_override=res_b["idx"], block_major=False)
    np.testing.assert_array_equal(res_b["idx"], res_r["idx"])
    assert np.abs(res_b["out"] - res_r["out"]).max() <= 1e-5
    assert np.abs(res_b["lse"] - res_r["lse"]).max() <= 1e-5

    g = np.random.default_rng(0xF8)
    T, M = wl.rows, wl.max_blocks
    idx = np.full((T, topk), -1, np.int32)
    for t in range(T):
        nb = (wl.q_start + t) // 32 + 1
        k = g.integers(0, topk + 1)
        idx[t, :k] = g.integers(-3, nb + 6, size=k)   # some past p, some negative, some repeated
    idx[5, :] = 7                                       # one block 16 times
    idx[6, :] = M + 3                                   # all out of range: empty set
    idx[7, :4] = [M - 1, M, 0, 0]
    res_b = G.gpu_prefill(dev, cfg_u, idx_override=idx)
    res_r = G.gpu_prefill(dev, cfg_u, idx_override=idx, block_major=False)
    assert np.abs(res_b["out"] - res_r["out"]).max() <= 1e-5
    fin = np.isfinite(res_r["lse"])
    np.testing.assert_array_equal(fin, np.isfinite(res_b["lse"]))
    assert np.abs(res_b["lse"][fin] - res_r["lse"][fin]).max() <= 1e-5
    assert np.all(res_b["out"][6] == 0) and np.all(np.isneginf(res_b["lse"][6]))
    allrows = np.arange(T)
    q = wl.q_rows(allrows)
    for t in list(range(0, T, 97)) + [5, 6, 7, T - 1]:
        p = wl.q_start + t
        sel = [int(j) for j in idx[t] if 0 <= j < M and j * 32 <= p]   # duplicates attend twice
        if not sel:
            continue
        toks = np.concatenate([oracle.attended_tokens([j], p, cfg_o) for j in sel])
        k_, v_ = G.fetcher(wl, 0, 0)(toks)
        o2, l2 = oracle.attend(q[t], k_, v_, np.arange(toks.size), cfg_o.sm_scale)
        G.check_attention(res_b["out"][t], res_b["lse"][t], o2, l2)


def test_prefill_block_major_unaligned_block_idx():
    """block_idx at a 4-byte offset (not 16-byte aligned) sends the bucketing
    down its narrow-load path: the output equals the aligned call's bit for
    bit (each pair's partial has its own slot, so the order of the pairs in
    a bucket never reaches the result), and both match the oracle."""
    wl = W.prefill_case("prefill unaligned block_idx S=4700 q_start=3000 T=1700", 0xFA, 4700, 3000, 1700)
    print("case:", wl.name, flush=True)
    cfg_u, cfg_o = G.cfg_for(wl), G.ocfg()
    topk = cfg_u.topk_blocks
    dev = SD.generate(wl)
    res = G.gpu_prefill(dev, cfg_u)
    T, M, H, D = wl.rows, wl.max_blocks, wl.heads, wl.head_dim
    buf = torch.full((T * topk + 1,), -7, dtype=torch.int32, device="cuda")
    idx_u = buf[1:].view(T, topk)
    idx_u.copy_(torch.from_numpy(res["idx"]).cuda())
    assert idx_u.data_ptr() % 16 != 0
    ab = U.workspace_size(cfg_u, U.OP_ATTN_PREFILL, T, M)
    aws = torch.full((ab,), 0x3C, dtype=torch.uint8, device="cuda")
    out = torch.full((T, H, D), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    U.sparse_attn_prefill(cfg_u, dev.kv(0), dev.q, wl.q_start, T, idx_u, out, lse, ws=aws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), res["out"])
    np.testing.assert_array_equal(lse.cpu().numpy(), res["lse"])
    allrows = np.arange(T)
    q = wl.q_rows(allrows)
    for t in range(0, T, 211):
        got = [int(x) for x in res["idx"][t] if x >= 0]
        o2, l2 = G.oracle_attend_with(wl, 0, 0, q[t], got, wl.q_start + t, cfg_o)
        G.check_attention(res["out"][t], res["lse"][t], o2, l2)


def test_prefill_attention_graph_capture_and_concurrent_streams():
    """The block-major prefill attention forks its window pass onto a second
    stream and joins it back: captured in a HIP graph and replayed with eager
    work in between, and called on two streams at once with their own
    workspaces, it gives the eager results bit for bit."""
    wl = W.prefill_case("prefill attention graph S=9000 q_start=7000 T=1500", 0xFA, 9000, 7000, 1500)
    print("case:", wl.name, flush=True)
    cfg = G.cfg_for(wl)
    dev = SD.generate(wl)
    ref = G.gpu_prefill(dev, cfg)
    T, M, H, D = wl.rows, wl.max_blocks, wl.heads, wl.head_dim
    kv = dev.kv(0)
    idx = torch.from_numpy(ref["idx"]).cuda()
    ab = U.workspace_size(cfg, U.OP_ATTN_PREFILL, T, M)
    aws = torch.zeros(ab, dtype=torch.uint8, device="cuda")
    out = torch.zeros((T, H, D), dtype=torch.float32, device="cuda")
    lse = torch.zeros((T, H), dtype=torch.float32, device="cuda")
    cap = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=cap):
        U.sparse_attn_prefill(cfg, kv, dev.q, wl.q_start, T, idx, out, lse, ws=aws, stream=cap.cuda_stream)
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        aws.fill_(0xA5)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(out.cpu().numpy().view(np.uint32), ref["out"].view(np.uint32))
        np.testing.assert_array_equal(lse.cpu().numpy().view(np.uint32), ref["lse"].view(np.uint32))
        G.gpu_prefill(dev, cfg)  # eager work between replays
    # two calls at once on two streams, each with its own workspace and outputs
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    aws2 = torch.zeros(ab, dtype=torch.uint8, device="cuda")
    out2 = torch.full((T, H, D), float("nan"), dtype=torch.float32, device="cuda")
    lse2 = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    out.fill_(float("nan"))
    lse.fill_(float("nan"))
    torch.cuda.synchronize()
    for _ in range(3):
        U.sparse_attn_prefill(cfg, kv, dev.q, wl.q_start, T, idx, out, lse, ws=aws, stream=s1.cuda_stream)
        U.sparse_attn_prefill(cfg, kv, dev.q, wl.q_start, T, idx, out2, lse2, ws=aws2, stream=s2.cuda_stream)
    torch.cuda.synchronize()
    for o, l in ((out, lse), (out2, lse2)):
        np.testing.assert_array_equal(o.cpu().numpy().view(np.uint32), ref["out"].view(np.uint32))
        np.testing.assert_array_equal(l.cpu().numpy().view(np.uint32), ref["lse"].view(np.uint32))
