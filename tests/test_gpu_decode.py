"""GPU parity of the decode path (indexer score + block max, top-k selection,
sparse attention) against the CPU oracle, through the C ABI."""
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


def _wl(name, seed, lens, layers=1, values="normal"):
    lens = np.asarray(lens, np.int64)
    return W.Workload(name=name, seed=seed, batch=len(lens), layers=layers, ctx_lens=lens,
                      max_blocks=int(max(1, -(-int(lens.max()) // 32))), values=values)


def test_single_sequence_s2048():
    wl = W.config1()
    print("case: decode S=2048 B=1", flush=True)
    dev = SD.generate(wl)
    G.full_decode_check(dev, wl, 0, 0, [0], G.cfg_for(wl), G.ocfg())


def test_edge_lengths_ragged_batch():
    lens = [0, 1, 31, 32, 33, 127, 128, 129, 160, 511, 512, 513, 544, 1000, 4095, 4096, 4097]
    wl = _wl("edge lengths", 0xE1, lens)
    print("case: decode edge lengths", lens, flush=True)
    dev = SD.generate(wl)
    G.full_decode_check(dev, wl, 0, 0, range(wl.batch), G.cfg_for(wl), G.ocfg())


def test_batches_at_and_above_256_sequences():
    """The decode indexer numbers only the live (sequence, chunk) units for
    batches of up to 256 sequences and takes every unit above that: a
    256-sequence and a 300-sequence batch of short, ragged contexts (empty
    ones and ones inside the local window included), checked on a sample of
    sequences (every score, -inf entries included; selection; attention)."""
    g = np.random.default_rng(0xE9)
    for B in (256, 300):
        lens = g.integers(0, 3000, B)
        lens[:6] = [0, 1, 100, 129, 2999, 0]
        wl = _wl(f"decode batch {B}", 0xE9 + B, lens)
        print("case:", wl.name, flush=True)
        dev = SD.generate(wl)
        seqs = sorted(set([0, 1, 2, 3, 4, 5, B - 1] + [int(x) for x in g.choice(B, 20, replace=False)]))
        G.full_decode_check(dev, wl, 0, 0, seqs, G.cfg_for(wl), G.ocfg())


def test_several_tiles_and_ragged_tail():
    wl = _wl("ragged 3 seqs", 0xE2, [32768, 20001, 9999], layers=2)
    print("case: decode ragged S<=32768, 2 layers", flush=True)
    dev = SD.generate(wl)
    for li in range(2):
        G.full_decode_check(dev, wl, li, li, range(wl.batch), G.cfg_for(wl), G.ocfg())


def test_small_integer_inputs_exact():
    """Integer-valued bf16 inputs: every float32 dot is exact, so block scores
    match bit for bit and the many exact ties pin the lowest-id rule."""
    wl = _wl("small ints", 0xE3, [3000, 2049, 7777, 600], values="small_int")
    print("case: decode small-int exact", flush=True)
    dev = SD.generate(wl)
    cfg_u, cfg_o = G.cfg_for(wl), G.ocfg()
    res = G.gpu_decode(dev, 0, cfg_u)
    ties = 0
    for b in range(wl.batch):
        ref = G.oracle_decode(wl, 0, b, cfg_o)
        ncand = ref["block_scores"].size
        np.testing.assert_array_equal(res["scores"][b, :ncand], ref["block_scores"])
        got = [int(x) for x in res["idx"][b] if x >= 0]
        assert got == ref["selected"]
        ties += int(np.sum(ref["block_scores"] == ref["cutoff"]) >= 2)
        G.check_attention(res["out"][b], res["lse"][b], ref["out"], ref["lse"])
    assert ties >= 1, "the case should exercise a tie at the cutoff"


@pytest.mark.parametrize("topk,local", [(16, 4), (4, 4), (8, 1), (200, 4), (64, 4)])
def test_topk_variants(topk, local):
    wl = _wl(f"topk {topk} local {local}", 0xE4 + topk, [32768, 2048, 700, 6000])
    print(f"case: decode topk={topk} local={local}", flush=True)
    dev = SD.generate(wl)
    G.full_decode_check(dev, wl, 0, 0, range(wl.batch), G.cfg_for(wl, topk, local), G.ocfg(topk, local))


def test_topk_all_blocks_is_dense_attention():
    wl = W.config1()
    cfg_u = G.cfg_for(wl, topk=64)
    res = G.gpu_decode(SD.generate(wl), 0, cfg_u)
    assert list(res["idx"][0]) == list(range(64))
    L = 2048
    q = wl.q(0, 0)
    k = wl.kv(W.ROLE_K, 0, 0, 0, L)
    v = wl.kv(W.ROLE_V, 0, 0, 0, L)
    qf = oracle.widen(q)
    want = np.zeros((10, 128))
    want_lse = np.zeros(10)
    for h in range(10):
        z = oracle.widen(k[h]) @ qf[h] / np.sqrt(128.0)
        w = np.exp(z - z.max())
        want[h] = (w / w.sum()) @ oracle.widen(v[h])
        want_lse[h] = z.max() + np.log(w.sum())
    G.check_attention(res["out"][0], res["lse"][0], want, want_lse)


def test_topk_kernel_ties_nan_signed_zero():
    """Block scores supplied directly: ties, NaN, -0.0/+0.0, -inf."""
    cfg_u, cfg_o = U.make_cfg(), G.ocfg()
    rng = np.random.default_rng(5)
    B, M = 6, 300
    lens = np.array([300 * 32, 290 * 32 - 5, 40 * 32, 17 * 32, 16 * 32, 1], np.int32)
    sc = rng.integers(-3, 3, (B, M)).astype(np.float32)
    sc[0, ::7] = np.nan
    sc[1, :50] = -0.0
    sc[1, 50:100] = 0.0
    sc[1, 100:] = -1.0
    sc[2, :] = -np.inf
    sc[2, 5] = 1.0
    sc[3, :] = np.nan
    sc[4, :] = 7.0
    scores = torch.from_numpy(sc).cuda()
    ctx = torch.from_numpy(lens).cuda()
    idx = torch.full((B, 16), -9, dtype=torch.int32, device="cuda")
    nsel = torch.full((B,), -9, dtype=torch.int32, device="cuda")
    U.block_topk_decode(cfg_u, scores, ctx, B, M, idx, nsel)
    torch.cuda.synchronize()
    idx = idx.cpu().numpy()
    for b in range(B):
        p = int(lens[b]) - 1
        ref = oracle.select_blocks(sc[b, : oracle.candidate_count(p, cfg_o)], p, cfg_o)
        got = [int(x) for x in idx[b] if x >= 0]
        assert got == ref["selected"], (b, got, ref["selected"])
        assert nsel[b].item() == min(16, p // 32 + 1)


@pytest.mark.parametrize("M,topk,pattern", [
    (4100, 16, "normal"),      # 256-thread register variant, full
    (10000, 16, "normal"),     # 1024-thread register variant
    (20000, 16, "normal"),     # generic variant (scores re-read per pass)
    (2000, 16, "all_equal"),   # > 512 ties at the cutoff: ordered compaction
    (3000, 600, "normal"),     # R > 512: ordered compaction
    (3000, 600, "int"),        # R > 512 with ties
    (20000, 40, "int"),        # generic variant with ties
])
def test_topk_kernel_variants_direct(M, topk, pattern):
    cfg_u, cfg_o = U.make_cfg(topk_blocks=topk), G.ocfg(topk=topk)
    rng = np.random.default_rng(M + topk)
    B = 3
    lens = np.array([M * 32, M * 32 - 40, (M // 2) * 32 + 7], np.int32)
    if pattern == "normal":
        sc = rng.standard_normal((B, M)).astype(np.float32)
    elif pattern == "int":
        sc = rng.integers(-4, 4, (B, M)).astype(np.float32)
    else:
        sc = np.full((B, M), 2.5, np.float32)
    scores = torch.from_numpy(sc).cuda()
    ctx = torch.from_numpy(lens).cuda()
    idx = torch.full((B, topk), -9, dtype=torch.int32, device="cuda")
    U.block_topk_decode(cfg_u, scores, ctx, B, M, idx)
    torch.cuda.synchronize()
    idx = idx.cpu().numpy()
    for b in range(B):
        p = int(lens[b]) - 1
        ref = oracle.select_blocks(sc[b, : oracle.candidate_count(p, cfg_o)], p, cfg_o)
        got = [int(x) for x in idx[b] if x >= 0]
        assert got == ref["selected"], (b, got[:20], ref["selected"][:20])


def test_deterministic_and_order_free():
    wl = _wl("determinism", 0xE5, [20000, 5000])
    dev = SD.generate(wl)
    cfg_u = G.cfg_for(wl)
    a = G.gpu_decode(dev, 0, cfg_u)
    b = G.gpu_decode(dev, 0, cfg_u)
    for k in ("scores", "idx", "out", "lse"):
        np.testing.assert_array_equal(a[k], b[k])
    # The kept blocks in reverse order, mixed with -1 and out-of-range ids
    # (which the kernel skips), give the same attention.
    extra = np.array([[-1, wl.max_blocks + 5, -3, 10**6]] * 2, np.int32)
    perm = np.concatenate([a["idx"][:, ::-1], extra], axis=1)
    perm = perm[:, [0, 16, 1, 17, 2, 3, 18, 4, 5, 6, 7, 8, 19, 9, 10, 11, 12, 13, 14, 15]]
    out, lse = G.gpu_attn_decode(dev, 0, G.cfg_for(wl, topk=20), perm)
    np.testing.assert_allclose(out, a["out"], rtol=0, atol=1e-6)
    np.testing.assert_allclose(lse, a["lse"], rtol=0, atol=1e-6)


def test_device_generator_matches_host():
    wl = _wl("generator", 0xE6, [1000, 777, 64], layers=2)
    wl.edits = W.planted_edits(wl, 5.0, per_query=3)
    assert wl.edits
    h = SD.from_host(wl)
    d = SD.generate(wl)
    torch.cuda.synchronize()
    for name in ("k", "v", "kidx", "q", "q_idx", "block_table", "ctx_lens"):
        assert torch.equal(getattr(h, name), getattr(d, name)), name


def test_planted_query_selects_planted_blocks():
    wl = W.config3(batch=2, layers=1, S=32768)
    dev = SD.generate(wl)
    res = G.gpu_decode(dev, 0, G.cfg_for(wl))
    for e in wl.edits:
        got = [int(x) for x in res["idx"][e.seq] if x >= 0]
        assert got[:12] == sorted((e.tokens // 32).tolist())


@pytest.mark.parametrize("lens,topk,local", [
    ([0, 1, 31, 32, 33, 127, 128, 129, 511, 512, 513, 4095, 4097], 16, 4),
    ([32768, 20001, 9999, 700], 16, 4),
    ([32768, 5000], 64, 4),
    ([32768, 3000], 256, 8),
    ([140000, 70000, 1000], 16, 4),      # > 4096 candidates: 16 keys per thread
])
def test_fused_select_attention_equals_separate_calls(lens, topk, local):
    wl = _wl(f"fused {topk}", 0xE7 + topk, lens)
    print("case: fused selection+attention", lens, topk, local, flush=True)
    dev = SD.generate(wl)
    cfg = G.cfg_for(wl, topk, local)
    ref = G.gpu_decode(dev, 0, cfg)
    B, H, D = wl.batch, wl.heads, wl.head_dim
    scores = torch.from_numpy(ref["scores"]).cuda()
    idx = torch.full((B, topk), -7, dtype=torch.int32, device="cuda")
    nsel = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    out = torch.full((B, H, D), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, H), float("nan"), dtype=torch.float32, device="cuda")
    U.topk_attn_decode(cfg, dev.kv(0), dev.q[0], scores, idx, out, lse, n_sel=nsel)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(idx.cpu().numpy(), ref["idx"])
    np.testing.assert_array_equal(nsel.cpu().numpy(), ref["nsel"])
    np.testing.assert_array_equal(out.cpu().numpy(), ref["out"])
    np.testing.assert_array_equal(lse.cpu().numpy(), ref["lse"])


def test_fused_select_attention_rejects_unsupported():
    cfg = U.make_cfg(topk_blocks=300)
    wl = _wl("fused unsupported", 0xE8, [1000])
    dev = SD.generate(wl)
    with pytest.raises(U.UocrError) as e:
        U.topk_attn_decode(cfg, dev.kv(0), dev.q[0], torch.zeros(1, wl.max_blocks, device="cuda"),
                           torch.zeros(1, 300, dtype=torch.int32, device="cuda"),
                           torch.zeros(1, 10, 128, device="cuda"))
    assert e.value.status == 5


def test_nan_key_in_candidate_block_ranks_last():
    """A NaN indexer key inside a remote candidate block: the block max over
    its 32 scores is NaN, and a NaN score ranks last (news.rkmt.cn/news/25027
    Sec. 5 step 2, the block score as the maximum of its keys' scores; the
    ranking rule for NaN is this path's documented reading).  Oracle and
    kernel must agree on which blocks are NaN and on the selection."""
    wl = _wl("nan key", 0xE7, [4000, 3000])
    print("case: decode NaN indexer key in candidate blocks", flush=True)
    dev = SD.generate(wl)
    cfg_u, cfg_o = G.cfg_for(wl), G.ocfg()
    tab = dev.block_table.cpu().numpy()
    planted = {0: [(5, 3), (40, 31)], 1: [(0, 0), (70, 17)]}  # (block, key in block)
    kidx_host = {}
    for b, lst in planted.items():
        kid = wl.kidx(0, b, 0, int(wl.ctx_lens[b])).copy()
        for j, i in lst:
            kid[32 * j + i, 7] = 0x7FC0  # one NaN dimension
            dev.kidx[0][int(tab[b, j]), i, 7] = 0x7FC0
        kidx_host[b] = kid
    torch.cuda.synchronize()
    res = G.gpu_decode(dev, 0, cfg_u)
    for b, lst in planted.items():
        ref = G.oracle_decode(wl, 0, b, cfg_o, kidx=kidx_host[b])
        G.check_scores(res["scores"][b], ref, wl.q_idx(0, b), kidx_host[b], wl.max_blocks)
        G.check_selection(res["idx"][b], ref, cfg_u.topk_blocks)
        for j, _ in lst:
            assert np.isnan(ref["block_scores"][j]) and np.isnan(res["scores"][b, j])
            assert j not in ref["selected"] and j not in res["idx"][b]
