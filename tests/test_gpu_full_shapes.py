"""Oracle parity of the five measured workloads at their own shapes, through
the C ABI (news.rkmt.cn/news/25027 Sec. 5 steps 2-4): every decode query of
the 16 x 12 x 32K and 16 x 12 x 128K steps (the latter also with the
literal +4 sigma planting), every sequence of the 64-document ragged batch
with and without page tags, and 256 rows of the 2048-row prefill chunk at
129024 of 131072, spread over every row tile and every row position inside a
32-token block.  The oracle takes the device inputs themselves (copied to
the host), and each query is checked for its block scores, its selection
(band rule), the GPU's attention on the GPU's selection and the GPU's
attention on the oracle's own index set.  Also: the prefill path repeats bit
for bit."""
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


def _release(*objs):
    del objs
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _same_selection(a, b, what):
    np.testing.assert_array_equal(a["scores"].view(np.uint32), b["scores"].view(np.uint32), err_msg=what + " scores")
    np.testing.assert_array_equal(a["idx"], b["idx"], err_msg=what + " selection")
    np.testing.assert_allclose(a["out"], b["out"], rtol=0, atol=1e-5, err_msg=what + " attention")


def _every_query(wl):
    return [(li, b) for li in range(wl.layers) for b in range(wl.batch)]


def test_config2_every_query():
    """16 sequences x 12 layers at 32768 tokens: all 192 query-layers, with
    the automatic schedule (per-layer launches at this size) and the one
    launch."""
    _release()
    wl = W.config2()
    print("case:", wl.name, flush=True)
    dev = SD.generate(wl)
    cfg = G.cfg_for(wl)
    res = G.gpu_decode_step(dev, cfg, U.STEP_AUTO)
    summary = G.check_decode_full(dev, res, _every_query(wl), cfg, G.ocfg())
    print("config 2:", summary, flush=True)
    one = G.gpu_decode_step(dev, cfg, U.STEP_ONE_LAUNCH)
    assert one["err"] == 0
    _same_selection(one, res, "one launch vs per-layer")
    _release(dev)


@pytest.mark.parametrize("sigmas", [None, 4.0], ids=["planted_above_noise", "planted_literal_4sigma"])
def test_config3_every_query(sigmas):
    """16 sequences x 12 layers at 131072 tokens (the headline step, one
    launch): all 192 query-layers.  ``planted_literal_4sigma`` moves the
    planted keys by 4 sigma exactly, below the noise ceiling of 128K keys,
    so many blocks sit near the cutoff."""
    _release()
    wl = W.config3(sigmas=sigmas)
    print("case:", wl.name, wl.notes, flush=True)
    dev = SD.generate(wl)
    cfg = G.cfg_for(wl)
    res = G.gpu_decode_step(dev, cfg, U.STEP_ONE_LAUNCH)
    assert res["err"] == 0
    summary = G.check_decode_full(dev, res, _every_query(wl), cfg, G.ocfg())
    print("config 3", wl.notes, summary, flush=True)
    _release(dev)


def test_config4_every_sequence_plain_and_page_tags():
    """64 ragged multi-page documents, 1 layer: every sequence, plain ranking
    and page-aware ranking, through the automatic schedule (per-layer
    launches), the one launch and the three separate entry points."""
    _release()
    wl = W.config4()
    print("case:", wl.name, flush=True)
    dev = SD.generate(wl)
    cfg = G.cfg_for(wl)
    tags = np.tile(W.page_tags(wl.max_blocks), (wl.batch, 1)).astype(np.int32)
    qpages = np.array([W.page_of(int(L) - 1) for L in wl.ctx_lens], np.int32)
    for t, q in ((None, None), (tags, qpages)):
        res = G.gpu_decode_step(dev, cfg, U.STEP_AUTO, t, q)
        summary = G.check_decode_full(dev, res, _every_query(wl), cfg, G.ocfg(), t, q)
        print("config 4", "page tags" if t is not None else "plain", summary, flush=True)
        one = G.gpu_decode_step(dev, cfg, U.STEP_ONE_LAUNCH, t, q)
        assert one["err"] == 0
        _same_selection(one, res, "one launch vs per-layer")
    sep = G.gpu_decode(dev, 0, cfg)
    plain = G.gpu_decode_step(dev, cfg, U.STEP_AUTO)
    _same_selection({k: sep[k][None] for k in ("scores", "idx", "out")}, plain, "separate entry points")
    _release(dev)


def _prefill_rows(T):
    # 8 rows per 64: one per row-in-block residue class over the chunk, every
    # row tile, both chunk ends
    rows = {8 * k + (k % 8) for k in range(T // 8)} | {0, 1, 31, 32, T - 1}
    return sorted(r for r in rows if r < T)


def test_config5_rows_every_tile():
    """The 2048-row chunk at 129024 of 131072 (64 context splits per row),
    block-major attention as measured: 256 rows against the oracle."""
    _release()
    wl = W.config5()
    print("case:", wl.name, flush=True)
    dev = SD.generate(wl)
    cfg_u, cfg_o = G.cfg_for(wl), G.ocfg()
    T, topk = wl.rows, cfg_u.topk_blocks
    res = G.gpu_prefill(dev, cfg_u)
    S = int(wl.ctx_lens[0])
    kidx = dev.host_kidx(0, 0, S)
    q, qi = dev.host_prefill_queries()
    fetch = dev.host_kv_fetch(0, 0)
    rows = _prefill_rows(T)
    assert len(rows) >= 256
    refs = oracle.prefill_rows_fetch(q, qi, kidx, fetch, wl.q_start, rows, cfg_o)
    idx_oracle = res["idx"].copy()
    differ = 0
    for r in refs:
        t = r["row"]
        assert res["nsel"][t] == min(topk, (wl.q_start + t) // 32 + 1)
        _, d = G.check_query_end_to_end(r, q[t], fetch, wl.q_start + t, cfg_o, res["idx"][t], res["out"][t],
                                        res["lse"][t])
        differ += int(d)
        idx_oracle[t] = G.pad_idx(r["selected"], topk)
    res_o = G.gpu_prefill(dev, cfg_u, idx_override=idx_oracle)
    for r in refs:
        t = r["row"]
        G.check_attention(res_o["out"][t], res_o["lse"][t], r["out"], r["lse"])
    print(f"config 5: {len(rows)} rows, {differ} selections differ inside the band", flush=True)
    _release(dev)


def test_prefill_path_repeats_bit_for_bit():
    """Scoring, merge and block-major attention of the 2048-row 128K chunk,
    run twice with differently filled workspaces: the bucketing's pair order
    comes from LDS atomics and may change, the results may not."""
    _release()
    wl = W.config5()
    print("case: prefill repeat,", wl.name, flush=True)
    dev = SD.generate(wl)
    cfg = G.cfg_for(wl)
    a = G.gpu_prefill(dev, cfg, fill=(0xA5, 0x5A))
    b = G.gpu_prefill(dev, cfg, fill=(0x00, 0xFF))
    for k in ("idx", "nsel"):
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)
    for k in ("out", "lse"):
        np.testing.assert_array_equal(a[k].view(np.uint32), b[k].view(np.uint32), err_msg=k)
    _release(dev)
