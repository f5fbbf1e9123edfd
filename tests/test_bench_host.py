"""Host checks of bench.py that need no GPU: the algorithmic bytes behind
the decode roofline, counted from the method's steps (news.rkmt.cn/news/25027
Sec. 5) with the oracle's block bookkeeping, the band rule of the bench's
parity record, and the one-GPU guard."""
import importlib.util
import os
import subprocess
import sys

import oracle
from synth import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_headline_step_bytes():
    """16 sequences x 12 layers at 131072 tokens: per (layer, sequence) the
    indexer reads every candidate block's 32 x 128 bf16 keys and table entry,
    the indexer query and the length, and writes a score per block; the
    selection reads the candidate scores and the length and writes 16 ids; the
    attention reads K and V of the 512 attended tokens for 10 heads, q, the
    ids and their table entries, the length, and writes out and lse."""
    wl = W.config3()
    cfg = oracle.SparseCfg()
    H, D, Di = 10, 128, 128
    total = 0
    for b in range(wl.batch):
        p = int(wl.ctx_lens[b]) - 1
        ncand = oracle.candidate_count(p, cfg)
        kept = list(range(cfg.topk_blocks - cfg.local_blocks)) + oracle.local_blocks(p, cfg)
        ntok = oracle.attended_tokens(kept, p, cfg).size
        assert ntok == 512
        indexer = ncand * (cfg.block_size * Di * 2 + 4) + Di * 2 + 4 + wl.max_blocks * 4
        topk = ncand * 4 + 4 + cfg.topk_blocks * 4
        attn = 2 * ntok * H * D * 2 + H * D * 2 + cfg.topk_blocks * 4 * 2 + 4 + H * D * 4 + H * 4
        total += indexer + topk + attn
    total *= wl.layers
    assert total == 6_950_477_568
    assert sum(_bench().decode_bytes(wl)) * wl.layers == total


def test_prefill_chunk_flops():
    """2048 rows at offset 129024 of a 131072-token context: each row scores
    the 32 keys of each of its candidate blocks with a 128-dim dot product."""
    wl = W.config5()
    cfg = oracle.SparseCfg()
    flops = sum(oracle.candidate_count(wl.q_start + t, cfg) * cfg.block_size * 128 * 2 for t in range(wl.rows))
    assert flops == 68_123_885_568
    assert _bench().prefill_flops(wl) == flops


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr


def _tiny_query(seed=7, L=1500, H=10, D=128):
    """One decode query over an L-token context (47 blocks) from the synth
    generator's bf16 rounding; K/V fetched from host arrays."""
    import numpy as np
    g = np.random.default_rng(seed)

    def bf16(x):
        b = np.asarray(x, np.float32).view(np.uint32)
        return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)

    q, qi = bf16(g.standard_normal((H, D))), bf16(g.standard_normal(D))
    kidx = bf16(g.standard_normal((L, D)))
    k, v = bf16(g.standard_normal((H, L, D))), bf16(g.standard_normal((H, L, D)))
    fetch = lambda toks: (k[:, toks, :], v[:, toks, :])
    return q, qi, kidx, fetch, L


def test_parity_tally_band_rule():
    """The bench's parity record: the oracle's own result is exact; a GPU
    selection that swaps the cutoff block for an unselected block whose score
    lies within the 1e-4 band is accepted (its attention is checked against
    the oracle recomputed on that set), outside the band it is a mismatch;
    attention off by more than the tolerance fails."""
    import numpy as np
    bench = _bench()
    cfg = oracle.SparseCfg()
    q, qi, kidx, fetch, L = _tiny_query()
    p = L - 1
    ref = oracle.decode_query_fetch(q, qi, kidx, fetch, L, cfg)
    sel = ref["selected"]
    idx_row = np.array(sel + [-1] * (cfg.topk_blocks - len(sel)), np.int32)

    t = bench.ParityTally()
    t.add("exact", ref, idx_row, ref["out"].astype(np.float32), ref["lse"].astype(np.float32), q, fetch, p, cfg)
    assert t.record()["pass"] and t.exact == 1

    # the remote block at the cutoff, and the best unselected candidate
    remote = [j for j in sel if j not in ref["local"]]
    bs = ref["block_scores"].astype(np.float64)
    j_cut = min(remote, key=lambda j: (bs[j], -j))
    out_blocks = [j for j in range(oracle.candidate_count(p, cfg)) if j not in sel]
    j_in = max(out_blocks, key=lambda j: bs[j])
    got = sorted(set(sel) - {j_cut} | {j_in})
    toks = oracle.attended_tokens(got, p, cfg)
    k, v = fetch(toks)
    o2, l2 = oracle.attend(q, k, v, np.arange(toks.size), cfg.sm_scale)
    row = np.array(got + [-1] * (cfg.topk_blocks - len(got)), np.int32)

    near = dict(ref)
    near["block_scores"] = ref["block_scores"].copy()
    near["block_scores"][j_in] = np.float32(ref["cutoff"] * (1 - 5e-5 * np.sign(ref["cutoff"])))
    t = bench.ParityTally()
    t.add("in band", near, row, o2.astype(np.float32), l2.astype(np.float32), q, fetch, p, cfg)
    r = t.record()
    assert r["pass"] and r["selection_differences_inside_band"] == 1, r

    t = bench.ParityTally()
    t.add("outside band", ref, row, o2.astype(np.float32), l2.astype(np.float32), q, fetch, p, cfg)
    r = t.record()
    assert not r["pass"] and r["selection_mismatches_outside_band"] == 1

    bad = ref["out"].astype(np.float32).copy()
    bad[3, 5] += 5e-3
    t = bench.ParityTally()
    t.add("attention", ref, idx_row, bad, ref["lse"].astype(np.float32), q, fetch, p, cfg)
    r = t.record()
    assert not r["pass"] and r["attention_on_gpu_selection"]["max_abs"] > 4e-3
