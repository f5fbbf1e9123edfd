"""Host checks of bench.py that need no GPU: the algorithmic bytes behind
the decode roofline, counted from the method's steps (news.rkmt.cn/news/25027
Sec. 5) with the oracle's block bookkeeping, and the one-GPU guard."""
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
