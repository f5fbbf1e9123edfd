"""GPU parity of the dense full-context decode attention (the comparator for
the pages' per-step speed claim against full attention, leheavengame.com OCR
2 release article Sec. 1) against the CPU oracle's attention over every token
0..p, through the C ABI."""
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


def gpu_dense(dev, cfg):
    wl = dev.wl
    B, M, H, D = wl.batch, wl.max_blocks, wl.heads, wl.head_dim
    nbytes = U.workspace_size(cfg, U.OP_DENSE_ATTN_DECODE, B, M)
    ws = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device="cuda")
    out = torch.full((B, H, D), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, H), float("nan"), dtype=torch.float32, device="cuda")
    U.dense_attn_decode(cfg, dev.kv(0), dev.q[0], out, lse, ws=ws)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("lens", [[0, 1, 31, 32, 33, 100, 2048, 2049, 5000],
                                  [20000, 32768, 12345]])
def test_dense_attention_matches_oracle(lens):
    wl = _wl("dense comparator", 0xC1 + len(lens), lens)
    print("case: dense decode attention", lens, flush=True)
    dev = SD.generate(wl)
    cfg_u, cfg_o = G.cfg_for(wl), G.ocfg()
    out, lse = gpu_dense(dev, cfg_u)
    for b, L in enumerate(lens):
        toks = np.arange(L, dtype=np.int64)
        k, v = G.fetcher(wl, 0, b)(toks)
        ro, rl = oracle.attend(wl.q(0, b), k, v, np.arange(L), cfg_o.sm_scale)
        G.check_attention(out[b], lse[b], ro, rl)


def test_dense_equals_sparse_when_every_block_is_kept():
    """With topk_blocks >= the block count the sparse path keeps every block,
    so both GPU paths compute the same dense attention (to rounding)."""
    lens = [300, 511, 4000, 1]
    wl = _wl("dense vs sparse", 0xC7, lens)
    print("case: dense vs sparse with topk = all blocks", flush=True)
    dev = SD.generate(wl)
    cfg = U.make_cfg(topk_blocks=128, local_blocks=4)
    out_d, lse_d = gpu_dense(dev, cfg)
    res = G.gpu_decode(dev, 0, cfg)
    for b in range(len(lens)):
        G.check_attention(res["out"][b], res["lse"][b], out_d[b].astype(np.float64), lse_d[b].astype(np.float64))
