"""GPU test of uocr_sparse_decode_step_static, the decode step that allocates
nothing (its one-launch counters live in the library's static device
array): through the C ABI, two calls in a row -- the second with a smaller
batch, fewer layers and shorter contexts -- each against
uocr_sparse_decode_step with a workspace on the same inputs (the same
kernels: equal bit for bit) and sampled queries against the oracle
(news.rkmt.cn/news/25027 Sec. 5 steps 2-4)."""
from __future__ import annotations

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import block_sparse_long_sr_amd as U  # noqa: E402
from synth import device as SD  # noqa: E402
from synth import workloads as W  # noqa: E402
import gpu_harness as G  # noqa: E402


def _wl(name, seed, lens, layers):
    lens = np.asarray(lens, np.int64)
    return W.Workload(name=name, seed=seed, batch=len(lens), layers=layers, ctx_lens=lens,
                      max_blocks=int(max(1, -(-int(lens.max()) // 32))))


def run_static(dev, cfg, schedule):
    wl = dev.wl
    nl, B, M, H, D = dev.q.shape[0], wl.batch, wl.max_blocks, wl.heads, wl.head_dim
    topk = cfg.topk_blocks
    kv = U.make_kv(dev.k[0], dev.v[0], dev.kidx[0], dev.block_table, dev.ctx_lens, wl.pool_blocks, B, M)
    scores = torch.full((nl, B, M), float("nan"), dtype=torch.float32, device="cuda")
    idx = torch.full((nl, B, topk), -7, dtype=torch.int32, device="cuda")
    nsel = torch.full((nl, B), -7, dtype=torch.int32, device="cuda")
    out = torch.full((nl, B, H, D), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((nl, B, H), float("nan"), dtype=torch.float32, device="cuda")
    status = torch.full((1,), -5, dtype=torch.int32, device="cuda")
    U.sparse_decode_step_static(cfg, kv, nl, dev.q_idx, dev.q, scores, idx, out, lse, n_sel=nsel, status=status,
                                schedule=schedule)
    torch.cuda.synchronize()
    return {"scores": scores.cpu().numpy(), "idx": idx.cpu().numpy(), "nsel": nsel.cpu().numpy(),
            "out": out.cpu().numpy(), "lse": lse.cpu().numpy(), "status": int(status.cpu()[0])}


def _equal(a, b, what):
    for k in ("scores", "out", "lse"):
        np.testing.assert_array_equal(a[k].view(np.uint32), b[k].view(np.uint32), err_msg=f"{what}: {k}")
    for k in ("idx", "nsel"):
        np.testing.assert_array_equal(a[k], b[k], err_msg=f"{what}: {k}")


def test_static_scratch_step_matches_workspace_step_twice():
    big = _wl("static step: 16 seqs x 3 layers", 0x57A1, [0, 1, 33, 500, 4097, 9000, 20001, 31000, 1200, 65,
                                                       2049, 777, 16000, 128, 129, 40000], layers=3)
    small = _wl("static step: 5 seqs x 2 layers", 0x57A2, [3000, 31, 6000, 1, 2500], layers=2)
    for wl in (big, small):
        print("case:", wl.name, flush=True)
        dev = SD.generate(wl)
        cfg = G.cfg_for(wl)
        ref = G.gpu_decode_step(dev, cfg, U.STEP_ONE_LAUNCH)
        assert ref["err"] == 0
        got = run_static(dev, cfg, U.STEP_ONE_LAUNCH)
        assert got["status"] == 0
        _equal(got, ref, wl.name)
        # against the oracle on the device inputs (③'s bar), a few queries
        nl = wl.layers
        queries = [(0, 0), (nl - 1, wl.batch - 1), (nl // 2, wl.batch // 2), (0, wl.batch - 2)]
        G.check_decode_full(dev, got, queries, cfg, G.ocfg())
        # the per-layer schedule of the same entry point needs no counters
        per = run_static(dev, cfg, U.STEP_PER_LAYER)
        assert per["status"] == 0
        ref_per = G.gpu_decode_step(dev, cfg, U.STEP_PER_LAYER)
        _equal(per, ref_per, wl.name + " per layer")
        del dev
        torch.cuda.empty_cache()
