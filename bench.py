"""Benchmark of the SR-SWA block-sparse attention hot path on one MI355X.

Workload (the headline case): decode batch of 16 sequences x 12 layers at
S = 131072 tokens (4096 blocks of 32), 10 heads x 128 bf16 K/V, 1 x 128
indexer, 12 planted blocks per query, all resident in HBM (~135 GB).  One
step = for each of the 12 layers of each sequence, in layer order: indexer
score + block max, top-k block selection, sparse attention.  By default the
step is one uocr_sparse_decode_step launch (work items in ticket order,
layer l + 1 of a sequence after its layer l); --multi-launch runs it as
per-layer launches of the separate entry points on micro-batch streams.
``value`` is decode query-heads/s (16 * 12 * 10 per step).

The same JSON line carries the roofline of the dominant kernel (the
one-launch step kernel, HBM bound, or the decode indexer with
--multi-launch) timed with HIP events, the CPU oracle's throughput on a
bounded sample of the same workload, and the chunked-prefill case
(2048 rows at offset 129024 of a 131072-token context) with the MFMA
roofline of its scoring kernel.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse-attn decode query-heads/s at 128K ctx; achieved HBM GB/s vs peak"
HBM_PEAK_GBPS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
KERNEL_SOURCES = {
    "decode_step": ["block_sparse_long_sr_amd/csrc/decode_step.hip",
                    "block_sparse_long_sr_amd/csrc/indexer_common.h",
                    "block_sparse_long_sr_amd/csrc/attn_common.h",
                    "block_sparse_long_sr_amd/csrc/select_common.h",
                    "block_sparse_long_sr_amd/csrc/device_common.h"],
    "indexer_decode": ["block_sparse_long_sr_amd/csrc/indexer_decode.hip",
                       "block_sparse_long_sr_amd/csrc/indexer_common.h",
                       "block_sparse_long_sr_amd/csrc/device_common.h"],
    "indexer_prefill": ["block_sparse_long_sr_amd/csrc/indexer_prefill.hip",
                        "block_sparse_long_sr_amd/csrc/device_common.h"],
}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_digest(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def decode_bytes(wl, cfg_topk=16, local=4, heads=10, D=128, Di=128):
    """Algorithmic HBM bytes of one decode layer launch triple, per kernel."""
    idx_b = topk_b = attn_b = 0
    for b in range(wl.batch):
        L = int(wl.ctx_lens[b])
        nb = -(-L // 32)
        ncand = max(0, nb - local)
        # indexer: candidate key tiles + their table entries + q_idx + ctx + score row written
        idx_b += ncand * 32 * Di * 2 + ncand * 4 + Di * 2 + 4 + wl.max_blocks * 4
        # top-k: candidate scores read + ctx + ids written
        topk_b += ncand * 4 + 4 + cfg_topk * 4
        # attention: K and V of the attended tokens + q + ids + table + out + lse
        p = L - 1
        toks = 15 * 32 + (p % 32) + 1 if nb >= 16 else L
        attn_b += 2 * toks * heads * D * 2 + heads * D * 2 + cfg_topk * 4 * 2 + heads * D * 4 + heads * 4 + 4
    return idx_b, topk_b, attn_b


TRAFFIC_FILES = {"decode_step": "profiles/decode_step_128k_traffic.txt",
                 "indexer_decode": "profiles/indexer_score_decode_128k_traffic.txt",
                 "indexer_prefill": "profiles/indexer_score_prefill_2048_traffic.txt"}


def traffic_for(kernel):
    """Measured HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE,
    copy-calibrated) from the committed summary, or None when the summary is
    missing or was taken on a different kernel source."""
    path = os.path.join(ROOT, TRAFFIC_FILES[kernel])
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as f:
        for line in f:
            if line.startswith("#") or ":" not in line:
                continue
            k, v = line.split(":", 1)
            rec[k.strip()] = v.strip()
    if rec.get("source_digest") != source_digest(KERNEL_SOURCES[kernel]):
        return None
    return int(float(rec["hbm_bytes_per_launch"]))


def host_description():
    """The host the CPU oracle runs on: CPU model, cores this process may
    use, and the BLAS library numpy calls with its thread count."""
    from threadpoolctl import threadpool_info
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = [{"library": d.get("internal_api"), "version": d.get("version"), "threads": d.get("num_threads")}
            for d in threadpool_info() if d.get("user_api") == "blas"]
    return {"cpu_model": model, "affinity_cores": len(os.sched_getaffinity(0)), "os_cpu_count": os.cpu_count(),
            "blas": blas}


# Parity rule of the decode path against the oracle (the same rule the GPU
# tests apply): selections equal except blocks whose oracle score lies within
# 1e-4 relative of the cutoff (equal sizes, local blocks kept); attention
# max-abs <= 2e-3 and relative L2 <= 1e-3 per query, lse within 1e-4.
BAND, ATT_MAX_ABS, ATT_REL_L2, LSE_ABS = 1e-4, 2e-3, 1e-3, 1e-4


class ParityTally:
    """Per-query comparison of GPU selections and attention outputs with the
    oracle's, accumulated into the bench record."""

    def __init__(self):
        self.queries = 0
        self.exact = 0
        self.in_band = 0
        self.outside_band = 0
        self.failures = []
        self.att = {"max_abs": 0.0, "rel_l2": 0.0, "lse_abs": 0.0}
        self.att_oracle_set = {"max_abs": 0.0, "rel_l2": 0.0, "lse_abs": 0.0}

    @staticmethod
    def _errors(out, lse, ref_out, ref_lse):
        import numpy as np
        g = out.astype(np.float64)
        err = float(np.abs(g - ref_out).max()) if g.size else 0.0
        nrm = float(np.linalg.norm(ref_out))
        rel = float(np.linalg.norm(g - ref_out) / nrm) if nrm > 0 else float(np.linalg.norm(g))
        fin = np.isfinite(ref_lse)
        lerr = float(np.abs(lse[fin] - ref_lse[fin]).max()) if fin.any() else 0.0
        if not np.all(np.isneginf(lse[~fin])) or not np.all(np.isfinite(g)):
            lerr = float("inf")
        return err, rel, lerr

    def _attention(self, key, where, out, lse, ref_out, ref_lse):
        err, rel, lerr = self._errors(out, lse, ref_out, ref_lse)
        acc = self.att if key == "gpu" else self.att_oracle_set
        acc["max_abs"] = max(acc["max_abs"], err)
        acc["rel_l2"] = max(acc["rel_l2"], rel)
        acc["lse_abs"] = max(acc["lse_abs"], lerr)
        if not (err <= ATT_MAX_ABS and rel <= ATT_REL_L2 and lerr <= LSE_ABS):
            self.failures.append(f"{where}: attention ({key} set) max-abs {err:.2e} rel-L2 {rel:.2e} lse {lerr:.2e}")

    def add(self, where, ref, idx_row, out, lse, q, fetch, p, cfg_o):
        """One query: ``ref`` is the oracle's result; the GPU's selection
        ``idx_row`` and its attention on that selection (out, lse)."""
        import numpy as np
        import oracle
        self.queries += 1
        got = [int(x) for x in idx_row if x >= 0]
        want = ref["selected"]
        band = set()
        if ref["cutoff"] is not None:
            c = ref["cutoff"]
            band = set(np.nonzero(np.abs(ref["block_scores"].astype(np.float64) - c) <= BAND * abs(c))[0].tolist())
        well_formed = (got == sorted(got) and list(idx_row[len(got):]) == [-1] * (len(idx_row) - len(got))
                       and len(got) == len(want) and all(j in got for j in ref["local"]))
        if got == want:
            self.exact += 1
            self._attention("gpu", where, out, lse, ref["out"], ref["lse"])
        elif well_formed and set(got) - band == set(want) - band:
            self.in_band += 1
            toks = oracle.attended_tokens(got, p, cfg_o)
            k, v = fetch(toks)
            o2, l2 = oracle.attend(q, k, v, np.arange(toks.size), cfg_o.sm_scale)
            self._attention("gpu", where, out, lse, o2, l2)
        else:
            self.outside_band += 1
            self.failures.append(f"{where}: selection gpu {got} oracle {want}")

    def add_oracle_set(self, where, out, lse, ref_out, ref_lse):
        """The GPU's attention run on the oracle's own index set."""
        self._attention("oracle", where, out, lse, ref_out, ref_lse)

    def record(self):
        return {"queries": self.queries, "selection_exact": self.exact,
                "selection_differences_inside_band": self.in_band,
                "selection_mismatches_outside_band": self.outside_band,
                "attention_on_gpu_selection": self.att, "attention_on_oracle_selection": self.att_oracle_set,
                "tolerance": {"band_rel": BAND, "max_abs": ATT_MAX_ABS, "rel_l2": ATT_REL_L2, "lse_abs": LSE_ABS},
                "pass": not self.failures, "failures": self.failures[:8]}


def cpu_baseline(U, dev, wl, n_layers, gpu, cfg):
    """The CPU oracle on every (layer, sequence) query of the step, on the
    device inputs copied to the host: once with numpy's BLAS on all its
    threads (results kept) and once on one thread; the time spent copying
    inputs and fetching K/V rows is excluded.  The kept results are then
    compared with the GPU's outputs of the timed step (``gpu``: host copies
    of idx [L][B][topk], out [L][B][H][D], lse [L][B][H]), and the GPU's
    attention is run once more on the oracle's own index sets.  Returns
    (timing, parity record)."""
    import numpy as np
    import torch
    import oracle
    from threadpoolctl import threadpool_limits

    cfg_o = oracle.SparseCfg()
    B, H = wl.batch, wl.heads
    topk = cfg_o.topk_blocks
    t_all = t_one = 0.0
    nq = 0
    tally = ParityTally()
    idx_o = np.full((n_layers, B, topk), -1, np.int32)
    ref_att = {}
    for l in range(n_layers):
        for b in range(B):
            L = int(wl.ctx_lens[b])
            kidx = dev.host_kidx(l, b, L)
            q, qi = dev.host_decode_queries(l, b)
            base_fetch = dev.host_kv_fetch(l, b)
            fetch_time = [0.0]

            def fetch(toks):
                t0 = time.perf_counter()
                r = base_fetch(toks)
                fetch_time[0] += time.perf_counter() - t0
                return r

            fetch_time[0] = 0.0
            t0 = time.perf_counter()
            ref = oracle.decode_query_fetch(q, qi, kidx, fetch, L, cfg_o)
            t_all += time.perf_counter() - t0 - fetch_time[0]
            with threadpool_limits(limits=1):
                fetch_time[0] = 0.0
                t0 = time.perf_counter()
                oracle.decode_query_fetch(q, qi, kidx, fetch, L, cfg_o)
                t_one += time.perf_counter() - t0 - fetch_time[0]
            nq += 1
            tally.add(f"layer {l} seq {b}", ref, gpu["idx"][l, b], gpu["out"][l, b], gpu["lse"][l, b], q,
                      base_fetch, L - 1, cfg_o)
            idx_o[l, b, :len(ref["selected"])] = ref["selected"]
            ref_att[(l, b)] = (ref["out"], ref["lse"])
    out2 = torch.empty((B, H, 128), dtype=torch.float32, device="cuda")
    lse2 = torch.empty((B, H), dtype=torch.float32, device="cuda")
    for l in range(n_layers):
        U.sparse_attn_decode(cfg, dev.kv(l), dev.q[l], torch.from_numpy(idx_o[l]).cuda(), out2, lse2)
        o, s = out2.cpu().numpy(), lse2.cpu().numpy()
        for b in range(B):
            tally.add_oracle_set(f"layer {l} seq {b}", o[b], s[b], *ref_att[(l, b)])
    return {"queries": nq, "seconds_all_threads": t_all, "seconds_one_thread": t_one}, tally.record()


def micro_batch_step(U, torch, dev, cfg, bufs, n_groups, separate=False, base=None):
    """The decode step as per-layer launches over micro-batches: the batch is
    split into ``n_groups`` groups of sequences, each running its layers in
    order on its own HIP stream (default priority), so that one group's
    latency-bound selection + attention overlaps another group's
    bandwidth-bound scoring.  Each group calls the entry points on views of
    the batch (descriptor pointers offset by the group's first sequence).
    Returns (step, fork, join): fork(base) makes the group streams wait for
    ``base``, join(base) makes ``base`` wait for them.  With one group and
    ``base`` given, that group runs on ``base`` itself."""
    wl = dev.wl
    B, M, L = wl.batch, wl.max_blocks, dev.q.shape[0]
    scores, idx, out, lse = bufs
    ns = max(1, min(n_groups, B))
    bounds = [(B * i) // ns for i in range(ns + 1)]
    groups = []
    for i in range(ns):
        b0, b1 = bounds[i], bounds[i + 1]
        gkv = [U.make_kv(dev.k[l], dev.v[l], dev.kidx[l], dev.block_table[b0:b1], dev.ctx_lens[b0:b1],
                         wl.pool_blocks, b1 - b0, M) for l in range(L)]
        groups.append((b0, b1, gkv, base if (ns == 1 and base is not None) else torch.cuda.Stream()))

    def step():
        for l in range(L):
            for b0, b1, gkv, st in groups:
                h_ = st.cuda_stream
                U.indexer_score_decode(cfg, gkv[l], dev.q_idx[l, b0:b1], scores[l, b0:b1], stream=h_)
                if separate:
                    U.block_topk_decode(cfg, scores[l, b0:b1], dev.ctx_lens[b0:b1], b1 - b0, M, idx[l, b0:b1],
                                        stream=h_)
                    U.sparse_attn_decode(cfg, gkv[l], dev.q[l, b0:b1], idx[l, b0:b1], out[l, b0:b1],
                                         lse[l, b0:b1], stream=h_)
                else:
                    U.topk_attn_decode(cfg, gkv[l], dev.q[l, b0:b1], scores[l, b0:b1], idx[l, b0:b1],
                                       out[l, b0:b1], lse[l, b0:b1], stream=h_)

    def fork(base_):
        ev = torch.cuda.Event()
        ev.record(base_)
        for _, _, _, st in groups:
            if st is not base_:
                st.wait_event(ev)

    def join(base_):
        for _, _, _, st in groups:
            if st is not base_:
                ev = torch.cuda.Event()
                ev.record(st)
                base_.wait_event(ev)

    return step, fork, join


def time_steps(torch, stream, step, reps, warmup, fork=None, join=None):
    """Average duration (ms) of ``reps`` back-to-back steps after ``warmup``
    untimed ones: one event pair on ``stream`` around the whole run."""
    fork = fork or (lambda b: None)
    join = join or (lambda b: None)
    fork(stream)
    for _ in range(warmup):
        step()
    join(stream)
    torch.cuda.synchronize()
    a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a_.record(stream)
    fork(stream)
    for _ in range(reps):
        step()
    join(stream)
    b_.record(stream)
    torch.cuda.synchronize()
    return a_.elapsed_time(b_) / reps


def schedule_timings(U, torch, dev, cfg, bufs, step_ws, reps, warmup, step_bytes):
    """The same decode step under each schedule, on the same inputs: the one
    launch (every layer's queries given before it starts), per-layer
    launches on one stream, and per-layer launches over two micro-batch
    streams.  The per-layer schedules need each layer's queries only when
    that layer starts, as a model produces them."""
    wl = dev.wl
    B, L, H = wl.batch, dev.q.shape[0], wl.heads
    scores, idx, out, lse = bufs
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    kv0 = dev.kv(0)
    res = {}

    def lib_step(sched):
        return lambda: U.sparse_decode_step(cfg, kv0, L, dev.q_idx, dev.q, scores, idx, out, lse, ws=step_ws,
                                            stream=sh, schedule=sched)

    res["one_launch"] = time_steps(torch, stream, lib_step(U.STEP_ONE_LAUNCH), reps, warmup)
    res["per_layer_one_stream"] = time_steps(torch, stream, lib_step(U.STEP_PER_LAYER), reps, warmup)
    st2, fk, jn = micro_batch_step(U, torch, dev, cfg, bufs, 2)
    res["per_layer_two_streams"] = time_steps(torch, stream, st2, reps, warmup, fk, jn)
    return {k: {"us_per_step": v * 1e3, "query_heads_per_s": B * L * H / (v * 1e-3),
                "hbm_frac": step_bytes / (v * 1e-3) / 1e9 / HBM_PEAK_GBPS} for k, v in res.items()}


def prefill_flops(wl, local=4):
    """Algorithmic work of the prefill scoring kernel: a 128-dim bf16 dot
    product (2 x 128 FLOP) for every key of every candidate (row, block)."""
    rowblocks = sum(max(0, (wl.q_start + t) // 32 + 1 - local) for t in range(wl.rows))
    return rowblocks * 32 * 128 * 2


def run_prefill(U, SD, W, torch, iters=5):
    wl = W.config5()
    dev = SD.generate(wl)
    cfg = U.make_cfg()
    T, M = wl.rows, wl.max_blocks
    kv = dev.kv(0)
    ws_bytes = U.workspace_size(cfg, U.OP_INDEXER_PREFILL, T, M)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    wsarg = (ws.data_ptr(), ws_bytes)
    idx = torch.empty((T, 16), dtype=torch.int32, device="cuda")
    out = torch.empty((T, 10, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((T, 10), dtype=torch.float32, device="cuda")
    # block-major attention: (row, slot) pairs bucketed by block, per-slot partials, merge
    aws = torch.empty(U.workspace_size(cfg, U.OP_ATTN_PREFILL, T, M), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    def scoring():
        U.indexer_score_prefill(cfg, kv, dev.q_idx, wl.q_start, T, wsarg, stream=sh)

    def merge():
        U.block_topk_prefill(cfg, wsarg, wl.q_start, T, M, idx, stream=sh)

    def attention():
        U.sparse_attn_prefill(cfg, kv, dev.q, wl.q_start, T, idx, out, lse, ws=aws, stream=sh)

    def loop(parts, n):
        for _ in range(2):
            for f in parts:
                f()
        a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a_.record(stream)
        for _ in range(n):
            for f in parts:
                f()
        b_.record(stream)
        torch.cuda.synchronize()
        return a_.elapsed_time(b_) / n

    # The chunk step (scoring, merge, attention) timed with one event pair
    # around back-to-back steps (no events between its kernels); then each
    # phase timed inside the step with an event pair around it (which adds
    # the phase's launch latency to it).
    t_step = loop((scoring, merge, attention), 4 * iters)
    # the same step captured once in a HIP graph and replayed back to back
    # (the window pass's fork and join are captured with it)
    cap = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=cap):
        U.indexer_score_prefill(cfg, kv, dev.q_idx, wl.q_start, T, wsarg, stream=cap.cuda_stream)
        U.block_topk_prefill(cfg, wsarg, wl.q_start, T, M, idx, stream=cap.cuda_stream)
        U.sparse_attn_prefill(cfg, kv, dev.q, wl.q_start, T, idx, out, lse, ws=aws, stream=cap.cuda_stream)
    torch.cuda.synchronize()
    t_graph = loop((graph.replay,), 4 * iters)
    del graph
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(iters + 2)]
    for i in range(iters + 2):
        e = ev[i]
        e[0].record(stream)
        scoring()
        e[1].record(stream)
        merge()
        e[2].record(stream)
        attention()
        e[3].record(stream)
    torch.cuda.synchronize()
    t_sc = sum(ev[i][0].elapsed_time(ev[i][1]) for i in range(2, iters + 2)) / iters
    t_mg = sum(ev[i][1].elapsed_time(ev[i][2]) for i in range(2, iters + 2)) / iters
    t_at = sum(ev[i][2].elapsed_time(ev[i][3]) for i in range(2, iters + 2)) / iters
    # Scoring kernel alone, in steady state: 400 untimed launches (about 20
    # ms: under sustained matrix load the clock first drops, then settles
    # over about 10 ms), then seven batches of 10 back-to-back launches, one
    # event pair per batch; the median batch is reported, all seven are kept.
    nrep, nbatch = 10, 7
    for _ in range(400):
        U.indexer_score_prefill(cfg, kv, dev.q_idx, wl.q_start, T, wsarg, stream=sh)
    bev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nbatch)]
    for a_, b_ in bev:
        a_.record(stream)
        for _ in range(nrep):
            U.indexer_score_prefill(cfg, kv, dev.q_idx, wl.q_start, T, wsarg, stream=sh)
        b_.record(stream)
    torch.cuda.synchronize()
    batches = [a_.elapsed_time(b_) / nrep for a_, b_ in bev]
    t_sc_alone = sorted(batches)[nbatch // 2]
    flops = prefill_flops(wl)
    tflops = flops / (t_sc_alone * 1e-3) / 1e12
    attn_unique = int(wl.ctx_lens[0]) * 10 * 128 * 2 * 2
    res = {
        "workload": wl.name,
        "rows": T,
        "tokens_per_s": T / (t_step * 1e-3),
        "ms": {"step": t_step, "step_graph": t_graph, "scoring": t_sc, "merge": t_mg, "attention": t_at,
               "scoring_back_to_back": t_sc_alone},
        "ms_note": "step: back-to-back chunk steps, one event pair around them; step_graph: the same with the step "
                   "captured in a HIP graph and replayed; scoring/merge/attention: one event pair around each phase "
                   "inside the step (its launch latency included)",
        "scoring_back_to_back_batches_ms": batches,
        "scoring_in_step_TFLOPs": flops / (t_sc * 1e-3) / 1e12,
        # frac: the kernel in steady state (back-to-back batches above);
        # frac_in_step: the same FLOPs over the scoring launch as timed inside
        # the chunk step (an event pair around it, after the previous chunk's
        # attention).
        "scoring_roofline": {"bound": "mfma", "achieved": tflops, "peak": BF16_MFMA_PEAK_TFLOPS,
                             "unit": "TFLOP/s", "frac": tflops / BF16_MFMA_PEAK_TFLOPS,
                             "frac_in_step": flops / (t_sc * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS,
                             "flops_per_launch": flops, "traffic": traffic_for("indexer_prefill")},
        "attention_gathered_GBps": T * 2 * 512 * 10 * 128 * 2 / (t_at * 1e-3) / 1e9,
        "attention_unique_bytes_upper": attn_unique,
    }
    del dev, ws, aws, out
    torch.cuda.empty_cache()
    return res


def run_short_contexts(U, SD, W, torch, reps=50):
    """The whole decode step at the two short configurations: one 2048-token
    sequence with one layer, and 16 sequences x 12 layers at 32768 tokens;
    per-layer launches, the one launch and the automatic choice, each timed
    with one event pair around back-to-back steps on one stream."""
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    res = {}
    for wl in (W.config1(), W.config2()):
        dev = SD.generate(wl)
        cfg = U.make_cfg()
        nl, B, M, H, D = dev.q.shape[0], wl.batch, wl.max_blocks, wl.heads, wl.head_dim
        kv = U.make_kv(dev.k[0], dev.v[0], dev.kidx[0], dev.block_table, dev.ctx_lens, wl.pool_blocks, B, M)
        scores = torch.empty((nl, B, M), dtype=torch.float32, device="cuda")
        idx = torch.empty((nl, B, cfg.topk_blocks), dtype=torch.int32, device="cuda")
        out = torch.empty((nl, B, H, D), dtype=torch.float32, device="cuda")
        lse = torch.empty((nl, B, H), dtype=torch.float32, device="cuda")
        ws = torch.empty(U.workspace_size(cfg, U.OP_DECODE_STEP, nl * B, M), dtype=torch.uint8, device="cuda")
        us = {}
        for name, sched in (("per_layer", U.STEP_PER_LAYER), ("one_launch", U.STEP_ONE_LAUNCH), ("auto", U.STEP_AUTO)):
            def step():
                U.sparse_decode_step(cfg, kv, nl, dev.q_idx, dev.q, scores, idx, out, lse, ws=ws, stream=sh,
                                     schedule=sched)
            us[name] = time_steps(torch, stream, step, reps, 5) * 1e3
        if B >= 2:
            st2, fk, jn = micro_batch_step(U, torch, dev, cfg, (scores, idx, out, lse), 2)
            us["per_layer_two_streams"] = time_steps(torch, stream, st2, reps, 5, fk, jn) * 1e3
        idx_b, topk_b, attn_b = decode_bytes(wl)
        step_bytes = nl * (idx_b + topk_b + attn_b)
        res[wl.name] = {"layers": nl, "batch": B, "ctx_len": int(wl.ctx_lens.max()), "us_per_step": us,
                        "query_heads_per_s": {k: nl * B * H / (v * 1e-6) for k, v in us.items()},
                        "step_algorithmic_bytes": step_bytes,
                        "hbm_frac": {k: step_bytes / (v * 1e-6) / 1e9 / HBM_PEAK_GBPS for k, v in us.items()}}
        del dev, kv, scores, idx, out, lse, ws
        torch.cuda.empty_cache()
    return res


def run_page_gate(U, SD, W, torch, reps=20):
    """Page-aware ranking on the multi-page workloads: the ragged decode batch
    (64 documents of 400 image + 600 text tokens per page, query on the last
    page) and the 128K prefill chunk laid out in the same pages; each timed
    with and without the page tags (one event pair around back-to-back
    repetitions)."""
    import numpy as np

    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    res = {}

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a_.record(stream)
        for _ in range(reps):
            fn()
        b_.record(stream)
        torch.cuda.synchronize()
        return a_.elapsed_time(b_) / reps

    wl = W.config4()
    dev = SD.generate(wl)
    cfg = U.make_cfg()
    B, M, H = wl.batch, wl.max_blocks, 10
    tags = torch.from_numpy(np.tile(W.page_tags(M), (B, 1)).astype(np.int32)).cuda()
    qp = torch.from_numpy(np.array([W.page_of(L - 1) for L in wl.ctx_lens], np.int32)).cuda()
    kv_plain = dev.kv(0)
    kv_gate = U.make_kv(dev.k[0], dev.v[0], dev.kidx[0], dev.block_table, dev.ctx_lens, wl.pool_blocks, B, M,
                        tags, qp)
    scores = torch.empty((B, M), dtype=torch.float32, device="cuda")
    idx = torch.empty((B, 16), dtype=torch.int32, device="cuda")
    out = torch.empty((B, H, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")

    def step(kv):
        U.indexer_score_decode(cfg, kv, dev.q_idx[0], scores, stream=sh)
        U.topk_attn_decode(cfg, kv, dev.q[0], scores, idx, out, lse, stream=sh)

    ws1 = torch.empty(U.workspace_size(cfg, U.OP_DECODE_STEP, B, M), dtype=torch.uint8, device="cuda")
    scores1 = scores.view(1, B, M)

    def lib_step(kv, sched):
        U.sparse_decode_step(cfg, kv, 1, dev.q_idx, dev.q, scores1, idx.view(1, B, 16), out.view(1, B, H, 128),
                             lse.view(1, B, H), ws=ws1, stream=sh, schedule=sched)

    t_plain = timed(lambda: step(kv_plain))
    t_gate = timed(lambda: step(kv_gate))
    t1_plain = timed(lambda: lib_step(kv_plain, U.STEP_ONE_LAUNCH))
    t1_gate = timed(lambda: lib_step(kv_gate, U.STEP_ONE_LAUNCH))
    ta_plain = timed(lambda: lib_step(kv_plain, U.STEP_AUTO))
    ta_gate = timed(lambda: lib_step(kv_gate, U.STEP_AUTO))
    # per-layer launches over two micro-batches of 32 documents on two
    # streams of the caller's, forked and joined once around the repeated
    # steps: each half's next step depends only on its own previous one, as
    # in a decode loop, so the halves run as two pipelines
    st2, fk, jn = micro_batch_step(U, torch, dev, cfg,
                                   (scores1, idx.view(1, B, 16), out.view(1, B, H, 128), lse.view(1, B, H)), 2)
    t2_plain = time_steps(torch, stream, st2, reps, 3, fk, jn)
    idx_b, topk_b, attn_b = decode_bytes(wl)
    step_bytes = idx_b + topk_b + attn_b
    us = {"plain": t_plain, "page_aware": t_gate, "one_launch_plain": t1_plain, "one_launch_page_aware": t1_gate,
          "auto_plain": ta_plain, "auto_page_aware": ta_gate, "two_streams_plain": t2_plain}
    res["decode"] = {"workload": wl.name, "queries": B, "algorithmic_bytes": step_bytes,
                     "two_streams_note": "two micro-batches of 32 documents on two streams, joined once around "
                                         "the repeated steps (two independent pipelines, as in a decode loop)",
                     "us": {k: v * 1e3 for k, v in us.items()},
                     "query_heads_per_s": {k: B * H / (v * 1e-3) for k, v in us.items()},
                     "hbm_frac": {k: step_bytes / (v * 1e-3) / 1e9 / HBM_PEAK_GBPS for k, v in us.items()}}
    del dev, scores, out, ws1
    torch.cuda.empty_cache()

    wl = W.config5()
    dev = SD.generate(wl)
    T, M = wl.rows, wl.max_blocks
    tags = torch.from_numpy(W.page_tags(M)[None, :].astype(np.int32)).cuda()
    rp = torch.from_numpy(np.array([W.page_of(wl.q_start + t) for t in range(T)], np.int32)).cuda()
    kv_plain = dev.kv(0)
    kv_gate = U.make_kv(dev.k[0], dev.v[0], dev.kidx[0], dev.block_table, dev.ctx_lens, wl.pool_blocks, 1, M,
                        tags, rp)
    ws_bytes = U.workspace_size(cfg, U.OP_INDEXER_PREFILL, T, M)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    wsarg = (ws.data_ptr(), ws_bytes)
    bidx = torch.empty((T, 16), dtype=torch.int32, device="cuda")

    def score(kv):
        U.indexer_score_prefill(cfg, kv, dev.q_idx, wl.q_start, T, wsarg, stream=sh)
        U.block_topk_prefill(cfg, wsarg, wl.q_start, T, M, bidx, stream=sh)

    res["prefill_scoring_and_merge"] = {"workload": wl.name + ", pages of 400 image + 600 text tokens",
                                        "us": {"plain": timed(lambda: score(kv_plain)) * 1e3,
                                               "page_aware": timed(lambda: score(kv_gate)) * 1e3}}
    del dev, ws
    torch.cuda.empty_cache()
    return res


def run_rope(U, torch, reps=20):
    """page2d coordinates from the token stream (a page marker every 1000
    tokens), cache write and query rotation: one decode layer of 16 sequences
    (one new token each) and one 2048-token prefill chunk, into block-major
    pools of 128K-token sequences; one event pair around back-to-back calls."""
    import numpy as np

    H, D, M = 10, 128, 4096
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    cfg = U.make_cfg()
    g = np.random.default_rng(7)
    res = {}
    for name, B, n in (("decode: 16 sequences x 1 new token", 16, 16), ("prefill: 2048 new tokens", 1, 2048)):
        P = B * M
        kp = torch.zeros((P, H, 32, D), dtype=torch.int16, device="cuda")
        vp = torch.zeros_like(kp)
        ip = torch.zeros((P, 32, D), dtype=torch.int16, device="cuda")
        table = torch.from_numpy(g.permutation(P).reshape(B, M).astype(np.int32)).cuda()
        ctx = torch.full((B,), M * 32, dtype=torch.int32, device="cuda")
        kv = U.make_kv(kp, vp, ip, table, ctx, P, B, M)
        per = n // B  # new tokens per sequence
        seq = torch.from_numpy((np.arange(n) // per).astype(np.int32)).cuda()
        pos = torch.from_numpy((M * 32 - per + np.arange(n) % per).astype(np.int32)).cuda()
        marker = 151
        stream_toks = torch.from_numpy(np.where(np.arange(n) % 1000 == 0, marker, 5).astype(np.int32)).cuda()
        coord_state = torch.zeros((B, 2), dtype=torch.int32, device="cuda")
        tok = torch.empty(n, dtype=torch.int32, device="cuda")
        page = torch.empty(n, dtype=torch.int32, device="cuda")
        kn = torch.randn((n, H, D), device="cuda").to(torch.bfloat16).view(torch.int16)
        vn = torch.randn((n, H, D), device="cuda").to(torch.bfloat16).view(torch.int16)
        ixn = torch.randn((n, D), device="cuda").to(torch.bfloat16).view(torch.int16)
        q = torch.randn((n, H, D), device="cuda").to(torch.bfloat16).view(torch.int16)
        qi = torch.randn((n, D), device="cuda").to(torch.bfloat16).view(torch.int16)

        def call():
            U.page_coords(B, per, stream_toks, marker, coord_state, tok, page, stream=sh)
            U.rope_cache_write(cfg, kv, n, seq, pos, tok, page, kn, vn, ixn, stream=sh)
            U.rope_queries(cfg, n, tok, page, q=q, q_idx=qi, stream=sh)

        call()
        torch.cuda.synchronize()
        a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a_.record(stream)
        for _ in range(reps):
            call()
        b_.record(stream)
        torch.cuda.synchronize()
        us = a_.elapsed_time(b_) / reps * 1e3
        moved = n * (H * D * 2 * 2 + D * 2) * 2 + n * (H * D + D) * 2 * 2   # cache rows in+out, queries in+out
        res[name] = {"us": us, "bytes": moved, "GBps": moved / (us * 1e-6) / 1e9}
        del kp, vp, ip
        torch.cuda.empty_cache()
    return res


def run_page_window(U):
    """Peak KV of the page-window schedule (host block pool, no GPU work):
    documents of 400 image + 600 text tokens per page, windows of 10 pages,
    the last 128 text tokens kept across a boundary, against keeping every
    block; bytes for 12 layers of K, V (10 heads x 128, bf16) and indexer K
    (128, bf16) per token slot."""
    import time

    slot_bytes = 12 * (2 * 10 * 128 * 2 + 128 * 2)   # 64512 B per token slot, all layers
    W, tail, img, txt = 10, 128, 400, 600
    res = {"window_pages": W, "text_tail_tokens": tail, "page_tokens": {"image": img, "text": txt},
           "bytes_per_token_slot": slot_bytes, "documents": {}}
    for pages in (100, 1000):
        pool = U.BlockPool(1 << 20)
        t0 = time.perf_counter()
        peaks = pool.page_window_run(0, [img] * pages, [txt] * pages, W, tail)
        host_us = (time.perf_counter() - t0) * 1e6
        full_blocks = -(-pages * (img + txt) // 32)
        res["documents"][f"{pages} pages"] = {
            "windows": len(peaks), "peak_blocks": pool.peak, "peak_GB": pool.peak * 32 * slot_bytes / 1e9,
            "no_eviction_blocks": full_blocks, "no_eviction_GB": full_blocks * 32 * slot_bytes / 1e9,
            "host_us": host_us}
        pool.close()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--graph", action="store_true",
                    help="with --multi-launch: capture one decode step as a HIP graph and time its replays")
    ap.add_argument("--multi-launch", action="store_true",
                    help="run the step as per-layer launches (indexer, then selection + attention) on micro-batch "
                         "streams instead of the one uocr_sparse_decode_step launch")
    ap.add_argument("--separate", action="store_true",
                    help="run selection and attention as two launches instead of the fused one")
    ap.add_argument("--streams", type=int, default=2,
                    help="micro-batches of sequences, each on its own HIP stream (default priority)")
    ap.add_argument("--cpu-layers", type=int, default=12,
                    help="layers of the workload the CPU oracle is timed on (x16 queries)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-schedules", action="store_true",
                    help="skip timing the step under the other schedules (one launch, per-layer on one and on two "
                         "streams)")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-page-gate", action="store_true", help="skip the page-aware ranking measurement")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense full-context comparator")
    ap.add_argument("--no-rope", action="store_true", help="skip the page2d cache-write measurement")
    ap.add_argument("--no-short", action="store_true",
                    help="skip the short-context step timings (one 2048-token query; 16 x 12 layers at 32K)")
    ap.add_argument("--no-layout", action="store_true",
                    help="skip the decode step on the contiguous block layout")
    ap.add_argument("--prefill-only", action="store_true",
                    help="run only the chunked-prefill case (profiling)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only copy 1 GiB device-to-device 5 times (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the decode step shards by sequence with no communication across GPUs)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.calibrate_copy:
        torch.cuda.set_device(0)
        a = torch.ones(1 << 29, dtype=torch.int16, device="cuda")   # 1 GiB
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": a.numel() * 2, "copies": 5}))
        return

    import block_sparse_long_sr_amd as U
    from synth import device as SD
    from synth import workloads as W

    torch.cuda.set_device(0)
    if args.prefill_only:
        print(json.dumps({"prefill": run_prefill(U, SD, W, torch)}), flush=True)
        return
    t0 = time.time()
    wl = W.config3()
    log(f"generating {wl.name} on the GPU")
    dev = SD.generate(wl)
    torch.cuda.synchronize()
    pool_gb = (dev.k.numel() + dev.v.numel() + dev.kidx.numel()) * 2 / 1e9
    log(f"generated in {time.time() - t0:.1f}s; pools {pool_gb:.1f} GB")

    cfg = U.make_cfg()
    B, M, L, H = wl.batch, wl.max_blocks, wl.layers, 10
    scores = torch.empty((L, B, M), dtype=torch.float32, device="cuda")
    idx = torch.empty((L, B, 16), dtype=torch.int32, device="cuda")
    out = torch.empty((L, B, H, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((L, B, H), dtype=torch.float32, device="cuda")
    kvs = [dev.kv(l) for l in range(L)]
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    one_launch = not args.multi_launch
    step_ws = None
    step_ws_sched = torch.empty(U.workspace_size(cfg, U.OP_DECODE_STEP, L * B, M), dtype=torch.uint8, device="cuda")
    if one_launch:
        wsb = U.workspace_size(cfg, U.OP_DECODE_STEP, L * B, M)
        step_ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
        kv0 = dev.kv(0)
        fork = join = lambda base: None

        def step():
            U.sparse_decode_step(cfg, kv0, L, dev.q_idx, dev.q, scores, idx, out, lse, ws=step_ws, stream=sh,
                                 schedule=U.STEP_ONE_LAUNCH)
    else:
        step, fork, join = micro_batch_step(U, torch, dev, cfg, (scores, idx, out, lse), args.streams,
                                            separate=args.separate, base=None if args.graph else stream)

    fork(stream)
    for _ in range(args.warmup):
        step()
        if step_ws is not None:
            U.check_decode_step(step_ws)   # every warm-up step: no dependency wait gave up
    join(stream)
    torch.cuda.synchronize()
    graph = None
    if args.graph and not one_launch:
        # One step (12 layers of every micro-batch group) captured as a HIP
        # graph; each replay relaunches all of its kernels on the same inputs.
        graph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        with torch.cuda.graph(graph, stream=cap):
            fork(cap)
            step()
            join(cap)
        torch.cuda.synchronize()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    if graph is not None:
        for _ in range(args.steps):
            graph.replay()
    else:
        fork(stream)
        for _ in range(args.steps):
            step()
        join(stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_total = e0.elapsed_time(e1)
    ms_step = ms_total / args.steps
    if step_ws is not None:
        U.check_decode_step(step_ws)   # the last timed step (each call clears the word first)
    # the timed step's outputs, kept for the parity check against the oracle
    gpu_out = {"idx": idx.cpu().numpy(), "out": out.cpu().numpy(), "lse": lse.cpu().numpy()}
    qh_per_s = B * L * H * args.steps / (ms_total * 1e-3)
    log(f"decode step {ms_step * 1e3:.1f} us, {qh_per_s / 1e6:.3f} M query-heads/s")

    # Per-kernel durations (separate pass, one stream, whole batch): one event
    # pair around the 12 back-to-back launches of a kernel (one per layer), so
    # that the average per launch is the kernel's own duration plus the short
    # dispatch gap between consecutive launches on a stream.
    ksteps = max(3, min(10, args.steps))

    def timed(launch):
        pairs = []
        for _ in range(ksteps):
            a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a_.record(stream)
            for l in range(L):
                launch(l)
            b_.record(stream)
            pairs.append((a_, b_))
        torch.cuda.synchronize()
        return sum(a_.elapsed_time(b_) for a_, b_ in pairs) / (len(pairs) * L)

    t_step_kernel = None
    if one_launch:
        # the one-launch step timed alone, back to back on one stream: its
        # main kernel plus the tiny counter-clearing kernel before it
        pairs = []
        for _ in range(ksteps):
            a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a_.record(stream)
            step()
            b_.record(stream)
            pairs.append((a_, b_))
        torch.cuda.synchronize()
        t_step_kernel = sum(a_.elapsed_time(b_) for a_, b_ in pairs) / len(pairs)
    t_idx = timed(lambda l: U.indexer_score_decode(cfg, kvs[l], dev.q_idx[l], scores[l], stream=sh))
    t_topk = timed(lambda l: U.block_topk_decode(cfg, scores[l], dev.ctx_lens, B, M, idx[l], stream=sh))
    t_attn = timed(lambda l: U.sparse_attn_decode(cfg, kvs[l], dev.q[l], idx[l], out[l], lse[l], stream=sh))
    t_fused = timed(lambda l: U.topk_attn_decode(cfg, kvs[l], dev.q[l], scores[l], idx[l], out[l], lse[l],
                                                 stream=sh))
    idx_bytes, topk_bytes, attn_bytes = decode_bytes(wl)
    achieved = idx_bytes / (t_idx * 1e-3) / 1e9
    step_bytes = L * (idx_bytes + topk_bytes + attn_bytes)
    log(f"indexer {t_idx * 1e3:.1f} us ({achieved:.0f} GB/s), topk {t_topk * 1e3:.1f} us, "
        f"attention {t_attn * 1e3:.1f} us, fused topk+attention {t_fused * 1e3:.1f} us")

    result = {
        "metric": METRIC,
        "value": qh_per_s,
        "unit": "query-heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": B, "layers": L, "ctx_len": int(wl.ctx_lens[0]),
                   "heads": H, "head_dim": 128, "block_size": 32, "topk_blocks": 16, "local_blocks": 4,
                   "queries_per_step": B * L, "plant": wl.notes, "seed": hex(wl.seed),
                   "launches": "one uocr_sparse_decode_step per step" if one_launch else
                               f"per layer, {args.streams} micro-batch streams" + (", HIP graph" if args.graph else "")},
        "tokens_per_s": B / (ms_step * 1e-3),
        "step_hbm_GBps": step_bytes / (ms_step * 1e-3) / 1e9,
        "step_hbm_frac": step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "step_algorithmic_bytes": step_bytes,
        "kernel_us": {"indexer_score_decode": t_idx * 1e3, "block_topk_decode": t_topk * 1e3,
                      "sparse_attn_decode": t_attn * 1e3, "topk_attn_decode": t_fused * 1e3},
        "step_launches": ("decode_step_clear_kernel + decode_step_kernel" if one_launch else
                          "indexer_score_decode + " + ("block_topk_decode + sparse_attn_decode" if args.separate
                                                       else "topk_attn_decode") + " per layer"),
    }
    if one_launch:
        step_achieved = step_bytes / (t_step_kernel * 1e-3) / 1e9
        result["kernel_us"]["sparse_decode_step"] = t_step_kernel * 1e3
        result["roofline"] = {"kernel": "decode_step_kernel", "bound": "hbm", "achieved": step_achieved,
                              "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": step_achieved / HBM_PEAK_GBPS,
                              "algorithmic_bytes_per_launch": step_bytes,
                              "traffic": traffic_for("decode_step")}
        result["indexer_roofline"] = {"kernel": "indexer_score_decode", "bound": "hbm", "achieved": achieved,
                                      "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                                      "algorithmic_bytes_per_launch": idx_bytes,
                                      "traffic": traffic_for("indexer_decode")}
        log(f"one-launch step kernel {t_step_kernel * 1e3:.1f} us ({step_achieved:.0f} GB/s algorithmic)")
    else:
        result["roofline"] = {"kernel": "indexer_score_decode", "bound": "hbm", "achieved": achieved,
                              "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                              "algorithmic_bytes_per_launch": idx_bytes,
                              "traffic": traffic_for("indexer_decode")}

    if not args.no_schedules:
        # the same step under each schedule (the headline's included, for a
        # like-for-like comparison in one place)
        result["step_schedules"] = schedule_timings(U, torch, dev, cfg, (scores, idx, out, lse), step_ws_sched,
                                                    args.steps, args.warmup, step_bytes)
        log("step schedules: " + ", ".join(f"{k} {v['us_per_step']:.1f} us ({v['hbm_frac']:.3f} of HBM peak)"
                                           for k, v in result["step_schedules"].items()))

    if not args.no_cpu_baseline:
        log(f"CPU oracle on {B * args.cpu_layers} query-layers (all BLAS threads, then one thread), "
            f"checked against the timed step's outputs")
        timing, parity = cpu_baseline(U, dev, wl, args.cpu_layers, gpu_out, cfg)
        nq = timing["queries"]
        host = host_description()
        blas_threads = max([d["threads"] or 1 for d in host["blas"]] or [1])
        result["cpu_baseline"] = {
            "value": nq * H / timing["seconds_all_threads"], "unit": "query-heads/s", "cores": blas_threads,
            "kind": "oracle",
            "sample": f"every query of the step: {nq} decode queries ({args.cpu_layers} layers x {B} sequences) of "
                      f"the same workload on the same device inputs copied to the host, "
                      f"{timing['seconds_all_threads']:.1f} s with numpy's BLAS on {blas_threads} threads (the "
                      f"dot products; the block max, sort and softmax are single-threaded); oracle time only",
            "single_thread": {"value": nq * H / timing["seconds_one_thread"], "cores": 1,
                              "seconds": timing["seconds_one_thread"]},
            "host": host,
        }
        result["parity"] = dict(parity, what="the timed step's selections and attention outputs against the CPU "
                                              "oracle on the same inputs, every query")
        log(f"cpu oracle {nq * H / timing['seconds_all_threads']:.1f} query-heads/s on {blas_threads} BLAS threads, "
            f"{nq * H / timing['seconds_one_thread']:.1f} on one; parity: {parity['selection_exact']} exact, "
            f"{parity['selection_differences_inside_band']} inside the band, "
            f"{parity['selection_mismatches_outside_band']} outside; attention max-abs "
            f"{parity['attention_on_gpu_selection']['max_abs']:.2e} rel-L2 "
            f"{parity['attention_on_gpu_selection']['rel_l2']:.2e}; pass={parity['pass']}")

    if not args.no_dense:
        # Dense full-context attention of the same step (the comparator for the
        # pages' per-step speed claim against full attention): every query
        # attends to all 131072 tokens of its sequence in each of the 12 layers.
        wsb = U.workspace_size(cfg, U.OP_DENSE_ATTN_DECODE, B, M)
        dws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
        dwarg = (dws.data_ptr(), wsb)
        U.dense_attn_decode(cfg, kvs[0], dev.q[0], out[0], lse[0], ws=dwarg, stream=sh)
        torch.cuda.synchronize()
        reps = 2
        a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a_.record(stream)
        for _ in range(reps):
            for l in range(L):
                U.dense_attn_decode(cfg, kvs[l], dev.q[l], out[l], lse[l], ws=dwarg, stream=sh)
        b_.record(stream)
        torch.cuda.synchronize()
        ms_dense = a_.elapsed_time(b_) / reps
        dense_bytes = L * sum(int(x) * 10 * 128 * 2 * 2 for x in wl.ctx_lens)
        result["dense_comparator"] = {
            "what": "full-context decode attention (all tokens, 10 heads) for the same 12 layers x 16 sequences",
            "ms_per_step": ms_dense, "sparse_ms_per_step": ms_step, "speedup_sparse_over_dense": ms_dense / ms_step,
            "kv_bytes_per_step": dense_bytes, "achieved_GBps": dense_bytes / (ms_dense * 1e-3) / 1e9}
        log(f"dense full-context attention step {ms_dense:.2f} ms ({dense_bytes / (ms_dense * 1e-3) / 1e9:.0f} GB/s): "
            f"sparse step is {ms_dense / ms_step:.1f}x faster")
        del dws
    del dev, kvs
    torch.cuda.empty_cache()
    if one_launch and not args.no_layout:
        # The same step with every sequence's blocks in consecutive pool slots
        # (what a fresh lowest-id-first block pool hands out), against the
        # seeded random placement of the headline figure.
        wl_c = W.config3()
        wl_c.layout = "contiguous"
        dev = SD.generate(wl_c)
        kv_c = dev.kv(0)

        def step_c():
            U.sparse_decode_step(cfg, kv_c, L, dev.q_idx, dev.q, scores, idx, out, lse, ws=step_ws, stream=sh,
                                 schedule=U.STEP_ONE_LAUNCH)

        for _ in range(args.warmup):
            step_c()
        a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a_.record(stream)
        for _ in range(args.steps):
            step_c()
        b_.record(stream)
        torch.cuda.synchronize()
        ms_c = a_.elapsed_time(b_) / args.steps
        result["contiguous_layout"] = {
            "what": "the same step with each sequence's blocks in consecutive pool slots (headline: seeded random "
                    "placement)",
            "ms_per_step": ms_c, "query_heads_per_s": B * L * H / (ms_c * 1e-3),
            "step_hbm_GBps": step_bytes / (ms_c * 1e-3) / 1e9}
        log(f"contiguous block layout: decode step {ms_c * 1e3:.1f} us ({step_bytes / (ms_c * 1e-3) / 1e9:.0f} GB/s)")
        del dev, kv_c
        torch.cuda.empty_cache()
    del scores, out
    torch.cuda.empty_cache()
    if not args.no_prefill:
        log("chunked prefill T=2048 at 129024 of 131072")
        result["prefill"] = run_prefill(U, SD, W, torch)
        pf = result["prefill"]
        log(f"prefill chunk step {pf['ms']['step'] * 1e3:.1f} us ({pf['ms']['step_graph'] * 1e3:.1f} us as a HIP graph); scoring {pf['ms']['scoring_back_to_back'] * 1e3:.1f} us "
            f"back to back ({pf['scoring_roofline']['achieved']:.0f} TFLOP/s), {pf['ms']['scoring'] * 1e3:.1f} us in the "
            f"step; merge {pf['ms']['merge'] * 1e3:.1f} us; attention {pf['ms']['attention'] * 1e3:.1f} us")

    if not args.no_page_gate:
        log("page-aware ranking: ragged multi-page decode and the 128K prefill chunk, with and without page tags")
        result["page_gate"] = run_page_gate(U, SD, W, torch)
        pg = result["page_gate"]
        log("ragged decode B=64: " + ", ".join(f"{k} {v:.1f} us" for k, v in pg["decode"]["us"].items()) + "; "
            f"prefill scoring+merge {pg['prefill_scoring_and_merge']['us']['page_aware']:.1f} us "
            f"(plain {pg['prefill_scoring_and_merge']['us']['plain']:.1f} us)")

    if not args.no_short:
        result["short_context"] = run_short_contexts(U, SD, W, torch)
        for k, v in result["short_context"].items():
            log(f"{k}: " + ", ".join(f"{n} {u:.1f} us" for n, u in v["us_per_step"].items()) + " per step")

    if not args.no_rope:
        result["page2d_rope_cache_write"] = run_rope(U, torch)
        for k, v in result["page2d_rope_cache_write"].items():
            log(f"page2d coordinates + rope + cache write, {k}: {v['us']:.1f} us ({v['GBps']:.0f} GB/s)")

    result["page_window_kv"] = run_page_window(U)
    for k, v in result["page_window_kv"]["documents"].items():
        log(f"page-window schedule, {k}: peak KV {v['peak_GB']:.2f} GB ({v['peak_blocks']} blocks), "
            f"{v['no_eviction_GB']:.2f} GB without eviction")

    print(json.dumps(result), flush=True)
    if "parity" in result and not result["parity"]["pass"]:
        log("PARITY FAILURE: " + "; ".join(result["parity"]["failures"]))
        sys.exit(3)


if __name__ == "__main__":
    main()
