"""Host-side checks of the seeded workload generator (no GPU)."""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
from synth import rng, workloads as W


def test_splitmix64_reference_values():
    # SplitMix64 seeded with 0: the first outputs as published with the
    # algorithm (state += GAMMA; then the output mix).
    want = [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]
    got = [int(w) for w in rng.words(0, np.arange(3))]
    assert got == want


def test_bf16_rounding_nearest_even():
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-9, -2.5, 3.0e-5], np.float32)
    b = rng.f32_to_bf16_bits(x)
    back = rng.bf16_bits_to_f32(b)
    assert back[0] == 1.0
    assert back[1] == 1.0                      # tie -> even (mantissa 0)
    assert back[2] == np.float32(1.0 + 2**-7)  # above half -> up
    assert back[3] == -2.5
    assert abs(back[4] - 3.0e-5) / 3.0e-5 < 2**-8


def test_normal_moments_and_determinism():
    key = rng.stream_key(0x5EED0002, W.tensor_id(W.ROLE_KIDX, 3, 7))
    a = rng.normal_bf16(key, np.arange(400_000))
    b = rng.normal_bf16(key, np.arange(400_000))
    np.testing.assert_array_equal(a, b)
    x = rng.bf16_bits_to_f32(a).astype(np.float64)
    assert abs(x.mean()) < 0.01
    assert abs(x.std() - 1.0) < 0.01
    assert np.abs(x).max() <= 4.9
    # slices regenerate the same bits
    np.testing.assert_array_equal(rng.normal_bf16(key, np.arange(1000, 1100)), a[1000:1100])


def test_small_int_values():
    v = rng.bf16_bits_to_f32(rng.small_int_bf16(rng.stream_key(1, 2), np.arange(50_000)))
    assert set(np.unique(v).tolist()) == {-2.0, -1.0, 0.0, 1.0, 2.0}


def test_block_table_is_a_partition():
    wl = W.config4(batch=12)
    tab = wl.block_table()
    used = []
    for b in range(wl.batch):
        nb = wl.nblocks(b)
        assert np.all(tab[b, :nb] >= 0)
        assert np.all(tab[b, nb:] == -1)
        used.extend(tab[b, :nb].tolist())
    assert sorted(used) == list(range(wl.pool_blocks))


def test_config4_structure():
    wl = W.config4()
    assert wl.batch == 64
    assert np.all(wl.ctx_lens % 1000 == 0)
    assert wl.ctx_lens.min() >= 5000 and wl.ctx_lens.max() <= 65000
    for e in wl.edits:
        pages = np.unique(e.tokens // 1000)
        assert 1 <= pages.size <= 3
        assert np.all(e.tokens % 1000 < 400)                 # image tokens only
        assert pages.max() < wl.ctx_lens[e.seq] // 1000 - 1  # not the last page


def test_config4_correlation_cosine():
    wl = W.config4(batch=3)
    e = wl.edits[0]
    q = oracle.widen(wl.q_idx(0, e.seq))
    k = oracle.widen(wl.kidx(0, e.seq, int(e.tokens[0]), int(e.tokens[0]) + 400))
    cos = (k @ q) / (np.linalg.norm(k, axis=1) * np.linalg.norm(q))
    assert abs(cos.mean() - 0.5) < 0.05


def test_host_pools_match_logical_tensors():
    wl = W.decode_uniform("tiny", 3, 3, 2, 100)
    wl.ctx_lens = np.array([100, 33, 64])
    wl.max_blocks = 4
    tab = wl.block_table()
    kp, vp, ip = wl.host_pools(1)
    for b in range(3):
        L = int(wl.ctx_lens[b])
        k = wl.kv(W.ROLE_K, 1, b, 0, L)
        ki = wl.kidx(1, b, 0, L)
        for t in range(L):
            pb = tab[b, t // 32]
            np.testing.assert_array_equal(kp[pb, :, t % 32, :], k[:, t, :])
            np.testing.assert_array_equal(ip[pb, t % 32, :], ki[t])
        if L % 32:
            assert np.all(kp[tab[b, L // 32], :, L % 32:, :] == 0x7FC0)


@pytest.mark.slow
def test_planted_blocks_are_the_top12_with_clear_cutoff():
    wl = W.config3(batch=2, layers=1)
    S = 131072
    cfg = oracle.SparseCfg()
    for b in range(2):
        e = [x for x in wl.edits if x.seq == b][0]
        ki = wl.kidx(0, b, 0, S)
        s = oracle.indexer_scores(wl.q_idx(0, b), ki)
        ncand = oracle.candidate_count(S - 1, cfg)
        bm = oracle.block_maxima(s, S - 1, ncand, cfg)
        sel = oracle.select_blocks(bm, S - 1, cfg)
        assert sel["remote"] == sorted((e.tokens // 32).tolist())
        ranked = sel["ranked"]
        c12, c13 = bm[ranked[11]], bm[ranked[12]]
        assert (c12 - c13) / abs(c12) > 1e-2
