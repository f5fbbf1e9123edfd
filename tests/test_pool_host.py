"""Host logic of the block pool and the page-window schedule (no GPU): the
C ABI's uocr_pool_* and uocr_page_window_run against the oracle's schedule
(leheavengame.com OCR 2 release article, Sec. 2 route A, storage half).

A label shadow of the physical token slots follows every append through the
block table, so the tokens a compacted table reaches can be compared with
the oracle's token list, not only the counts."""
import ctypes
import random

import pytest

import oracle

BLOCK = 32


@pytest.fixture(scope="module")
def U():
    import block_sparse_long_sr_amd as U
    return U


def _run_with_shadow(U, img, txt, W, tail, num_blocks):
    """Drive the schedule through pool_append / pool_keep, writing each
    appended token's label into the slot the block table gives it."""
    pool = U.BlockPool(num_blocks)
    slots = {}
    n = len(img)
    wins = oracle.page_window.windows(n, W)
    peaks = []

    def append(label_list):
        _, before = pool.table(0, num_blocks)
        pool.append(0, len(label_list))
        row, length = pool.table(0, num_blocks)
        assert length == before + len(label_list)
        for i, lab in enumerate(label_list):
            p = before + i
            slots[(row[p // BLOCK], p % BLOCK)] = lab

    for w, (first, last) in enumerate(wins):
        pages = oracle.page_window.new_pages(w, first, last)
        peak = pool.used
        shared_lo = shared_hi = None
        for k in pages:
            if k == last - 1:
                shared_lo = pool.table(0, num_blocks)[1]
            append([("img", k, i) for i in range(img[k])])
            if k == last - 1:
                shared_hi = pool.table(0, num_blocks)[1]
            peak = max(peak, pool.used)
        for k in pages:
            append([("txt", k, i) for i in range(txt[k])])
            peak = max(peak, pool.used)
        peaks.append(peak)
        if w + 1 < len(wins):
            end = pool.table(0, num_blocks)[1]
            pool.keep(0, [(shared_lo, shared_hi), (max(shared_hi, end - tail), end)])
    row, length = pool.table(0, num_blocks)
    seq = [slots[(row[p // BLOCK], p % BLOCK)] for p in range(length)]
    return pool, peaks, row, seq


def _doc(seed):
    rng = random.Random(seed)
    n = rng.randint(1, 16)
    W = rng.randint(2, 6)
    tail = rng.choice([0, 1, 31, 32, 33, 128])
    img = [rng.choice([0, rng.randint(1, 120)]) for _ in range(n)]
    txt = [rng.choice([0, rng.randint(1, 120)]) for _ in range(n)]
    return img, txt, W, tail


@pytest.mark.parametrize("seed", range(12))
def test_pool_keeps_the_oracles_tokens(U, seed):
    img, txt, W, tail = _doc(seed)
    ref = oracle.page_window_schedule(img, txt, W, tail)
    pool, peaks, row, seq = _run_with_shadow(U, img, txt, W, tail, 4096)
    assert peaks == ref["window_peaks"]
    assert seq == ref["final"]
    assert pool.used == -(-len(seq) // BLOCK)
    assert pool.peak == ref["peak"]
    live = [b for b in row if b >= 0]
    assert len(set(live)) == len(live) and all(0 <= b < 4096 for b in live)


@pytest.mark.parametrize("seed", range(12))
def test_page_window_run_matches_the_oracle(U, seed):
    img, txt, W, tail = _doc(seed)
    ref = oracle.page_window_schedule(img, txt, W, tail)
    pool = U.BlockPool(4096)
    assert pool.page_window_run(0, img, txt, W, tail) == ref["window_peaks"]
    row, length = pool.table(0, 4096)
    assert length == len(ref["final"]) and pool.used == -(-length // BLOCK) and pool.peak == ref["peak"]
    # same allocation order as the step-by-step driver, so the same table row
    _, _, row2, _ = _run_with_shadow(U, img, txt, W, tail, 4096)
    assert row == row2


def test_page_window_run_fits_exactly_its_peak(U):
    img, txt, W, tail = [400] * 25, [600] * 25, 10, 128
    peak = oracle.page_window_schedule(img, txt, W, tail)["peak"]
    assert U.BlockPool(peak).page_window_run(0, img, txt, W, tail)[0] == peak
    with pytest.raises(U.UocrError) as e:
        U.BlockPool(peak - 1).page_window_run(0, img, txt, W, tail)
    assert e.value.status == 6


def test_pool_allocation_and_errors(U):
    pool = U.BlockPool(6, max_seqs=2)
    pool.append(0, 33)  # blocks 0, 1
    pool.append(1, 1)   # block 2
    pool.append(0, 31)  # fills block 1 exactly
    assert pool.table(0, 4) == ([0, 1, -1, -1], 64) and pool.used == 3
    pool.append(0, 1)
    assert pool.table(0, 4) == ([0, 1, 3, -1], 65)
    with pytest.raises(U.UocrError) as e:
        pool.append(1, 3 * 32)  # needs 3 more, 2 free: nothing changes
    assert e.value.status == 6 and pool.table(1, 4) == ([2, -1, -1, -1], 1) and pool.used == 4
    pool.keep(0, [(40, 41)])  # block 1 only; it is not the last block, so it counts 32
    assert pool.table(0, 4) == ([1, -1, -1, -1], 32) and pool.used == 2
    pool.append(1, 31)  # fills block 2
    pool.append(0, 1)   # lowest free id first: 0
    assert pool.table(0, 4) == ([1, 0, -1, -1], 33)
    pool.keep(0, [(0, 0), (32, 33)])  # an empty range keeps nothing; the last block keeps its fill of 1
    assert pool.table(0, 4) == ([0, -1, -1, -1], 1) and pool.peak == 4
    pool.keep(0, [])
    assert pool.table(0, 4) == ([-1, -1, -1, -1], 0)
    pool.append(0, 3)
    for bad in ([(2, 1)], [(0, 4)], [(1, 2), (0, 1)], [(-1, 1)]):
        with pytest.raises(U.UocrError) as e:
            pool.keep(0, bad)
        assert e.value.status == 2
    assert pool.table(0, 4)[1] == 3
    with pytest.raises(U.UocrError):
        pool.append(2, 1)  # no sequence 2
    with pytest.raises(U.UocrError):
        pool.table(1, 0)  # the row holds no entry for the sequence's block
    with pytest.raises(ValueError):
        U.BlockPool(-1)
    assert U._lib.uocr_pool_used(None) == -1 and U._lib.uocr_pool_peak(None) == -1
    # the schedule needs an empty sequence and a window of at least 2 pages
    with pytest.raises(U.UocrError):
        pool.page_window_run(0, [1], [1], 3, 0)
    with pytest.raises(U.UocrError):
        U.BlockPool(8).page_window_run(0, [1, 2], [1, 2], 1, 0)
    assert U.BlockPool(8).page_window_run(0, [], [], 4, 0) == []
