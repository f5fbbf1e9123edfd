"""Pins of the oracle's page-window schedule (leheavengame.com OCR 2 release
article, Sec. 2 route A, storage half) -- checked against a hand-worked
fixture, the no-eviction special case, a page-count-independent bound and
invariants, with planted mistakes that each of them must catch."""
import os
import random

import pytest

import oracle
from oracle import page_window as pw

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_window.txt")


def _golden_cases():
    cases, cur = [], None
    for line in open(GOLDEN):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        key, *vals = line.split()
        if key == "case":
            cur = {"name": vals[0], "runs": []}
            cases.append(cur)
        elif key == "run":
            cur["runs"].append((vals[0], int(vals[1]), int(vals[2]), int(vals[3])))
        elif key in ("window", "tail", "length"):
            cur[key] = int(vals[0])
        else:
            cur[key] = [int(v) for v in vals]
    return cases


def _expand(runs):
    return [(kind, page, first + i) for kind, page, first, count in runs for i in range(count)]


def _golden_pass() -> bool:
    for c in _golden_cases():
        r = oracle.page_window_schedule(c["image"], c["text"], c["window"], c["tail"])
        if r["window_peaks"] != c["peaks"] or len(r["final"]) != c["length"] or r["final"] != _expand(c["runs"]):
            return False
    return True


def test_golden_documents():
    cases = _golden_cases()
    assert [c["name"] for c in cases] == ["A", "B"]
    for c in cases:
        assert sum(run[3] for run in c["runs"]) == c["length"]
    assert _golden_pass()


@pytest.mark.parametrize("seed", range(6))
def test_one_window_keeps_everything(seed):
    # W >= pages: one window, nothing is released, the peak is the whole document
    rng = random.Random(seed)
    n = rng.randint(1, 7)
    img = [rng.randint(0, 90) for _ in range(n)]
    txt = [rng.randint(0, 90) for _ in range(n)]
    r = oracle.page_window_schedule(img, txt, rng.randint(max(n, 2), 12), rng.randint(0, 200))
    total = sum(img) + sum(txt)
    assert r["window_peaks"] == [-(-total // 32)]
    expect = [("img", k, i) for k in range(n) for i in range(img[k])]
    expect += [("txt", k, i) for k in range(n) for i in range(txt[k])]
    assert r["final"] == expect


def test_peak_is_bounded_independently_of_page_count():
    # pages of 400 image + 600 text tokens, W = 10, tail 128: the first
    # window holds its W pages; a later one at most the kept blocks of the
    # shared image and the tail plus its W-1 new pages; neither grows with
    # the document
    I, X, W, tail = 400, 600, 10, 128
    later = (-(-I // 32) + 1) + (-(-tail // 32) + 1) + (-(-(W - 1) * (I + X) // 32) + 1)
    bound = max(-(-W * (I + X) // 32), later)
    peaks = []
    for n in (10, 19, 46, 100, 181):
        r = oracle.page_window_schedule([I] * n, [X] * n, W, tail)
        assert r["peak"] <= bound and max(r["window_peaks"][1:], default=0) <= later
        peaks.append(r["peak"])
    assert max(peaks) <= bound
    no_evict = oracle.page_window_schedule([I] * 181, [X] * 181, 181, tail)["peak"]
    assert no_evict == -(-181 * (I + X) // 32) > 10 * bound


@pytest.mark.parametrize("seed", range(10))
def test_invariants_on_random_documents(seed):
    rng = random.Random(100 + seed)
    n = rng.randint(2, 14)
    W = rng.randint(2, 5)
    tail = rng.choice([0, 1, 31, 32, 33, 100])
    img = [rng.choice([0, rng.randint(1, 80)]) for _ in range(n)]
    txt = [rng.choice([0, rng.randint(1, 80)]) for _ in range(n)]
    r = oracle.page_window_schedule(img, txt, W, tail)
    wins = pw.windows(n, W)
    assert len(r["window_peaks"]) == len(wins)
    # windows cover every page, adjacent windows share exactly one page
    assert wins[0][0] == 0 and wins[-1][1] == n
    for (f0, l0), (f1, l1) in zip(wins, wins[1:]):
        assert f1 == l0 - 1 and l0 - f0 == W
    final = r["final"]
    # no token twice, and surviving tokens keep their append order
    assert len(set(final)) == len(final)
    order = {}
    for w, (first, last) in enumerate(wins):
        for kind in ("img", "txt"):
            for k in pw.new_pages(w, first, last):
                order[(kind, k)] = len(order)
    ranks = [(order[(t[0], t[1])], t[2]) for t in final]
    assert ranks == sorted(ranks)
    # the last window's new pages are all present, images then text, at the end
    first, last = wins[-1]
    tail_part = [("img", k, i) for k in pw.new_pages(len(wins) - 1, first, last) for i in range(img[k])]
    tail_part += [("txt", k, i) for k in pw.new_pages(len(wins) - 1, first, last) for i in range(txt[k])]
    assert final[len(final) - len(tail_part):] == tail_part
    if len(wins) >= 2:
        # the last boundary kept the shared page's image and the previous window's text tail
        shared = wins[-1][0]
        assert all(("img", shared, i) in final for i in range(img[shared]))
        f, l = wins[-2]
        prev_text = [("txt", k, i) for k in pw.new_pages(len(wins) - 2, f, l) for i in range(txt[k])]
        if tail > 0:
            assert all(t in final for t in prev_text[-tail:])
    # every kept block is whole: only the last block may be partial
    assert len(final) == 0 or -(-len(final) // 32) <= r["window_peaks"][-1]


def _no_overlap_windows(n_pages, window_pages):
    return [(f, min(f + window_pages, n_pages)) for f in range(0, n_pages, window_pages)]


def _reappend_shared(w, first, last):
    return range(first, last)


def _drop_shared_image(seq, shared_page, window_text, text_tail):
    return set(window_text[-text_tail:]) if text_tail > 0 else set()


def _first_text_instead_of_last(seq, shared_page, window_text, text_tail):
    keep = {j for j, t in enumerate(seq) if t[0] == "img" and t[1] == shared_page}
    return keep | set(window_text[:text_tail])


def _token_granular_compaction(seq, keep):
    return [seq[j] for j in sorted(keep)]


@pytest.mark.parametrize("name,mut", [
    ("windows", _no_overlap_windows),
    ("new_pages", _reappend_shared),
    ("keep_positions", _drop_shared_image),
    ("keep_positions", _first_text_instead_of_last),
    ("compact", _token_granular_compaction),
])
def test_planted_mistake_is_caught(name, mut, monkeypatch):
    monkeypatch.setattr(pw, name, mut)
    assert not _golden_pass(), f"a planted mistake in {name} went unnoticed"
