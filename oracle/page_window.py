"""Page-window schedule of continuous decoding, token by token.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[lehvn] Sec. 2 (route A, storage half): the document is parsed in page
windows, adjacent windows share one page; on entering the next window the
shared page's visual KV and the text at the end of the previous window are
kept, the rest is released.  Sec. 3: the serving deployment's base window is
10 pages.

Readings taken:
* window w covers pages w(W-1) .. w(W-1)+W-1; its first page (w > 0) is the
  shared page: its visual tokens are reused and its text was produced in
  window w-1, so window w appends the visual tokens of its other pages, then
  their text;
* the closing text of the previous window is its last text_tail text tokens;
* the cache is paged in blocks of 32 token slots and memory is released per
  block: a block holding any kept token is kept whole (its other tokens stay
  in the context), and kept blocks are renumbered in order.

Tokens are labelled ("img"|"txt", page, index); the sequence is a list of
labels and a block is 32 consecutive list entries.
"""
from __future__ import annotations

from typing import Dict, List, Sequence, Tuple

BLOCK = 32
Label = Tuple[str, int, int]


def _blocks(n_tokens: int) -> int:
    return -(-n_tokens // BLOCK)


def windows(n_pages: int, window_pages: int) -> List[Tuple[int, int]]:
    """Page ranges [first, last) of the windows: stride W-1, so adjacent
    windows share one page; the last window is the first to reach the last
    page."""
    out = []
    first = 0
    while first < n_pages:
        last = min(first + window_pages, n_pages)
        out.append((first, last))
        if last == n_pages:
            break
        first += window_pages - 1
    return out


def new_pages(w: int, first: int, last: int) -> range:
    """Pages whose tokens window w appends: all of them in window 0, all but
    the shared first page afterwards."""
    return range(first if w == 0 else first + 1, last)


def keep_positions(seq: List[Label], shared_page: int, window_text: List[int], text_tail: int) -> set:
    """Positions kept at a window boundary: the shared page's image tokens
    and the last text_tail positions of the window's text."""
    keep = {j for j, t in enumerate(seq) if t[0] == "img" and t[1] == shared_page}
    if text_tail > 0:
        keep |= set(window_text[-text_tail:])
    return keep


def compact(seq: List[Label], keep: set) -> List[Label]:
    """Keep every 32-slot block that holds a kept position, whole and in
    order; the kept blocks are renumbered 0, 1, ..."""
    kept_blocks = sorted({j // BLOCK for j in keep})
    return [t for b in kept_blocks for t in seq[b * BLOCK:(b + 1) * BLOCK]]


def page_window_schedule(image_tokens: Sequence[int], text_tokens: Sequence[int], window_pages: int,
                         text_tail: int) -> Dict:
    """Run the schedule; returns the per-window peak block counts, the
    overall peak, and the final token list."""
    assert window_pages >= 2 and text_tail >= 0
    assert len(image_tokens) == len(text_tokens)
    seq: List[Label] = []
    peaks: List[int] = []
    wins = windows(len(image_tokens), window_pages)
    for w, (first, last) in enumerate(wins):
        pages = new_pages(w, first, last)
        peak = _blocks(len(seq))
        for k in pages:
            seq.extend(("img", k, i) for i in range(image_tokens[k]))
            peak = max(peak, _blocks(len(seq)))
        for k in pages:
            seq.extend(("txt", k, i) for i in range(text_tokens[k]))
            peak = max(peak, _blocks(len(seq)))
        peaks.append(peak)
        if w + 1 < len(wins):
            window_text = [j for j, t in enumerate(seq) if t[0] == "txt" and t[1] in pages]
            seq = compact(seq, keep_positions(seq, last - 1, window_text, text_tail))
    return {"window_peaks": peaks, "peak": max(peaks, default=0), "final": seq}
