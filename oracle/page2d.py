"""page2d rotary position encoding and the cache write, on the CPU.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[rkmt] Sec. 4 ("page2d position encoding") and Sec. 6 (conclusions):
* the 128 dims of a head form 64 rotation pairs, split between two axes: the
  page axis takes ``page_pairs`` = 1 pair, the token axis the other 63;
* token axis: theta 10000, coordinate = the token's offset inside its page;
  page axis: theta 256, coordinate = page number mod 2 (``page_mod``);
* "resample": the token axis samples its own spectrum over its reduced
  dimension count -- read as the standard rotary frequencies
  theta^(-2i/d) with d = 2 * 63 = 126 dims, i = 0..62;
* the angles are concatenated token-first, cat(tok, page), and then doubled,
  cat(ang, ang), into the cos/sin vectors: the rotate-half layout, where dim
  i pairs with dim i + 64;
* the main attention's q/k and the indexer's q/k share the coordinates; K
  is stored rotated in the cache.
The rotation is exact in float64 and rounded once to bfloat16 (nearest, ties
to even).

Coordinates ([rkmt] Sec. 4, how positions are built and advanced): a page
marker token opens a new page, so the page coordinate counts markers, and
the token coordinate is the running count inside the current page.  In
decoding, a {page, tok} state advances one token at a time: a marker adds one
to page and sends tok back to the start of that page's segment; any other
token adds one to tok.  Reading taken: the segment start is coordinate 0 and
the marker is the first token of its page, so prefill of a stream and
token-by-token decode are the same rule (``page_coords``), and prefill of a
concatenation equals prefill of its first part followed by the rest.
"""
from __future__ import annotations

import numpy as np

from .sr_swa import widen

TOK_THETA = 10000.0
PAGE_THETA = 256.0
PAGE_PAIRS = 1
PAGE_MOD = 2


def page_coords(tokens, marker: int, state=(0, -1)):
    """(tok_pos, page_pos, state after) of a token stream from ``state`` =
    (page, tok) of the token before it ([rkmt] Sec. 4): a marker token opens
    page + 1 at tok 0; any other token is tok + 1 on the same page."""
    page, tok = int(state[0]), int(state[1])
    tok_pos = np.empty(len(tokens), np.int64)
    page_pos = np.empty(len(tokens), np.int64)
    for i, x in enumerate(tokens):
        if int(x) == marker:
            page += 1
            tok = 0
        else:
            tok += 1
        tok_pos[i] = tok
        page_pos[i] = page
    return tok_pos, page_pos, (page, tok)


def page2d_inv_freq(head_dim: int = 128, tok_theta: float = TOK_THETA, page_theta: float = PAGE_THETA,
                    page_pairs: int = PAGE_PAIRS):
    """(inv_tok [63], inv_page [1]) for a 128-dim head ([rkmt] Sec. 4, 6)."""
    d_tok = head_dim - 2 * page_pairs
    d_page = 2 * page_pairs
    inv_tok = tok_theta ** (-np.arange(0, d_tok, 2, dtype=np.float64) / d_tok)
    inv_page = page_theta ** (-np.arange(0, d_page, 2, dtype=np.float64) / d_page)
    return inv_tok, inv_page


def page2d_angles(tok_pos: int, page_pos: int, head_dim: int = 128) -> np.ndarray:
    """The head_dim/2 rotation angles of a token: token angles, then page."""
    inv_tok, inv_page = page2d_inv_freq(head_dim)
    return np.concatenate([float(tok_pos) * inv_tok, float(int(page_pos) % PAGE_MOD) * inv_page])


def rope_page2d_f64(x: np.ndarray, tok_pos: int, page_pos: int) -> np.ndarray:
    """Rotate float64 rows x [..., 128] (rotate-half pairs (i, i + 64))."""
    x = np.asarray(x, dtype=np.float64)
    half = x.shape[-1] // 2
    ang = page2d_angles(tok_pos, page_pos, x.shape[-1])
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def bf16_bits_nearest(x: np.ndarray) -> np.ndarray:
    """float64 -> bfloat16 bit patterns, rounded once to nearest (ties to
    even), the sign of zero kept.  Finite values of normal bf16 range only."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                          # x = m * 2^e, 0.5 <= |m| < 1
    scale = np.ldexp(1.0, e - 8)                # bf16 keeps 8 significant bits
    r = np.where(x == 0.0, x, np.round(x / scale) * scale)     # np.round: half to even; zeros keep their sign
    f = r.astype(np.float32)                    # exact: r has <= 8 significant bits
    assert np.all(np.isfinite(f))
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def rope_page2d(x_bits: np.ndarray, tok_pos: int, page_pos: int) -> np.ndarray:
    """Rotated bf16 bit patterns of bf16 rows x_bits [..., 128]."""
    return bf16_bits_nearest(rope_page2d_f64(widen(x_bits), tok_pos, page_pos))


def cache_write(k_pool, v_pool, kidx_pool, block_table, seq: int, pos: int, k_new, v_new, kidx_new,
                tok_pos: int, page_pos: int):
    """Write one new token of sequence ``seq`` at position ``pos`` into the
    block-major pools (numpy arrays, modified in place): K and the indexer K
    rotated, V as given.  Pools: K/V [P][H][32][D], indexer K [P][32][Di]."""
    pb = int(block_table[seq][pos // 32])
    r = pos % 32
    k_pool[pb, :, r, :] = rope_page2d(k_new, tok_pos, page_pos)
    v_pool[pb, :, r, :] = v_new
    kidx_pool[pb, r, :] = rope_page2d(kidx_new, tok_pos, page_pos)
