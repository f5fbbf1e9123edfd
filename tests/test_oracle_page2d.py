"""Pins of the oracle's page2d rotary encoding and cache write
(news.rkmt.cn/news/25027 Sec. 4 and Sec. 6): hand-worked values, the
identity, isometry, relative-position and composition properties of a
rotation, the page-parity axis, the bfloat16 rounding rule and the block-major
placement -- each of which a plausible mistake (pair layout, theta, page
modulus, rounding) breaks."""
from __future__ import annotations

import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden():
    consts, cases = {}, []
    with open(os.path.join(GOLDEN, "page2d_rope.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            k, *v = line.split()
            if k == "case":
                cases.append(v)
            else:
                consts[k] = v
    return consts, cases


def _bits(x):
    return (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_golden_frequencies():
    c, _ = _golden()
    inv_tok, inv_page = oracle.page2d_inv_freq()
    assert inv_tok.size == int(c["tok_pairs"][0]) and inv_page.size == int(c["page_pairs"][0])
    assert inv_tok[0] == float(c["inv_tok_first"][0])
    assert abs(inv_tok[-1] - float(c["inv_tok_last"][0])) <= 1e-9
    assert inv_page[0] == float(c["inv_page"][0])


def test_golden_rotations():
    _, cases = _golden()
    for name, tok, page, *pairs in cases:
        x = np.zeros(128, np.uint16)
        x[int(name[1:])] = 0x3F80
        y = oracle.rope_page2d(x, int(tok), int(page))
        for dim, bits in zip(pairs[0::2], pairs[1::2]):
            assert y[int(dim)] == int(bits, 16), (name, tok, page, dim, hex(y[int(dim)]))
        touched = {int(d) for d in pairs[0::2]}
        assert all((y[d] & 0x7FFF) == 0 for d in range(128) if d not in touched), name   # +-0


def test_identity_at_origin_and_even_page():
    g = np.random.default_rng(1)
    x = _bits(g.standard_normal((10, 128)))
    np.testing.assert_array_equal(oracle.rope_page2d(x, 0, 0), x)
    np.testing.assert_array_equal(oracle.rope_page2d(x, 0, 6), x)    # page 6 mod 2 = 0


def test_isometry_and_composition():
    g = np.random.default_rng(2)
    x = g.standard_normal((4, 128))
    for tok, page in [(1, 0), (777, 1), (131071, 5)]:
        y = oracle.rope_page2d_f64(x, tok, page)
        np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-12)
    a = oracle.rope_page2d_f64(oracle.rope_page2d_f64(x, 300, 1), 41, 0)
    np.testing.assert_allclose(a, oracle.rope_page2d_f64(x, 341, 1), atol=1e-9)


def test_scores_depend_on_relative_offset_and_page_parity():
    g = np.random.default_rng(3)
    q, k = g.standard_normal(128), g.standard_normal(128)

    def score(tq, pq, tk, pk):
        return float(oracle.rope_page2d_f64(q, tq, pq) @ oracle.rope_page2d_f64(k, tk, pk))

    base = score(120, 3, 17, 3)
    assert abs(score(120 + 500, 3, 17 + 500, 3) - base) < 1e-9       # shift of both token offsets
    assert abs(score(120, 5, 17, 5) - base) < 1e-9                   # same parity, other pages
    assert abs(score(120, 3, 17, 4) - base) > 1e-6                   # adjacent page differs
    assert abs(score(120, 3, 17, 4) - score(120, 1, 17, 0)) < 1e-9   # only the parity difference matters


def test_bf16_rounding_is_nearest_even():
    one = 1.0
    ulp = 2.0 ** -7
    vals = np.array([one + ulp / 2, one + 3 * ulp / 2, one + ulp / 4, -(one + ulp / 2), 0.0, -0.0,
                     one + ulp / 2 + 2.0 ** -30], np.float64)
    got = oracle.bf16_bits_nearest(vals)
    want = [0x3F80, 0x3F82, 0x3F80, 0xBF80, 0x0000, 0x8000, 0x3F81]
    assert [int(v) for v in got] == want
    # against float32 values: exact for bf16-representable inputs
    g = np.random.default_rng(4)
    f = g.standard_normal(1000).astype(np.float32)
    b = _bits(f)
    wide = oracle.widen(b)
    np.testing.assert_array_equal(oracle.bf16_bits_nearest(wide), b)


def test_cache_write_places_rows_by_block_table():
    g = np.random.default_rng(5)
    P, H = 6, 10
    kp = np.zeros((P, H, 32, 128), np.uint16)
    vp = np.zeros_like(kp)
    ip = np.zeros((P, 32, 128), np.uint16)
    table = np.array([[4, 1, 5], [0, 2, 3]], np.int32)
    kn = _bits(g.standard_normal((H, 128)))
    vn = _bits(g.standard_normal((H, 128)))
    inn = _bits(g.standard_normal(128))
    oracle.cache_write(kp, vp, ip, table, 1, 70, kn, vn, inn, 70 - 64, 2)
    # position 70 of sequence 1: logical block 2 -> pool block 3, row 6
    np.testing.assert_array_equal(vp[3, :, 6, :], vn)
    np.testing.assert_array_equal(kp[3, :, 6, :], oracle.rope_page2d(kn, 6, 2))
    np.testing.assert_array_equal(ip[3, 6, :], oracle.rope_page2d(inn, 6, 2))
    assert np.count_nonzero(vp) == np.count_nonzero(vp[3, :, 6, :])


def _mutants():
    import oracle.page2d as m

    def interleaved(x, tok_pos, page_pos):        # pairs (2i, 2i+1) instead of (i, i+64)
        x = np.asarray(x, np.float64)
        ang = m.page2d_angles(tok_pos, page_pos, x.shape[-1])
        c, s = np.cos(ang), np.sin(ang)
        y = x.copy()
        y[..., 0::2] = x[..., 0::2] * c - x[..., 1::2] * s
        y[..., 1::2] = x[..., 1::2] * c + x[..., 0::2] * s
        return y

    def yarn_theta(head_dim=128, tok_theta=None, page_theta=256.0, page_pairs=1):
        return ORIG["inv"](head_dim, 500000.0, page_theta, page_pairs)

    def no_page_mod(tok_pos, page_pos, head_dim=128):
        inv_tok, inv_page = m.page2d_inv_freq(head_dim)
        return np.concatenate([float(tok_pos) * inv_tok, float(page_pos) * inv_page])

    return {"rope_page2d_f64": interleaved, "page2d_inv_freq": yarn_theta, "page2d_angles": no_page_mod}


ORIG = {}


def _pins_pass():
    try:
        test_golden_frequencies()
        test_golden_rotations()
        test_identity_at_origin_and_even_page()
        test_scores_depend_on_relative_offset_and_page_parity()
    except AssertionError:
        return False
    return True


@pytest.mark.parametrize("name", sorted(_mutants().keys()))
def test_planted_mistake_is_caught(name, monkeypatch):
    import oracle.page2d as m
    ORIG["inv"] = m.page2d_inv_freq
    mut = _mutants()[name]
    monkeypatch.setattr(m, name, mut)
    monkeypatch.setattr(oracle, name, mut)
    assert not _pins_pass(), f"a planted mistake in {name} went unnoticed"


def test_unmutated_page2d_passes_the_same_checks():
    assert _pins_pass()


# ---------------------------------------------------------------- coordinates

def _golden_coords():
    d = {}
    for line in open(os.path.join(os.path.dirname(__file__), "golden", "page_coords.txt")):
        if line.startswith("#") or not line.strip():
            continue
        k, *v = line.split()
        d[k] = [int(x) for x in v]
    return d


def test_page_coords_golden_stream():
    g = _golden_coords()
    tp, pp, st = oracle.page_coords(g["tokens"], g["marker"][0], tuple(g["start"]))
    assert list(tp) == g["tok"] and list(pp) == g["page"] and list(st) == g["after"]
    tp2, pp2, st2 = oracle.page_coords(g["tokens2"], g["marker"][0], st)
    assert list(tp2) == g["tok2"] and list(pp2) == g["page2"] and list(st2) == g["after2"]


def _closed_form(tokens, marker, state):
    """page = start page + markers so far; tok = distance to the last marker,
    or the start tok + 1 + index before the first one."""
    t = np.asarray(tokens)
    is_m = t == marker
    idx = np.arange(t.size)
    last = np.maximum.accumulate(np.where(is_m, idx, -1)) if t.size else idx
    page = state[0] + np.cumsum(is_m)
    tok = np.where(last >= 0, idx - last, state[1] + 1 + idx)
    return tok, page


@pytest.mark.parametrize("density", [0.0, 0.01, 0.3, 1.0])
def test_page_coords_closed_form_and_chunking(density):
    g = np.random.default_rng(int(density * 1000) + 5)
    marker = 9
    toks = np.where(g.random(5000) < density, marker, g.integers(0, 9, 5000))
    start = (int(g.integers(0, 50)), int(g.integers(-1, 300)))
    tp, pp, st = oracle.page_coords(toks, marker, start)
    ct, cp = _closed_form(toks, marker, start)
    np.testing.assert_array_equal(tp, ct)
    np.testing.assert_array_equal(pp, cp)
    # prefill of the whole stream == chunked prefill == one-token decode steps
    cuts = sorted(g.choice(np.arange(1, 5000), 7, replace=False))
    s, parts_t, parts_p = start, [], []
    for a, b in zip([0] + cuts, cuts + [5000]):
        a_t, a_p, s = oracle.page_coords(toks[a:b], marker, s)
        parts_t.append(a_t)
        parts_p.append(a_p)
    np.testing.assert_array_equal(np.concatenate(parts_t), tp)
    np.testing.assert_array_equal(np.concatenate(parts_p), pp)
    assert s == st
    s2 = start
    for x in toks[:300]:
        (t1,), (p1,), s2 = oracle.page_coords([x], marker, s2)
    assert (t1, p1) == (tp[299], pp[299])


def test_page_coords_planted_mistakes():
    g = _golden_coords()
    m = g["marker"][0]

    def no_reset(tokens, marker, state=(0, -1)):       # a marker advances tok instead of resetting it
        page, tok = state
        out_t, out_p = [], []
        for x in tokens:
            page += int(x == marker)
            tok += 1
            out_t.append(tok)
            out_p.append(page)
        return out_t, out_p, (page, tok)

    def marker_on_old_page(tokens, marker, state=(0, -1)):   # the marker stays on the page it closes
        page, tok = state
        out_t, out_p = [], []
        for x in tokens:
            if x == marker:
                out_t.append(0)
                out_p.append(page)
                page += 1
                tok = 0
            else:
                tok += 1
                out_t.append(tok)
                out_p.append(page)
        return out_t, out_p, (page, tok)

    for mut in (no_reset, marker_on_old_page):
        tp, pp, _ = mut(g["tokens"], m, tuple(g["start"]))
        assert list(tp) != g["tok"] or list(pp) != g["page"], mut.__name__
