"""Seeded synthetic workloads shaped like the pages' decode and prefill cases.

Shared by the tests, ``smoke()`` and ``bench.py`` on both sides of a parity
check: the CPU oracle receives tensors regenerated here on the host, the HIP
path receives the same bits written into device memory (by a host copy for
small cases, by ``synth/fill.hip`` for large ones).  Nothing here computes
any step of the attention method.

Logical element order (what the counter of ``synth.rng`` indexes):

* main K / V of (layer, seq): element (h, t, d) -> (t*H + h)*D + d
* indexer K of (layer, seq): element (t, d) -> t*Di + d
* decode q of (layer, seq): (h, d) -> h*D + d; decode q_idx: d
* prefill q: (t, h, d) -> (t*H + h)*D + d; prefill q_idx: (t, d) -> t*Di + d

Device layout (block-major, one pool per layer): K/V ``[P][H][32][D]``,
indexer K ``[P][32][Di]``; one block table ``[B][max_blocks]`` shared by all
layers maps (seq, logical block) to a pool block, drawn as a seeded
permutation so that gathers are genuinely scattered.

Structure edits ("direction edits"): an indexer key row k is moved along the
layer's indexer query q of the same sequence as
``k <- bf16(f32(k) + f32(c * f32(q)))`` with float32 operations (no fused
multiply-add) and ``c = float32(a / ||q||)`` from a float64 norm: the score
q.k then grows by a*||q||, i.e. by ``a`` standard deviations of a N(0,1) key's
score.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np

from . import rng

ROLE_Q, ROLE_QIDX, ROLE_K, ROLE_V, ROLE_KIDX, ROLE_STRUCT = 1, 2, 3, 4, 5, 6
BLOCK = 32
H_DEFAULT, D_DEFAULT, DI_DEFAULT = 10, 128, 128


def tensor_id(role: int, layer: int, seq: int) -> int:
    return (role << 48) | (layer << 24) | seq


@dataclass
class Edit:
    """Add c * q_idx to the indexer-key rows ``tokens`` of (layer, seq)."""
    layer: int
    seq: int
    tokens: np.ndarray  # int64 positions
    coef: np.float32


@dataclass
class Workload:
    name: str
    seed: int
    batch: int
    layers: int
    ctx_lens: np.ndarray            # int64 [B]
    max_blocks: int
    mode: str = "decode"            # "decode" | "prefill"
    values: str = "normal"          # "normal" | "small_int"
    heads: int = H_DEFAULT
    head_dim: int = D_DEFAULT
    index_dim: int = DI_DEFAULT
    q_start: int = 0                # prefill only
    rows: int = 0                   # prefill only (T)
    edits: List[Edit] = field(default_factory=list)
    notes: str = ""
    layout: str = "permuted"        # "permuted": pool blocks in a seeded random order; "contiguous": in order

    # ---- derived structure -------------------------------------------------
    def nblocks(self, b: int) -> int:
        return -(-int(self.ctx_lens[b]) // BLOCK)

    @property
    def pool_blocks(self) -> int:
        return int(sum(self.nblocks(b) for b in range(self.batch)))

    def key(self, role: int, layer: int, seq: int) -> int:
        return rng.stream_key(self.seed, tensor_id(role, layer, seq))

    def block_table(self) -> np.ndarray:
        """int32 [B, max_blocks]; unused entries are -1."""
        P = self.pool_blocks
        if self.layout == "contiguous":
            perm = np.arange(P, dtype=np.int64)  # each sequence a run of consecutive pool blocks
        else:
            perm = rng.permutation(self.key(ROLE_STRUCT, 0xFFFF, 0), P)
        tab = np.full((self.batch, self.max_blocks), -1, dtype=np.int32)
        off = 0
        for b in range(self.batch):
            n = self.nblocks(b)
            tab[b, :n] = perm[off:off + n]
            off += n
        return tab

    def _values(self, key: int, idx: np.ndarray) -> np.ndarray:
        if self.values == "normal":
            return rng.normal_bf16(key, idx)
        if self.values == "small_int":
            return rng.small_int_bf16(key, idx)
        raise ValueError(self.values)

    # ---- host generation of logical tensors --------------------------------
    def q(self, layer: int, seq: int) -> np.ndarray:
        """Decode query [H, D] (bf16 bits)."""
        n = self.heads * self.head_dim
        return self._values(self.key(ROLE_Q, layer, seq), np.arange(n)).reshape(self.heads, self.head_dim)

    def q_idx(self, layer: int, seq: int) -> np.ndarray:
        """Decode indexer query [Di] (bf16 bits)."""
        return self._values(self.key(ROLE_QIDX, layer, seq), np.arange(self.index_dim))

    def q_rows(self, rows: np.ndarray, layer: int = 0) -> np.ndarray:
        """Prefill queries of chunk rows ``rows``: [len(rows), H, D]."""
        HD = self.heads * self.head_dim
        idx = (np.asarray(rows, np.int64)[:, None] * HD + np.arange(HD)[None, :])
        return self._values(self.key(ROLE_Q, layer, 0), idx.ravel()).reshape(len(rows), self.heads, self.head_dim)

    def q_idx_rows(self, rows: np.ndarray, layer: int = 0) -> np.ndarray:
        """Prefill indexer queries of chunk rows: [len(rows), Di]."""
        Di = self.index_dim
        idx = np.asarray(rows, np.int64)[:, None] * Di + np.arange(Di)[None, :]
        return self._values(self.key(ROLE_QIDX, layer, 0), idx.ravel()).reshape(len(rows), Di)

    def kv(self, role: int, layer: int, seq: int, t0: int, t1: int) -> np.ndarray:
        """Main K (role=ROLE_K) or V (ROLE_V) tokens [t0, t1): [H, t1-t0, D]."""
        H, D = self.heads, self.head_dim
        t = np.arange(t0, t1, dtype=np.int64)
        idx = ((t[:, None, None] * H + np.arange(H)[None, :, None]) * D + np.arange(D)[None, None, :])
        v = self._values(self.key(role, layer, seq), idx.ravel()).reshape(t1 - t0, H, D)
        return np.ascontiguousarray(v.transpose(1, 0, 2))

    def kv_tokens(self, role: int, layer: int, seq: int, toks: np.ndarray) -> np.ndarray:
        """Main K or V of arbitrary token positions: [H, len(toks), D]."""
        H, D = self.heads, self.head_dim
        t = np.asarray(toks, dtype=np.int64)
        idx = ((t[:, None, None] * H + np.arange(H)[None, :, None]) * D + np.arange(D)[None, None, :])
        v = self._values(self.key(role, layer, seq), idx.ravel()).reshape(t.size, H, D)
        return np.ascontiguousarray(v.transpose(1, 0, 2))

    def kidx(self, layer: int, seq: int, t0: int, t1: int) -> np.ndarray:
        """Indexer keys of tokens [t0, t1), edits applied: [t1-t0, Di]."""
        Di = self.index_dim
        t = np.arange(t0, t1, dtype=np.int64)
        idx = t[:, None] * Di + np.arange(Di)[None, :]
        out = self._values(self.key(ROLE_KIDX, layer, seq), idx.ravel()).reshape(t1 - t0, Di)
        for e in self.edits:
            if e.layer != layer or e.seq != seq:
                continue
            sel = (e.tokens >= t0) & (e.tokens < t1)
            if not np.any(sel):
                continue
            rows = e.tokens[sel] - t0
            out[rows] = apply_direction(out[rows], self.edit_query(layer, seq), e.coef)
        return out

    def edit_query(self, layer: int, seq: int) -> np.ndarray:
        """The indexer query whose direction edits move keys along."""
        if self.mode == "decode":
            return self.q_idx(layer, seq)
        # prefill: the last row of the chunk
        return self.q_idx_rows(np.array([self.rows - 1]), layer)[0]

    # ---- block-major pools (host; small workloads only) --------------------
    def host_pools(self, layer: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
        """(K pool [P,H,32,D], V pool, indexer-K pool [P,32,Di]) as uint16.

        Slots past a sequence's length are filled with the bf16 NaN pattern
        0x7FC0: no correct kernel ever reads them into a result.
        """
        P, H, D, Di = self.pool_blocks, self.heads, self.head_dim, self.index_dim
        kp = np.full((P, H, BLOCK, D), 0x7FC0, dtype=np.uint16)
        vp = np.full((P, H, BLOCK, D), 0x7FC0, dtype=np.uint16)
        ip = np.full((P, BLOCK, Di), 0x7FC0, dtype=np.uint16)
        tab = self.block_table()
        for b in range(self.batch):
            L = int(self.ctx_lens[b])
            if L == 0:
                continue
            k = self.kv(ROLE_K, layer, b, 0, L)
            v = self.kv(ROLE_V, layer, b, 0, L)
            ki = self.kidx(layer, b, 0, L)
            for j in range(self.nblocks(b)):
                t0, t1 = j * BLOCK, min((j + 1) * BLOCK, L)
                pb = tab[b, j]
                kp[pb, :, : t1 - t0, :] = k[:, t0:t1, :]
                vp[pb, :, : t1 - t0, :] = v[:, t0:t1, :]
                ip[pb, : t1 - t0, :] = ki[t0:t1, :]
        return kp, vp, ip


def apply_direction(k_bits: np.ndarray, q_bits: np.ndarray, coef: np.float32) -> np.ndarray:
    """bf16(f32(k) + f32(coef * f32(q))), float32 operations, no FMA."""
    kf = rng.bf16_bits_to_f32(k_bits)
    qf = rng.bf16_bits_to_f32(q_bits)
    step = (np.float32(coef) * qf).astype(np.float32)
    return rng.f32_to_bf16_bits((kf + step).astype(np.float32))


def direction_coef(q_bits: np.ndarray, sigmas: float) -> np.float32:
    """c = float32(sigmas / ||q||), the norm taken in float64."""
    qf = rng.bf16_bits_to_f32(q_bits).astype(np.float64)
    return np.float32(sigmas / math.sqrt(float(np.dot(qf, qf))))


# ---------------------------------------------------------------------------
# The five workloads.  Seeds: workload i uses 0x5EED0000 + i.
# ---------------------------------------------------------------------------

def _uniform_lengths(n: int, S: int) -> np.ndarray:
    return np.full(n, S, dtype=np.int64)


def decode_uniform(name: str, seed: int, batch: int, layers: int, S: int,
                   values: str = "normal") -> Workload:
    nb = -(-S // BLOCK)
    return Workload(name=name, seed=seed, batch=batch, layers=layers,
                    ctx_lens=_uniform_lengths(batch, S), max_blocks=nb, values=values)


def config1(values: str = "normal") -> Workload:
    """Single sequence, 1 layer, 1 decode query, S=2048 (64 blocks)."""
    return decode_uniform("single-seq decode S=2048", 0x5EED0001, 1, 1, 2048, values)


def config2(batch: int = 16, layers: int = 12) -> Workload:
    """Decode, 16 sequences x 12 layers at S=32768 (1024 blocks)."""
    return decode_uniform(f"decode B={batch} L={layers} S=32768", 0x5EED0002, batch, layers, 32768)


def planted_edits(wl: Workload, sigmas: float, per_query: int = 12) -> List[Edit]:
    """12 planted blocks per (layer, seq): distinct remote-candidate blocks at
    seeded positions, one seeded key per block moved ``sigmas`` along q_idx."""
    edits = []
    for l in range(wl.layers):
        for b in range(wl.batch):
            L = int(wl.ctx_lens[b])
            ncand = max(0, (L - 1) // BLOCK + 1 - 4)
            if ncand < per_query:
                continue
            key = wl.key(ROLE_STRUCT, l, b)
            perm = rng.permutation(key, ncand)[:per_query]
            offs = rng.draw_ints(key, ncand, per_query, 0, BLOCK)
            toks = np.sort(perm * BLOCK + offs).astype(np.int64)
            edits.append(Edit(l, b, toks, direction_coef(wl.q_idx(l, b), sigmas)))
    return edits


def plant_sigmas(S: int) -> float:
    """'+4 sigma' read as 4 standard deviations above the noise ceiling
    sqrt(2 ln S) of S N(0,1) key scores (the literal +4 does not separate the
    planted blocks from the noise maximum, about 4.4-4.9 sigma at 128K)."""
    return 4.0 + math.sqrt(2.0 * math.log(S))


def config3(batch: int = 16, layers: int = 12, S: int = 131072, sigmas: Optional[float] = None) -> Workload:
    """Decode, 16 x 12 layers at S=131072 with 12 planted blocks per query."""
    wl = decode_uniform(f"decode B={batch} L={layers} S={S} planted", 0x5EED0003, batch, layers, S)
    wl.edits = planted_edits(wl, plant_sigmas(S) if sigmas is None else sigmas)
    wl.notes = f"planted +{plant_sigmas(S) if sigmas is None else sigmas:.3f} sigma"
    return wl


PAGE_TOKENS, PAGE_IMAGE = 1000, 400


def config4(batch: int = 64, min_pages: int = 5, max_pages: int = 65) -> Workload:
    """Ragged decode: 64 sequences of 1000*U{5..65} tokens (whole pages of 400
    image + 600 text tokens), 1 layer; the image keys of 1-3 seeded earlier
    pages are correlated with the indexer query (cos ~ 0.5)."""
    seed = 0x5EED0004
    skey = rng.stream_key(seed, tensor_id(ROLE_STRUCT, 0xFFFE, 0))
    pages = rng.draw_ints(skey, 0, batch, min_pages, max_pages + 1)
    lens = pages * PAGE_TOKENS
    max_blocks = int(-(-int(lens.max()) // BLOCK))
    wl = Workload(name=f"ragged decode B={batch} pages {min_pages}-{max_pages}", seed=seed,
                  batch=batch, layers=1, ctx_lens=lens.astype(np.int64), max_blocks=max_blocks)
    beta = math.sqrt(128.0 / 3.0)
    for b in range(batch):
        key = wl.key(ROLE_STRUCT, 0, b)
        npg = int(pages[b])
        ncorr = int(rng.draw_ints(key, 0, 1, 1, 4)[0])
        ncorr = min(ncorr, npg - 1)
        chosen = np.sort(rng.permutation(key ^ 0x5A5A, npg - 1)[:ncorr])
        toks = np.concatenate([np.arange(pg * PAGE_TOKENS, pg * PAGE_TOKENS + PAGE_IMAGE) for pg in chosen])
        wl.edits.append(Edit(0, b, toks.astype(np.int64), direction_coef(wl.q_idx(0, b), beta)))
    wl.notes = "pages: 400 image + 600 text tokens; correlated image keys of 1-3 earlier pages"
    return wl


def page_tags(max_blocks: int, page_tokens: int = PAGE_TOKENS, image_tokens: int = PAGE_IMAGE) -> np.ndarray:
    """Page tag of each logical block when a document is laid out as pages of
    ``image_tokens`` image tokens followed by text, ``page_tokens`` tokens per
    page: the page whose image tokens the block holds, or -1 for a block with
    none.  This is input metadata for the page-aware ranking (a block never
    holds image tokens of two pages while a page has more than 32 text
    tokens)."""
    tags = np.full(max_blocks, -1, np.int32)
    for j in range(max_blocks):
        lo, hi = j * BLOCK, j * BLOCK + BLOCK - 1
        for pg in range(lo // page_tokens, hi // page_tokens + 1):
            if lo < pg * page_tokens + image_tokens and hi >= pg * page_tokens:
                tags[j] = pg
    return tags


def page_of(position: int, page_tokens: int = PAGE_TOKENS) -> int:
    """Page holding token ``position`` (the query's page)."""
    return int(position) // page_tokens


def config5(rows: int = 2048, S: int = 131072) -> Workload:
    """Chunked prefill: 2048 new rows at offset S-2048 of an S-token context."""
    return Workload(name=f"chunked prefill T={rows} at {S - rows} of S={S}", seed=0x5EED0005, batch=1,
                    layers=1, ctx_lens=np.array([S], np.int64), max_blocks=-(-S // BLOCK),
                    mode="prefill", q_start=S - rows, rows=rows)


def prefill_case(name: str, seed: int, S: int, q_start: int, rows: int, values: str = "normal") -> Workload:
    """A smaller chunked-prefill case (parity tests)."""
    return Workload(name=name, seed=seed, batch=1, layers=1, ctx_lens=np.array([S], np.int64),
                    max_blocks=-(-S // BLOCK), mode="prefill", q_start=q_start, rows=rows, values=values)


CONFIGS = {1: config1, 2: config2, 3: config3, 4: config4, 5: config5}
