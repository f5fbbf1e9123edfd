"""CPU oracle for SR-SWA block-sparse attention -- TEST INFRASTRUCTURE ONLY.

This package is the slow, plain reference the HIP path is checked against.
Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  The library in ``block_sparse_long_sr_amd`` never
imports, calls or links anything here, and this package imports nothing from
the library: the two share no code.  Inputs are bfloat16 values passed as
their 16-bit patterns (``numpy.uint16``) and widened exactly.

Sources (cited by short name in the docstrings):

* [rkmt]   news.rkmt.cn/news/25027 -- Unlimited-OCR-2 architecture walk-through.
           Sec. 5 "SR-SWA: how the block-sparse attention is realised", steps
           1-4 (blocking, scoring, selection, computation); Sec. 3 (10 heads,
           MHA, the Lightning Indexer inside the attention layer); Sec. 4
           (K is stored already rotated in the cache).
* [lqnn]   www.lqnn.cn/news/271890 -- Unlimited-OCR-2-8bit explainer, section
           on the 128K KV-cache budget (16 blocks x 32 = 512 tokens, top-12
           remote + 4 local).
* [lehvn]  leheavengame.com article on the OCR 2 release (KV cache 47 GB ->
           1.77 GB), Sec. 2 route A (Page Gate, Token Sieve, Local Window)
           and Sec. 3 (the chunked-prefill [tokens, context/32] temporary).

Modules: ``sr_swa`` (steps 1-4 of the attention, the page-aware ranking),
``page2d`` (the page2d rotary encoding and the cache write, [rkmt]
Sec. 4) and ``page_window`` (the page-window schedule of continuous
decoding, [lehvn] Sec. 2 route A, storage half).

Where the pages leave a step open, the reading taken is stated at the
function that implements it.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``,
``tests/test_oracle_page2d.py`` and ``tests/test_oracle_page_window.py``
(brute force, dense-attention special cases, invariants, exact integer
cases, golden fixtures).  None is "parity unpinned".
"""
from .sr_swa import (  # noqa: F401
    SparseCfg,
    widen,
    block_count,
    local_blocks,
    candidate_count,
    indexer_scores,
    block_maxima,
    rank_candidates,
    page_tiers,
    select_blocks,
    attended_tokens,
    attend,
    decode_query,
    decode_query_fetch,
    prefill_rows,
    prefill_rows_fetch,
)
from .page2d import (  # noqa: F401
    page_coords,
    page2d_inv_freq,
    page2d_angles,
    rope_page2d_f64,
    rope_page2d,
    bf16_bits_nearest,
    cache_write,
)
from .page_window import page_window_schedule  # noqa: F401
