"""Python binding of libuocr_sparse.so, the SR-SWA block-sparse attention hot
path for MI355X (gfx950).

Argument marshalling only: every function forwards to the C entry point of
the same name (``uocr_<name>`` in ``include/uocr_sparse.h``) and raises
``UocrError`` on a non-zero status.  Tensor arguments are ``torch.Tensor``s on
the GPU (their ``data_ptr()`` is passed) or raw integer device pointers; the
stream defaults to torch's current stream.  There is no fallback: importing
this package without the built library raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

__all__ = [
    "SparseCfg", "KV", "UocrError", "lib_path", "make_cfg", "make_kv",
    "indexer_score_decode", "block_topk_decode", "sparse_attn_decode", "topk_attn_decode",
    "indexer_score_prefill", "block_topk_prefill", "sparse_attn_prefill",
    "workspace_size", "status_string", "last_error", "abi_version",
    "OP_INDEXER_DECODE", "OP_TOPK_DECODE", "OP_ATTN_DECODE",
    "OP_INDEXER_PREFILL", "OP_TOPK_PREFILL", "OP_ATTN_PREFILL", "OP_DENSE_ATTN_DECODE", "dense_attn_decode",
    "OP_DECODE_STEP", "sparse_decode_step", "sparse_decode_step_static", "check_decode_step", "DecodeStepWaitError", "STEP_AUTO", "STEP_ONE_LAUNCH", "STEP_PER_LAYER",
    "rope_cache_write", "rope_queries", "page_coords", "BlockPool", "PageWindow",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libuocr_sparse.so")

OP_INDEXER_DECODE, OP_TOPK_DECODE, OP_ATTN_DECODE = 0, 1, 2
OP_INDEXER_PREFILL, OP_TOPK_PREFILL, OP_ATTN_PREFILL = 3, 4, 5
OP_DENSE_ATTN_DECODE = 6
OP_DECODE_STEP = 7
STEP_AUTO, STEP_ONE_LAUNCH, STEP_PER_LAYER = 0, 1, 2


class SparseCfg(ctypes.Structure):
    """Mirror of ``uocr_sparse_cfg``."""
    _fields_ = [
        ("block_size", ctypes.c_int32),
        ("topk_blocks", ctypes.c_int32),
        ("local_blocks", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("index_dim", ctypes.c_int32),
        ("sm_scale", ctypes.c_float),
    ]


class KV(ctypes.Structure):
    """Mirror of ``uocr_kv`` (one layer's block-major cache)."""
    _fields_ = [
        ("k_pool", ctypes.c_void_p),
        ("v_pool", ctypes.c_void_p),
        ("kidx_pool", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
        ("ctx_lens", ctypes.c_void_p),
        ("num_blocks", ctypes.c_int64),
        ("batch", ctypes.c_int32),
        ("max_blocks", ctypes.c_int32),
        ("block_page", ctypes.c_void_p),
        ("query_page", ctypes.c_void_p),
    ]


class PageWindow(ctypes.Structure):
    _fields_ = [("window_pages", ctypes.c_int32), ("text_tail_tokens", ctypes.c_int32)]


class UocrError(RuntimeError):
    def __init__(self, status: int, func: str):
        self.status = status
        msg = _lib.uocr_last_error().decode(errors="replace")
        super().__init__(f"{func}: {_lib.uocr_status_string(status).decode()}: {msg}")


if not os.path.exists(lib_path):
    raise ImportError(
        f"{lib_path} is missing: build it with `python -m block_sparse_long_sr_amd.build` "
        "(there is no CPU fallback)")

_lib = ctypes.CDLL(lib_path)

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_SZ = ctypes.c_size_t
_CFG = ctypes.POINTER(SparseCfg)
_KV = ctypes.POINTER(KV)

_SIGS = {
    "uocr_indexer_score_decode": ([_CFG, _KV, _P, _P, _P], ctypes.c_int),
    "uocr_block_topk_decode": ([_CFG, _P, _P, _I32, _I32, _P, _P, _P], ctypes.c_int),
    "uocr_sparse_attn_decode": ([_CFG, _KV, _P, _P, _P, _P, _P, _SZ, _P], ctypes.c_int),
    "uocr_topk_attn_decode": ([_CFG, _KV, _P, _P, _P, _P, _P, _P, _P, _SZ, _P], ctypes.c_int),
    "uocr_dense_attn_decode": ([_CFG, _KV, _P, _P, _P, _P, _SZ, _P], ctypes.c_int),
    "uocr_sparse_decode_step": ([_CFG, _KV, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P], ctypes.c_int),
    "uocr_sparse_decode_step_static": ([_CFG, _KV, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P], ctypes.c_int),
    "uocr_rope_cache_write": ([_CFG, _KV, ctypes.c_int32, _P, _P, _P, _P, _P, _P, _P, _P], ctypes.c_int),
    "uocr_rope_queries": ([_CFG, ctypes.c_int32, _P, _P, _P, _P, _P], ctypes.c_int),
    "uocr_indexer_score_prefill": ([_CFG, _KV, _P, _I32, _I32, _P, _SZ, _P], ctypes.c_int),
    "uocr_block_topk_prefill": ([_CFG, _P, _SZ, _I32, _I32, _I32, _P, _P, _P], ctypes.c_int),
    "uocr_sparse_attn_prefill": ([_CFG, _KV, _P, _I32, _I32, _P, _P, _P, _P, _SZ, _P], ctypes.c_int),
    "uocr_page_coords": ([_I32, _I32, _P, _I32, _P, _P, _P, _P], ctypes.c_int),
    "uocr_pool_create": ([_I32, _I32], _P),
    "uocr_pool_destroy": ([_P], None),
    "uocr_pool_append": ([_P, _I32, ctypes.c_int64], ctypes.c_int),
    "uocr_pool_keep": ([_P, _I32, _P, _I32], ctypes.c_int),
    "uocr_pool_table": ([_P, _I32, _P, _I32, _P], ctypes.c_int),
    "uocr_pool_used": ([_P], ctypes.c_int64),
    "uocr_pool_peak": ([_P], ctypes.c_int64),
    "uocr_page_window_run": ([ctypes.POINTER(PageWindow), _P, _P, _I32, _P, _I32, _P, _I32, _P], ctypes.c_int),
    "uocr_workspace_size": ([_CFG, _I32, _I32, _I32], ctypes.c_size_t),
    "uocr_status_string": ([_I32], ctypes.c_char_p),
    "uocr_last_error": ([], ctypes.c_char_p),
    "uocr_abi_version": ([], ctypes.c_int32),
}
for _name, (_args, _res) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = _res


def _ptr(x) -> Optional[int]:
    """Device address of a tensor, an int pointer, or a (pointer, bytes) pair."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if isinstance(x, tuple):
        return int(x[0])
    if not x.is_contiguous():
        raise ValueError("tensor arguments must be contiguous (the C ABI takes dense row-major buffers)")
    return x.data_ptr()


def _nbytes(x) -> int:
    """Byte size of a workspace given as a tensor or a (pointer, bytes) pair."""
    if x is None:
        return 0
    if isinstance(x, tuple):
        return int(x[1])
    if isinstance(x, int):
        raise TypeError("pass a workspace as a tensor or a (pointer, bytes) pair")
    return x.numel() * x.element_size()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, func: str) -> None:
    if status != 0:
        raise UocrError(status, func)


def make_cfg(topk_blocks: int = 16, local_blocks: int = 4, num_heads: int = 10, head_dim: int = 128,
             index_dim: int = 128, block_size: int = 32, sm_scale: Optional[float] = None) -> SparseCfg:
    """Configuration with the released model's defaults (32 / 16 / 4 / 10 x 128)."""
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(head_dim)
    return SparseCfg(block_size, topk_blocks, local_blocks, num_heads, head_dim, index_dim, sm_scale)


def make_kv(k_pool, v_pool, kidx_pool, block_table, ctx_lens, num_blocks: int, batch: int, max_blocks: int,
            block_page=None, query_page=None) -> KV:
    """``block_page`` / ``query_page`` (int32 device tensors or None) turn on
    the page-aware ranking of the selecting entry points."""
    return KV(_ptr(k_pool), _ptr(v_pool), _ptr(kidx_pool), _ptr(block_table), _ptr(ctx_lens),
              int(num_blocks), int(batch), int(max_blocks), _ptr(block_page), _ptr(query_page))


def indexer_score_decode(cfg: SparseCfg, kv: KV, q_idx, block_scores, stream=None) -> None:
    _check(_lib.uocr_indexer_score_decode(ctypes.byref(cfg), ctypes.byref(kv), _ptr(q_idx), _ptr(block_scores),
                                          _stream(stream)), "indexer_score_decode")


def block_topk_decode(cfg: SparseCfg, block_scores, ctx_lens, batch: int, max_blocks: int, block_idx,
                      n_sel=None, stream=None) -> None:
    _check(_lib.uocr_block_topk_decode(ctypes.byref(cfg), _ptr(block_scores), _ptr(ctx_lens), batch, max_blocks,
                                       _ptr(block_idx), _ptr(n_sel), _stream(stream)), "block_topk_decode")


def sparse_attn_decode(cfg: SparseCfg, kv: KV, q, block_idx, out, lse=None, ws=None, stream=None) -> None:
    _check(_lib.uocr_sparse_attn_decode(ctypes.byref(cfg), ctypes.byref(kv), _ptr(q), _ptr(block_idx), _ptr(out),
                                        _ptr(lse), _ptr(ws), _nbytes(ws), _stream(stream)), "sparse_attn_decode")


def topk_attn_decode(cfg: SparseCfg, kv: KV, q, block_scores, block_idx, out, lse=None, n_sel=None, ws=None,
                     stream=None) -> None:
    _check(_lib.uocr_topk_attn_decode(ctypes.byref(cfg), ctypes.byref(kv), _ptr(q), _ptr(block_scores),
                                      _ptr(block_idx), _ptr(n_sel), _ptr(out), _ptr(lse), _ptr(ws), _nbytes(ws),
                                      _stream(stream)), "topk_attn_decode")


def dense_attn_decode(cfg: SparseCfg, kv: KV, q, out, lse=None, ws=None, stream=None) -> None:
    """Full-context attention of each sequence's query (the dense comparator);
    ``ws`` as for the other entries: a tensor or (pointer, bytes)."""
    _check(_lib.uocr_dense_attn_decode(ctypes.byref(cfg), ctypes.byref(kv), _ptr(q), _ptr(out), _ptr(lse), _ptr(ws),
                                       _nbytes(ws), _stream(stream)), "dense_attn_decode")


def sparse_decode_step(cfg: SparseCfg, kv: KV, n_layers: int, q_idx, q, block_scores, block_idx, out, lse=None,
                       n_sel=None, ws=None, stream=None, schedule: int = 0, check: bool = False) -> None:
    """Scoring, selection and attention of every layer of a batch;
    ``kv`` describes layer 0 of layer-major pools.  ``schedule``:
    STEP_AUTO, STEP_ONE_LAUNCH or STEP_PER_LAYER.  ``check=True`` (``ws`` a
    tensor) waits for the call on its stream and raises
    ``DecodeStepWaitError`` if a dependency wait of the one launch gave up
    (the workspace's error word; the results are then undefined)."""
    _check(_lib.uocr_sparse_decode_step(ctypes.byref(cfg), ctypes.byref(kv), int(n_layers), int(schedule),
                                        _ptr(q_idx), _ptr(q),
                                        _ptr(block_scores), _ptr(block_idx), _ptr(n_sel), _ptr(out), _ptr(lse),
                                        _ptr(ws), _nbytes(ws), _stream(stream)), "sparse_decode_step")
    if check:
        check_decode_step(ws, stream)


def sparse_decode_step_static(cfg: SparseCfg, kv: KV, n_layers: int, q_idx, q, block_scores, block_idx, out,
                              lse=None, n_sel=None, status=None, stream=None, schedule: int = 0) -> None:
    """``sparse_decode_step`` without a workspace (no allocation anywhere):
    the one launch keeps its counters in the library's static device array.
    ``status`` (int32 device tensor of one element, optional) gets 0, or 1
    if a dependency wait gave up.  Calls that overlap on one GPU race."""
    _check(_lib.uocr_sparse_decode_step_static(ctypes.byref(cfg), ctypes.byref(kv), int(n_layers), int(schedule),
                                               _ptr(q_idx), _ptr(q), _ptr(block_scores), _ptr(block_idx),
                                               _ptr(n_sel), _ptr(out), _ptr(lse), _ptr(status), _stream(stream)),
           "sparse_decode_step_static")


class DecodeStepWaitError(RuntimeError):
    """A dependency wait of the one-launch decode step gave up."""


def check_decode_step(ws, stream=None) -> None:
    """Wait for the work queued on ``stream`` and read the error word (the
    second 32-bit word) of a decode-step workspace tensor; raise
    ``DecodeStepWaitError`` when it is nonzero.  Each one-launch call clears
    it first, so it reports the last such call on this workspace."""
    import torch
    if not isinstance(ws, torch.Tensor):
        raise TypeError("check_decode_step reads the workspace: pass it as a tensor")
    if stream is None or isinstance(stream, int):
        torch.cuda.current_stream().synchronize() if stream is None else torch.cuda.synchronize()
    else:
        stream.synchronize()
    word = int(ws.view(torch.uint8)[4:8].cpu().view(torch.int32)[0])
    if word != 0:
        raise DecodeStepWaitError(f"a dependency wait of the one-launch decode step gave up (error word {word:#x}); "
                                  "its results are undefined")


def rope_cache_write(cfg: SparseCfg, kv: KV, n: int, seq, pos, tok_pos, page_pos, k_new, v_new, kidx_new,
                     stream=None) -> None:
    """Rotate (page2d) and store n new tokens' K, V, indexer K into kv's pools."""
    _check(_lib.uocr_rope_cache_write(ctypes.byref(cfg), ctypes.byref(kv), int(n), _ptr(seq), _ptr(pos), _ptr(tok_pos),
                                      _ptr(page_pos), _ptr(k_new), _ptr(v_new), _ptr(kidx_new), _stream(stream)),
           "rope_cache_write")


def rope_queries(cfg: SparseCfg, n: int, tok_pos, page_pos, q=None, q_idx=None, stream=None) -> None:
    """Rotate (page2d) n query tokens in place."""
    _check(_lib.uocr_rope_queries(ctypes.byref(cfg), int(n), _ptr(tok_pos), _ptr(page_pos), _ptr(q), _ptr(q_idx),
                                  _stream(stream)), "rope_queries")


def indexer_score_prefill(cfg: SparseCfg, kv: KV, q_idx, q_start: int, T: int, cand_ws, stream=None) -> None:
    _check(_lib.uocr_indexer_score_prefill(ctypes.byref(cfg), ctypes.byref(kv), _ptr(q_idx), q_start, T,
                                           _ptr(cand_ws), _nbytes(cand_ws), _stream(stream)),
           "indexer_score_prefill")


def block_topk_prefill(cfg: SparseCfg, cand_ws, q_start: int, T: int, max_blocks: int, block_idx, n_sel=None,
                       stream=None) -> None:
    _check(_lib.uocr_block_topk_prefill(ctypes.byref(cfg), _ptr(cand_ws), _nbytes(cand_ws), q_start, T, max_blocks,
                                        _ptr(block_idx), _ptr(n_sel), _stream(stream)), "block_topk_prefill")


def sparse_attn_prefill(cfg: SparseCfg, kv: KV, q, q_start: int, T: int, block_idx, out, lse=None, ws=None,
                        stream=None) -> None:
    _check(_lib.uocr_sparse_attn_prefill(ctypes.byref(cfg), ctypes.byref(kv), _ptr(q), q_start, T, _ptr(block_idx),
                                         _ptr(out), _ptr(lse), _ptr(ws), _nbytes(ws), _stream(stream)),
           "sparse_attn_prefill")


def page_coords(batch: int, n: int, tokens, marker: int, state, tok_pos, page_pos, stream=None) -> None:
    _check(_lib.uocr_page_coords(batch, n, _ptr(tokens), marker, _ptr(state), _ptr(tok_pos), _ptr(page_pos),
                                 _stream(stream)), "page_coords")


class BlockPool:
    """Host-side block pool of the paged caches (no GPU calls).

    Owns one ``uocr_pool``; ``table`` returns a sequence's block-table row
    and length, ready to upload as ``block_table`` / ``ctx_lens``.
    """

    def __init__(self, num_blocks: int, max_seqs: int = 1):
        self._h = _lib.uocr_pool_create(int(num_blocks), int(max_seqs))
        if not self._h:
            raise ValueError(f"uocr_pool_create: {last_error()}")

    def close(self) -> None:
        h, self._h = getattr(self, "_h", None), None
        if h:
            _lib.uocr_pool_destroy(h)

    def __del__(self):
        try:
            self.close()
        except Exception:  # interpreter shutdown: the library may already be gone
            pass

    def append(self, seq: int, n_tokens: int) -> None:
        _check(_lib.uocr_pool_append(self._h, int(seq), int(n_tokens)), "pool_append")

    def keep(self, seq: int, ranges) -> None:
        flat = (ctypes.c_int64 * (2 * len(ranges)))(*[int(v) for r in ranges for v in r])
        _check(_lib.uocr_pool_keep(self._h, int(seq), flat, len(ranges)), "pool_keep")

    def table(self, seq: int, max_blocks: int):
        row = (ctypes.c_int32 * max(int(max_blocks), 1))()
        length = ctypes.c_int64()
        _check(_lib.uocr_pool_table(self._h, int(seq), row, int(max_blocks), ctypes.byref(length)), "pool_table")
        return list(row)[:int(max_blocks)], int(length.value)

    @property
    def used(self) -> int:
        return int(_lib.uocr_pool_used(self._h))

    @property
    def peak(self) -> int:
        return int(_lib.uocr_pool_peak(self._h))

    def page_window_run(self, seq: int, image_tokens, text_tokens, window_pages: int, text_tail_tokens: int):
        """Run a document through the page-window schedule; returns the
        per-window peak block counts."""
        n = len(image_tokens)
        if len(text_tokens) != n:
            raise ValueError("image_tokens and text_tokens need one entry per page")
        img = (ctypes.c_int32 * max(n, 1))(*[int(v) for v in image_tokens])
        txt = (ctypes.c_int32 * max(n, 1))(*[int(v) for v in text_tokens])
        peaks = (ctypes.c_int64 * max(n, 1))()  # a document has at most one window per page
        n_windows = ctypes.c_int32(0)
        cfg = PageWindow(int(window_pages), int(text_tail_tokens))
        _check(_lib.uocr_page_window_run(ctypes.byref(cfg), img, txt, n, self._h, int(seq), peaks, n,
                                         ctypes.byref(n_windows)), "page_window_run")
        return [int(v) for v in peaks[:n_windows.value]]


def workspace_size(cfg: SparseCfg, op: int, rows: int, max_blocks: int) -> int:
    return int(_lib.uocr_workspace_size(ctypes.byref(cfg), op, rows, max_blocks))


def status_string(status: int) -> str:
    return _lib.uocr_status_string(status).decode()


def last_error() -> str:
    return _lib.uocr_last_error().decode(errors="replace")


def abi_version() -> int:
    return int(_lib.uocr_abi_version())
