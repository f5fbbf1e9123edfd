"""Host-side checks of the C ABI (no GPU): the library loads, exports every
function include/uocr_sparse.h declares, and rejects bad arguments on the
host before any HIP call."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "uocr_sparse.h")


def _ensure_built():
    lib = os.path.join(ROOT, "block_sparse_long_sr_amd", "libuocr_sparse.so")
    if not os.path.exists(lib):
        import importlib.util
        spec = importlib.util.spec_from_file_location("_uocr_build", os.path.join(ROOT, "block_sparse_long_sr_amd",
                                                                                   "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    return lib


@pytest.fixture(scope="module")
def U():
    _ensure_built()
    import block_sparse_long_sr_amd as U
    return U


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(uocr_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ["uocr_indexer_score_decode", "uocr_block_topk_decode", "uocr_sparse_attn_decode",
              "uocr_topk_attn_decode", "uocr_dense_attn_decode", "uocr_rope_cache_write", "uocr_rope_queries",
              "uocr_page_coords", "uocr_pool_create", "uocr_pool_destroy", "uocr_pool_append", "uocr_pool_keep",
              "uocr_pool_table", "uocr_pool_used", "uocr_pool_peak", "uocr_page_window_run",
              "uocr_indexer_score_prefill", "uocr_block_topk_prefill", "uocr_sparse_attn_prefill",
              "uocr_sparse_decode_step", "uocr_sparse_decode_step_static",
              "uocr_workspace_size", "uocr_status_string", "uocr_last_error", "uocr_abi_version"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(_ensure_built())
    for n in declared_functions():
        assert hasattr(lib, n), f"{n} not exported"


def test_struct_layouts_match_header(U, tmp_path):
    """The binding's ctypes mirrors have the sizes and field offsets that a C
    compiler gives the header's structs."""
    import subprocess
    mirrors = (("uocr_sparse_cfg", U.SparseCfg), ("uocr_kv", U.KV), ("uocr_page_window", U.PageWindow))
    fields = {st: [f for f, _ in cls._fields_] for st, cls in mirrors}
    lines = ["#include <stdio.h>", "#include <stddef.h>", '#include "uocr_sparse.h"', "int main(void) {"]
    for st, fs in fields.items():
        lines.append(f'  printf("{st} %zu\\n", sizeof({st}));')
        for f in fs:
            lines.append(f'  printf("{st}.{f} %zu\\n", offsetof({st}, {f}));')
    lines += ['  printf("abi %d\\n", UOCR_ABI_VERSION);', "  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = dict(l.split() for l in subprocess.run([str(exe)], check=True, capture_output=True,
                                                 text=True).stdout.splitlines())
    for st, cls in mirrors:
        assert int(got[st]) == ctypes.sizeof(cls)
        for f in fields[st]:
            assert int(got[f"{st}.{f}"]) == getattr(cls, f).offset, f
    assert int(got["abi"]) == U.abi_version() == 4


def test_status_strings(U):
    assert U.status_string(0) == "UOCR_OK"
    for c in range(1, 7):
        assert U.status_string(c).startswith("UOCR_E")
    assert U.status_string(6).startswith("UOCR_ECAPACITY")


FAKE = 0x10000  # a 16-byte aligned fake device address; never dereferenced


def _kv(U, batch=2, max_blocks=8, **kw):
    d = dict(k_pool=FAKE, v_pool=FAKE, kidx_pool=FAKE, block_table=FAKE, ctx_lens=FAKE,
             num_blocks=16, batch=batch, max_blocks=max_blocks)
    d.update(kw)
    return U.make_kv(d["k_pool"], d["v_pool"], d["kidx_pool"], d["block_table"], d["ctx_lens"],
                     d["num_blocks"], d["batch"], d["max_blocks"])


@pytest.mark.parametrize("field,value,code", [
    ("block_size", 16, 1), ("head_dim", 64, 1), ("index_dim", 64, 1), ("local_blocks", 0, 1),
    ("topk_blocks", 3, 1), ("topk_blocks", 5000, 1), ("num_heads", 0, 1), ("num_heads", 65, 1),
    ("sm_scale", 0.0, 1), ("sm_scale", float("nan"), 1), ("sm_scale", float("inf"), 1),
])
def test_bad_config_rejected(U, field, value, code):
    cfg = U.make_cfg()
    setattr(cfg, field, value)
    with pytest.raises(U.UocrError) as e:
        U.indexer_score_decode(cfg, _kv(U), FAKE, FAKE, stream=0)
    assert e.value.status == code
    assert field.split("_")[0] in U.last_error() or "must" in U.last_error()


def test_decode_argument_checks(U):
    cfg = U.make_cfg()
    with pytest.raises(U.UocrError) as e:
        U.indexer_score_decode(cfg, _kv(U), None, FAKE, stream=0)
    assert e.value.status == 1
    with pytest.raises(U.UocrError) as e:
        U.indexer_score_decode(cfg, _kv(U), FAKE + 8, FAKE, stream=0)   # misaligned bf16 pointer
    assert e.value.status == 1 and "aligned" in U.last_error()
    with pytest.raises(U.UocrError) as e:
        U.indexer_score_decode(cfg, _kv(U, max_blocks=0), FAKE, FAKE, stream=0)
    assert e.value.status == 2
    with pytest.raises(U.UocrError) as e:
        U.indexer_score_decode(cfg, _kv(U, batch=70000), FAKE, FAKE, stream=0)
    assert e.value.status == 2
    with pytest.raises(U.UocrError) as e:
        U.indexer_score_decode(cfg, _kv(U, num_blocks=0), FAKE, FAKE, stream=0)
    assert e.value.status == 2
    with pytest.raises(U.UocrError) as e:
        U.sparse_attn_decode(cfg, _kv(U, v_pool=None), FAKE, FAKE, FAKE, stream=0)
    assert e.value.status == 1 and "v_pool" in U.last_error()
    with pytest.raises(U.UocrError) as e:
        U.block_topk_decode(cfg, FAKE, FAKE, 2, 8, None, stream=0)
    assert e.value.status == 1 and "block_idx" in U.last_error()
    with pytest.raises(U.UocrError) as e:
        U.block_topk_decode(cfg, FAKE, FAKE, -1, 8, FAKE, stream=0)
    assert e.value.status == 2


def test_fused_decode_argument_checks(U):
    cfg = U.make_cfg(topk_blocks=257)
    with pytest.raises(U.UocrError) as e:
        U.topk_attn_decode(cfg, _kv(U), FAKE, FAKE, FAKE, FAKE, stream=0)
    assert e.value.status == 5 and "topk_blocks" in U.last_error()
    cfg = U.make_cfg()
    with pytest.raises(U.UocrError) as e:   # 16384 remote candidates at most
        U.topk_attn_decode(cfg, _kv(U, max_blocks=16384 + 5), FAKE, FAKE, FAKE, FAKE, stream=0)
    assert e.value.status == 5 and "max_blocks" in U.last_error()
    with pytest.raises(U.UocrError) as e:
        U.topk_attn_decode(cfg, _kv(U), FAKE, None, FAKE, FAKE, stream=0)
    assert e.value.status == 1 and "block_scores" in U.last_error()
    with pytest.raises(U.UocrError) as e:
        U.topk_attn_decode(cfg, _kv(U), FAKE, FAKE, FAKE, None, stream=0)
    assert e.value.status == 1 and "out" in U.last_error()
    assert U.workspace_size(cfg, 2, 16, 4096) == 0


def test_decode_step_argument_checks(U):
    cfg = U.make_cfg()
    need = U.workspace_size(cfg, U.OP_DECODE_STEP, 12 * 2, 8)
    assert need == -(-((2 + 3 * 24) * 4) // 256) * 256  # ticket, error word, three counters per slot
    ws = (0x100000, need)  # 256-byte aligned fake address; never dereferenced

    def call(kv=None, n_layers=12, ws=ws, c=cfg, q_idx=FAKE, schedule=0):
        U.sparse_decode_step(c, kv or _kv(U), n_layers, q_idx, FAKE, FAKE, FAKE, FAKE, ws=ws, stream=0,
                             schedule=schedule)

    for kwargs, code, text in (
            (dict(ws=None), 3, "ws"), (dict(ws=(0x100000, need - 1)), 3, "ws"),
            (dict(ws=(0x100000 + 16, need)), 1, "256"), (dict(n_layers=-1), 2, "n_layers"),
            (dict(q_idx=None), 1, "q_idx"), (dict(kv=_kv(U, kidx_pool=None)), 1, "kidx_pool"),
            (dict(schedule=3), 1, "schedule"), (dict(schedule=-1), 1, "schedule")):
        with pytest.raises(U.UocrError) as e:
            call(**kwargs)
        assert e.value.status == code and text in U.last_error(), (kwargs, U.last_error())
    big = U.make_cfg(topk_blocks=300, local_blocks=4)
    with pytest.raises(U.UocrError) as e:
        call(c=big)
    assert e.value.status == 5
    with pytest.raises(U.UocrError) as e:
        call(kv=_kv(U, max_blocks=20000))
    assert e.value.status == 5
    call(n_layers=0)                    # nothing to do: no launch, no error
    call(kv=_kv(U, batch=0), ws=None)


def test_decode_step_static_argument_checks(U):
    """The no-workspace decode step: the same checks as the workspace entry
    point, and the one launch's limit of its static counters (21844
    layer-sequence slots, i.e. 2 + 3 * 21844 <= 65536 words), all refused on
    the host before any HIP call."""
    cfg = U.make_cfg()

    def call(kv=None, n_layers=12, schedule=U.STEP_ONE_LAUNCH, status=None, q=FAKE):
        U.sparse_decode_step_static(cfg, kv or _kv(U), n_layers, FAKE, q, FAKE, FAKE, FAKE, status=status, stream=0,
                                    schedule=schedule)

    for kwargs, code, text in ((dict(n_layers=-1), 2, "n_layers"), (dict(q=None), 1, "q"),
                               (dict(status=FAKE + 2), 1, "status"), (dict(schedule=7), 1, "schedule")):
        with pytest.raises(U.UocrError) as e:
            call(**kwargs)
        assert e.value.status == code and text in U.last_error(), (kwargs, U.last_error())
    with pytest.raises(U.UocrError) as e:
        call(kv=_kv(U, batch=1), n_layers=21845)
    assert e.value.status == 5 and "21844" in U.last_error()
    with pytest.raises(U.UocrError) as e:   # the automatic choice takes the one launch here
        call(kv=_kv(U, batch=4, max_blocks=14336), n_layers=5462, schedule=U.STEP_AUTO)
    assert e.value.status == 5 and "21844" in U.last_error()
    call(n_layers=0)
    call(kv=_kv(U, batch=0))


def test_dense_decode_argument_checks(U):
    cfg = U.make_cfg()
    need = U.workspace_size(cfg, U.OP_DENSE_ATTN_DECODE, 16, 4096)
    assert need > 0 and need % (130 * 4) == 0 and need // (130 * 4) % (16 * 10) == 0
    with pytest.raises(U.UocrError) as e:
        U.dense_attn_decode(cfg, _kv(U), FAKE, FAKE, stream=0)        # no workspace
    assert e.value.status == 3
    small = U.workspace_size(cfg, U.OP_DENSE_ATTN_DECODE, 2, 8)
    with pytest.raises(U.UocrError) as e:
        U.dense_attn_decode(cfg, _kv(U), FAKE, FAKE, ws=(FAKE, small - 4), stream=0)
    assert e.value.status == 3
    with pytest.raises(U.UocrError) as e:
        U.dense_attn_decode(cfg, _kv(U, v_pool=None), FAKE, FAKE, ws=(FAKE, small), stream=0)
    assert e.value.status == 1 and "v_pool" in U.last_error()
    U.dense_attn_decode(cfg, _kv(U, batch=0), None, None, stream=0)   # empty batch: nothing to do


def test_rope_argument_checks(U):
    cfg = U.make_cfg()
    with pytest.raises(U.UocrError) as e:
        U.rope_cache_write(cfg, _kv(U), 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 8, FAKE, stream=0)
    assert e.value.status == 1 and "v_new" in U.last_error()
    with pytest.raises(U.UocrError) as e:
        U.rope_cache_write(cfg, _kv(U, kidx_pool=None), 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, stream=0)
    assert e.value.status == 1 and "kidx_pool" in U.last_error()
    with pytest.raises(U.UocrError) as e:
        U.rope_cache_write(cfg, _kv(U), -1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, stream=0)
    assert e.value.status == 2
    with pytest.raises(U.UocrError) as e:
        U.rope_queries(cfg, 3, None, FAKE, q=FAKE, stream=0)
    assert e.value.status == 1 and "tok_pos" in U.last_error()
    U.rope_queries(cfg, 3, None, None, stream=0)                     # nothing to rotate
    U.rope_cache_write(cfg, _kv(U), 0, None, None, None, None, None, None, None, stream=0)


def test_page_coords_argument_checks(U):
    with pytest.raises(U.UocrError) as e:
        U.page_coords(2, -1, FAKE, 7, FAKE, FAKE, FAKE, stream=0)
    assert e.value.status == 2
    with pytest.raises(U.UocrError) as e:
        U.page_coords(2, 5, FAKE, 7, None, FAKE, FAKE, stream=0)
    assert e.value.status == 1 and "state" in U.last_error()
    with pytest.raises(U.UocrError) as e:
        U.page_coords(2, 5, FAKE, 7, FAKE, FAKE + 2, FAKE, stream=0)   # misaligned int32 array
    assert e.value.status == 1 and "tok_pos" in U.last_error()
    U.page_coords(0, 5, None, 7, None, None, None, stream=0)          # empty: no-op
    U.page_coords(3, 0, None, 7, None, None, None, stream=0)


def test_page_tags_need_query_pages(U):
    cfg = U.make_cfg()
    kv = _kv(U)
    kv.block_page = FAKE
    with pytest.raises(U.UocrError) as e:      # tags without query pages
        U.topk_attn_decode(cfg, kv, FAKE, FAKE, FAKE, FAKE, stream=0)
    assert e.value.status == 1 and "query_page" in U.last_error()
    kv.query_page = FAKE + 2                    # misaligned int32 array
    with pytest.raises(U.UocrError) as e:
        U.topk_attn_decode(cfg, kv, FAKE, FAKE, FAKE, FAKE, stream=0)
    assert e.value.status == 1 and "query_page" in U.last_error()
    kv1 = _kv(U, batch=1, max_blocks=64)
    kv1.block_page = FAKE + 1
    kv1.query_page = FAKE
    ws = U.workspace_size(cfg, U.OP_INDEXER_PREFILL, 100, 64)
    with pytest.raises(U.UocrError) as e:
        U.indexer_score_prefill(cfg, kv1, FAKE, 1900, 100, (FAKE, ws), stream=0)
    assert e.value.status == 1 and "block_page" in U.last_error()


def test_page_tiered_prefill_context_limit(U):
    """With page tags a prefill ranking key spends one bit on the tier; up to
    16384 blocks the in-split ids take at most 8 bits, so scores still rank
    to 2^-14 relative (inside the 1e-4 band).  Longer tiered contexts (9-bit
    ids) are rejected; plain ranking still takes them."""
    cfg = U.make_cfg()
    for M, status in ((16385, 5), (32768, 5)):
        kv = _kv(U, batch=1, max_blocks=M)
        kv.block_page, kv.query_page = FAKE, FAKE
        with pytest.raises(U.UocrError) as e:
            U.indexer_score_prefill(cfg, kv, FAKE, 0, 100, (FAKE, 1 << 30), stream=0)
        assert e.value.status == status and "16384" in U.last_error()
    # 16384 blocks with tags passes every check (the launch itself is not
    # reached here: a bad workspace size stops it first)
    kv = _kv(U, batch=1, max_blocks=16384)
    kv.block_page, kv.query_page = FAKE, FAKE
    with pytest.raises(U.UocrError) as e:
        U.indexer_score_prefill(cfg, kv, FAKE, 0, 100, (FAKE, 16), stream=0)
    assert e.value.status == 3


def test_empty_batch_is_a_no_op(U):
    cfg = U.make_cfg()
    # batch 0: nothing to do, nothing launched, success without touching HIP
    U.indexer_score_decode(cfg, _kv(U, batch=0), None, None, stream=0)
    U.block_topk_decode(cfg, None, None, 0, 8, None, stream=0)
    U.sparse_attn_decode(cfg, _kv(U, batch=0), None, None, None, stream=0)
    U.topk_attn_decode(cfg, _kv(U, batch=0), None, None, None, None, stream=0)


def test_prefill_argument_checks(U):
    cfg = U.make_cfg()
    kv1 = _kv(U, batch=1, max_blocks=64)
    need = U.workspace_size(cfg, U.OP_INDEXER_PREFILL, 100, 64)
    assert need > 0
    assert need == U.workspace_size(cfg, U.OP_TOPK_PREFILL, 100, 64)
    attn_need = U.workspace_size(cfg, U.OP_ATTN_PREFILL, 100, 64)
    # block-major prefill attention: one fp32 partial (o[128], m, l + pad) per (row, head, slot) and the buckets
    assert attn_need >= 100 * 10 * 16 * (512 + 8) + 100 * 16 * 4
    assert U.workspace_size(cfg, U.OP_ATTN_PREFILL, 200, 64) > attn_need
    assert U.workspace_size(cfg, U.OP_ATTN_PREFILL, 100, 16385) == 0   # bucket counts must fit in LDS
    assert U.workspace_size(cfg, U.OP_ATTN_DECODE, 16, 4096) == 0
    with pytest.raises(U.UocrError) as e:
        U.indexer_score_prefill(cfg, _kv(U, batch=2, max_blocks=64), FAKE, 0, 100, (FAKE, need), stream=0)
    assert e.value.status == 2
    with pytest.raises(U.UocrError) as e:
        U.indexer_score_prefill(cfg, kv1, FAKE, 2000, 100, (FAKE, need), stream=0)   # 2100 > 64*32
    assert e.value.status == 2
    with pytest.raises(U.UocrError) as e:
        U.indexer_score_prefill(cfg, kv1, FAKE, -1, 100, (FAKE, need), stream=0)
    assert e.value.status == 2
    with pytest.raises(U.UocrError) as e:
        U.indexer_score_prefill(cfg, kv1, FAKE, 0, 100, (FAKE, need - 1), stream=0)
    assert e.value.status == 3
    with pytest.raises(U.UocrError) as e:
        U.indexer_score_prefill(cfg, kv1, FAKE, 0, 100, None, stream=0)
    assert e.value.status == 3
    with pytest.raises(U.UocrError) as e:
        U.block_topk_prefill(cfg, (FAKE, need - 1), 0, 100, 64, FAKE, stream=0)
    assert e.value.status == 3
    # the scoring's limit: 64 splits of at most 512 blocks
    assert U.workspace_size(cfg, U.OP_INDEXER_PREFILL, 100, 32768) > 0
    assert U.workspace_size(cfg, U.OP_INDEXER_PREFILL, 100, 32769) == 0
    with pytest.raises(U.UocrError) as e:
        U.indexer_score_prefill(cfg, _kv(U, batch=1, max_blocks=32769), FAKE, 0, 100, (FAKE, 1 << 30), stream=0)
    assert e.value.status == 5
    big = U.make_cfg(topk_blocks=40)
    with pytest.raises(U.UocrError) as e:
        U.indexer_score_prefill(big, kv1, FAKE, 0, 100, (FAKE, 1 << 30), stream=0)
    assert e.value.status == 5
    with pytest.raises(U.UocrError) as e:
        U.sparse_attn_prefill(cfg, kv1, FAKE, 2000, 100, FAKE, FAKE, stream=0)
    assert e.value.status == 2
    with pytest.raises(U.UocrError) as e:   # block-major attention workspace too small
        U.sparse_attn_prefill(cfg, kv1, FAKE, 0, 100, FAKE, FAKE, ws=(FAKE, attn_need - 1), stream=0)
    assert e.value.status == 3
    with pytest.raises(U.UocrError) as e:   # ... or not 256-byte aligned
        U.sparse_attn_prefill(cfg, kv1, FAKE, 0, 100, FAKE, FAKE, ws=(FAKE + 16, attn_need), stream=0)
    assert e.value.status == 1
    # T == 0 is a successful no-op
    U.indexer_score_prefill(cfg, kv1, None, 0, 0, None, stream=0)
    U.block_topk_prefill(cfg, None, 0, 0, 64, None, stream=0)
    U.sparse_attn_prefill(cfg, kv1, None, 0, 0, None, None, stream=0)


def test_last_error_is_cleared_by_success(U):
    cfg = U.make_cfg()
    with pytest.raises(U.UocrError):
        U.block_topk_decode(cfg, FAKE, FAKE, -1, 8, FAKE, stream=0)
    assert U.last_error() != ""
    U.block_topk_decode(cfg, None, None, 0, 8, None, stream=0)
    assert U.last_error() == ""


def test_binding_rejects_non_contiguous_tensors(U):
    import torch
    cfg = U.make_cfg()
    scores = torch.zeros(8, 4).t()          # a transposed view: not row-major
    assert not scores.is_contiguous()
    with pytest.raises(ValueError):
        U.block_topk_decode(cfg, scores, FAKE, 4, 8, FAKE, stream=0)
