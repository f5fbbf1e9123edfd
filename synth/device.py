"""Device-resident copies of the seeded workloads (bf16 bits in int16 tensors).

Two routes write the same bits: ``from_host`` copies the host-generated pools
(small cases), ``generate`` runs the fill kernels of ``synth/fill.hip`` on the
GPU (the 135 GB decode case cannot be generated on the host in reasonable
time).  Pool slots past a sequence's length hold the bf16 NaN pattern in both
routes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import List, Optional

import numpy as np

from . import workloads as W

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libuocr_synth.so")
NAN_BF16 = 0x7FC0
_lib = None


def build() -> str:
    """Compile libuocr_synth.so (gfx950) in place."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           os.path.join(_HERE, "fill.hip"), "-o", tmp]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"synth build failed:\n{r.stdout}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: run synth.device.build()")
        lib = ctypes.CDLL(LIB_PATH)
        P, I32, I64, U64, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_float
        lib.synth_fill_kv.argtypes = [P, P, I32, I32, I32, U64, I32, P]
        lib.synth_fill_kidx.argtypes = [P, P, I32, I32, U64, I32, P]
        lib.synth_fill_dense.argtypes = [P, I64, U64, I32, P]
        lib.synth_add_direction.argtypes = [P, P, P, I32, P, F, I32, P]
        for f in (lib.synth_fill_kv, lib.synth_fill_kidx, lib.synth_fill_dense, lib.synth_add_direction):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _mode(wl: W.Workload) -> int:
    return 0 if wl.values == "normal" else 1


@dataclass
class DeviceWorkload:
    """GPU tensors of a workload; pools are indexed [layer][block]..."""
    wl: W.Workload
    layers: List[int]
    k: "object"          # int16 [nl, P, H, 32, D]
    v: "object"
    kidx: "object"       # int16 [nl, P, 32, Di]
    block_table: "object"  # int32 [B, max_blocks]
    ctx_lens: "object"   # int32 [B]
    q: "object"          # decode: [nl, B, H, D]; prefill: [T, H, D]
    q_idx: "object"      # decode: [nl, B, Di]; prefill: [T, Di]

    def kv(self, li: int):
        """uocr KV descriptor of the li-th resident layer."""
        import block_sparse_long_sr_amd as U
        return U.make_kv(self.k[li], self.v[li], self.kidx[li], self.block_table, self.ctx_lens,
                         self.wl.pool_blocks, self.wl.batch, self.wl.max_blocks)

    # ---- host copies of the device inputs, in logical order ---------------
    # The oracle side of a full-size parity check takes its inputs from here:
    # the very bits the kernels read, gathered through the block table and
    # copied to the host (the 135 GB workloads are not regenerated on the
    # host).  Only generated inputs are read, never a kernel's output.

    def host_kidx(self, li: int, seq: int, n_tokens: int) -> np.ndarray:
        """Indexer keys of tokens [0, n_tokens) of sequence ``seq`` in resident
        layer ``li``: [n_tokens, Di] uint16."""
        nb = -(-int(n_tokens) // W.BLOCK)
        if nb == 0:
            return np.zeros((0, self.wl.index_dim), np.uint16)
        blocks = self.block_table[seq, :nb].long()
        rows = self.kidx[li].index_select(0, blocks).reshape(nb * W.BLOCK, -1)[:n_tokens]
        return rows.cpu().numpy().view(np.uint16)

    def host_kv_fetch(self, li: int, seq: int):
        """``fetch(tokens) -> (K, V)``, each [H, len(tokens), D] uint16: the main
        keys and values of the given token positions of ``seq`` in layer ``li``."""
        import torch

        tab = self.block_table
        dev = tab.device

        def fetch(toks):
            toks = np.asarray(toks, np.int64)
            t = torch.from_numpy(toks).to(dev)
            pb = tab[seq, t // W.BLOCK].long()
            off = t % W.BLOCK
            n = torch.arange(toks.size, device=dev)
            k = self.k[li].index_select(0, pb)[n, :, off, :]
            v = self.v[li].index_select(0, pb)[n, :, off, :]
            return (k.transpose(0, 1).contiguous().cpu().numpy().view(np.uint16),
                    v.transpose(0, 1).contiguous().cpu().numpy().view(np.uint16))

        return fetch

    def host_decode_queries(self, li: int, seq: int):
        """(q [H, D], q_idx [Di]) uint16 of a decode query."""
        return (self.q[li, seq].cpu().numpy().view(np.uint16), self.q_idx[li, seq].cpu().numpy().view(np.uint16))

    def host_prefill_queries(self):
        """(q [T, H, D], q_idx [T, Di]) uint16 of a prefill chunk."""
        return self.q.cpu().numpy().view(np.uint16), self.q_idx.cpu().numpy().view(np.uint16)


def _alloc(wl: W.Workload, layers: List[int], device):
    import torch
    P, H, D, Di, nl = wl.pool_blocks, wl.heads, wl.head_dim, wl.index_dim, len(layers)
    k = torch.empty((nl, P, H, 32, D), dtype=torch.int16, device=device)
    v = torch.empty((nl, P, H, 32, D), dtype=torch.int16, device=device)
    kidx = torch.empty((nl, P, 32, Di), dtype=torch.int16, device=device)
    return k, v, kidx


def _bits(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16))


def from_host(wl: W.Workload, layers: Optional[List[int]] = None, device="cuda") -> DeviceWorkload:
    """Copy host-generated tensors to the GPU (small workloads)."""
    import torch
    layers = list(range(wl.layers)) if layers is None else layers
    k, v, kidx = _alloc(wl, layers, device)
    for li, l in enumerate(layers):
        kp, vp, ip = wl.host_pools(l)
        k[li].copy_(_bits(kp))
        v[li].copy_(_bits(vp))
        kidx[li].copy_(_bits(ip))
    tab = torch.from_numpy(wl.block_table()).to(device)
    ctx = torch.from_numpy(wl.ctx_lens.astype(np.int32)).to(device)
    q, qi = _host_queries(wl, layers)
    return DeviceWorkload(wl, layers, k, v, kidx, tab, ctx, _bits(q).to(device), _bits(qi).to(device))


def _host_queries(wl: W.Workload, layers):
    if wl.mode == "prefill":
        rows = np.arange(wl.rows)
        return wl.q_rows(rows), wl.q_idx_rows(rows)
    q = np.stack([np.stack([wl.q(l, b) for b in range(wl.batch)]) for l in layers])
    qi = np.stack([np.stack([wl.q_idx(l, b) for b in range(wl.batch)]) for l in layers])
    return q, qi


def generate(wl: W.Workload, layers: Optional[List[int]] = None, device="cuda") -> DeviceWorkload:
    """Generate the workload on the GPU with the fill kernels."""
    import torch
    lib = _load()
    layers = list(range(wl.layers)) if layers is None else layers
    k, v, kidx = _alloc(wl, layers, device)
    for t in (k, v, kidx):
        t.fill_(NAN_BF16)
    tab = torch.from_numpy(wl.block_table()).to(device)
    ctx = torch.from_numpy(wl.ctx_lens.astype(np.int32)).to(device)
    stream = torch.cuda.current_stream().cuda_stream
    mode = _mode(wl)
    H, D, Di, B = wl.heads, wl.head_dim, wl.index_dim, wl.batch
    if wl.mode == "prefill":
        q = torch.empty((wl.rows, H, D), dtype=torch.int16, device=device)
        qi = torch.empty((wl.rows, Di), dtype=torch.int16, device=device)
        _ok(lib.synth_fill_dense(q.data_ptr(), q.numel(), wl.key(W.ROLE_Q, layers[0], 0), mode, stream))
        _ok(lib.synth_fill_dense(qi.data_ptr(), qi.numel(), wl.key(W.ROLE_QIDX, layers[0], 0), mode, stream))
    else:
        q = torch.empty((len(layers), B, H, D), dtype=torch.int16, device=device)
        qi = torch.empty((len(layers), B, Di), dtype=torch.int16, device=device)
    row_bytes = wl.max_blocks * 4
    for li, l in enumerate(layers):
        for b in range(B):
            L = int(wl.ctx_lens[b])
            trow = tab.data_ptr() + b * row_bytes
            _ok(lib.synth_fill_kv(k[li].data_ptr(), trow, L, H, D, wl.key(W.ROLE_K, l, b), mode, stream))
            _ok(lib.synth_fill_kv(v[li].data_ptr(), trow, L, H, D, wl.key(W.ROLE_V, l, b), mode, stream))
            _ok(lib.synth_fill_kidx(kidx[li].data_ptr(), trow, L, Di, wl.key(W.ROLE_KIDX, l, b), mode, stream))
            if wl.mode == "decode":
                _ok(lib.synth_fill_dense(q[li, b].data_ptr(), H * D, wl.key(W.ROLE_Q, l, b), mode, stream))
                _ok(lib.synth_fill_dense(qi[li, b].data_ptr(), Di, wl.key(W.ROLE_QIDX, l, b), mode, stream))
        for e in wl.edits:
            if e.layer != l:
                continue
            toks = torch.from_numpy(e.tokens.astype(np.int64)).to(device)
            if wl.mode == "decode":
                qrow = qi[li, e.seq]
            else:
                qrow = qi[wl.rows - 1]
            _ok(lib.synth_add_direction(kidx[li].data_ptr(), tab.data_ptr() + e.seq * row_bytes, toks.data_ptr(),
                                        int(toks.numel()), qrow.data_ptr(), float(e.coef), Di, stream))
            torch.cuda.current_stream().synchronize()  # toks must outlive the launch
    return DeviceWorkload(wl, layers, k, v, kidx, tab, ctx, q, qi)


def _ok(rc: int):
    if rc != 0:
        raise RuntimeError(f"synth fill launch failed with hipError {rc}")
