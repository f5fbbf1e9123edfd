"""Build libuocr_sparse.so (gfx950) in-tree with hipcc.

Usage: ``python block_sparse_long_sr_amd/build.py`` (a script: the package
itself refuses to import until the library exists) or ``build()``;
``build.py --host-sanitize DIR`` builds a host-side ASan/UBSan copy into DIR.  Every call
recompiles every source; the objects go to ``_build/`` and the shared library
next to this file, where the binding loads it.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_NAME = "libuocr_sparse.so"
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed fp32 VALU forms are kept out of generated code (-packed-fp32-ops);
# the host pass reports the feature as unknown, which is harmless.
DEVICE_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC"]

SOURCES = ["api.cpp", "indexer_decode.hip", "topk_decode.hip", "attn.hip", "indexer_prefill.hip", "dense_attn.hip", "rope.hip", "attn_prefill.hip", "decode_step.hip", "pool.cpp"]
# Extra hipcc flags per source file (none at present).
PER_FILE_FLAGS = {}


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def compile_objects(sources, src_dir, obj_dir, extra=()):
    os.makedirs(obj_dir, exist_ok=True)
    jobs = []
    for s in sources:
        src = os.path.join(src_dir, s)
        obj = os.path.join(obj_dir, os.path.splitext(s)[0] + ".o")
        if s.endswith(".hip"):
            cmd = [HIPCC, *DEVICE_FLAGS, *PER_FILE_FLAGS.get(s, []), *extra, "-c", src, "-o", obj]
        else:
            cmd = [HIPCC, *HOST_FLAGS, *extra, "-c", src, "-o", obj]
        jobs.append((cmd, obj))
    workers = min(len(jobs), max(1, min(8, (os.cpu_count() or 2))))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        outs = list(ex.map(lambda j: _run(j[0]), jobs))
    return [o for _, o in jobs], outs


# Host-side AddressSanitizer + UBSan for the library's host code (argument
# validation, planning, the block pool); device code is built as usual.
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def link(objs, out_path, extra=()):
    tmp = out_path + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra, *objs, "-o", tmp])
    os.replace(tmp, out_path)


def build_host_sanitized(out_dir: str) -> str:
    """Build a host-sanitized copy of the library and binding into
    out_dir/block_sparse_long_sr_amd/ (run Python with LD_PRELOAD of the
    clang ASan runtime and that directory first on sys.path)."""
    import shutil
    pkg = os.path.join(out_dir, "block_sparse_long_sr_amd")
    os.makedirs(pkg, exist_ok=True)
    shutil.copy(os.path.join(PKG, "__init__.py"), pkg)
    objs, _ = compile_objects(SOURCES, CSRC, os.path.join(ROOT, "_build", "uocr_sparse_hostsan"), extra=HOST_SANITIZE)
    lib = os.path.join(pkg, LIB_NAME)
    link(objs, lib, extra=["-fsanitize=address", "-fsanitize=undefined"])
    return lib


def build(verbose: bool = False) -> str:
    objs, outs = compile_objects(SOURCES, CSRC, os.path.join(ROOT, "_build", "uocr_sparse"))
    lib = os.path.join(PKG, LIB_NAME)
    link(objs, lib)
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    if "--host-sanitize" in sys.argv:
        print("built", build_host_sanitized(sys.argv[sys.argv.index("--host-sanitize") + 1]))
    else:
        build(verbose="-q" not in sys.argv)
