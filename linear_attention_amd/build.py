"""Build the HIP library ``liblightning.so`` in place (gfx950 only).

Usage: ``python -m linear_attention_amd.build``. ``__graft_entry__.build()``
calls :func:`build` as well.
"""

from __future__ import annotations

import hashlib
import os
import re
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "liblightning.so")

SOURCES = ["prefill_heads.hip", "prefill_slices.hip", "decode.hip", "backward.hip", "softmax.hip",
           "noalloc.hip", "lightning_api.cpp"]

HIPCC_FLAGS = [
    "-O3", "--offload-arch=gfx950", "-std=c++17", "-fPIC",
    "-fvisibility=hidden",
    # no packed fp32 VALU ops (v_pk_*_f32) anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


# Per-source additions. The softmax kernels rescale their MFMA accumulators with
# VALU work every key block; in VGPR form the accumulators need no copies
# between register files for that (204 instead of 284 registers per lane for
# the prefill kernel, two waves per SIMD instead of one).
EXTRA_FLAGS = {"softmax.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def source_hash() -> str:
    """sha256 (first 16 hex digits) over every file of csrc/ and include/ (names
    and contents, sorted by name) and the compile flags: the build identity the
    library reports through lt_build_id()."""
    h = hashlib.sha256()
    for d in (CSRC, INCLUDE):
        for name in sorted(os.listdir(d)):
            path = os.path.join(d, name)
            if os.path.isfile(path):
                h.update(os.path.relpath(path, ROOT).encode() + b"\0")
                with open(path, "rb") as f:
                    h.update(f.read())
    h.update(repr((HIPCC_FLAGS[:-4], sorted(EXTRA_FLAGS.items()))).encode())
    return h.hexdigest()[:16]


def built_id(path: str = LIB):
    """The build identity a built library carries, or None when it has none
    (missing file or no tag). Read from the file's bytes: loading the library
    here would keep this version mapped in the process even after a rebuild
    replaces the file."""
    if not os.path.exists(path):
        return None
    with open(path, "rb") as f:
        m = re.search(rb"LT_BUILD_ID=([0-9a-f]{16}|unknown)\0", f.read())
    return m.group(1).decode() if m else None


def library_is_current() -> bool:
    """True when liblightning.so exists and was built from the current sources."""
    return built_id() == source_hash()


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def _run(cmd, verbose, what):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed building {what}")


def build(verbose: bool = False) -> str:
    """Compile every HIP source (one object each, in parallel) and link
    liblightning.so (atomically replaced)."""
    tmp = LIB + ".tmp%d" % os.getpid()
    with tempfile.TemporaryDirectory(prefix="lt_build_") as work:
        objs = [os.path.join(work, s + ".o") for s in SOURCES]

        build_id = ["-DLT_BUILD_ID=\"%s\"" % source_hash()]

        def compile_one(i):
            src = SOURCES[i]
            _run([hipcc()] + HIPCC_FLAGS + EXTRA_FLAGS.get(src, []) + build_id +
                 ["-c", os.path.join(CSRC, src), "-o", objs[i]], verbose, src)

        with ThreadPoolExecutor(max_workers=min(len(SOURCES), 7)) as ex:
            list(ex.map(compile_one, range(len(SOURCES))))
        _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp], verbose,
             "liblightning.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
