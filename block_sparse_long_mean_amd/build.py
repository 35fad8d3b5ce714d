"""Build libbsa.so in-tree with hipcc for gfx950.

    python -m block_sparse_long_mean_amd.build

Each HIP source compiles to an object under _build/ (in parallel), then the
objects link into block_sparse_long_mean_amd/libbsa.so.  The library carries
a digest of the sources it was built from (bsa_build_digest()); the binding
refuses to load a library whose digest differs from the tree's.
"""
from __future__ import annotations

import concurrent.futures as cf
import hashlib
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
INCLUDE = os.path.join(os.path.dirname(PKG), "include")
LIB = os.path.join(PKG, "libbsa.so")
SOURCES = ["api.hip", "summary.hip", "gate.hip", "csr.hip", "attn.hip", "decode.hip"]
ARCH = os.environ.get("BSA_OFFLOAD_ARCH", "gfx950")
HEADER = os.path.join(INCLUDE, "bsa.h")


def source_digest() -> str:
    """sha256 (first 16 hex digits) over the library's sources: every file of
    csrc/ (sorted by name) and include/bsa.h, names and contents."""
    h = hashlib.sha256()
    files = sorted(os.listdir(CSRC))
    for name in files:
        path = os.path.join(CSRC, name)
        if not os.path.isfile(path):
            continue
        h.update(name.encode() + b"\0")
        with open(path, "rb") as f:
            h.update(f.read())
    h.update(b"bsa.h\0")
    with open(HEADER, "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


def is_current() -> bool:
    """Whether the built library holds the tree's source digest (read from the
    file, without loading it: a process that has loaded a library cannot load
    a rebuilt one from the same path)."""
    if not os.path.exists(LIB):
        return False
    with open(LIB, "rb") as f:
        return source_digest().encode() + b"\0" in f.read()


HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "-O3",
    "-std=c++17",
    f"--offload-arch={ARCH}",
    "-fPIC",
    "-fvisibility=hidden",
    # packed fp32 VALU ops stay off (device code only; the host pass warns)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def _filter(text: str) -> str:
    keep = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln]
    return "\n".join(keep)


def _compile(src: str, digest: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, f'-DBSA_BUILD_DIGEST="{digest}"', "-I" + INCLUDE, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{_filter(r.stdout + r.stderr)}")
    msg = _filter(r.stdout + r.stderr).strip()
    if msg:
        print(msg, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    digest = source_digest()
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda src: _compile(src, digest), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{_filter(r.stdout + r.stderr)}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} (sources {digest})")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
