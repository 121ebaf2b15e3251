"""Build libcsa.so (the C ABI of include/csa.h) for gfx950 with hipcc.

Every source is compiled to an object under _build/ (in parallel) and the
objects are linked into long_context_sparse_16_amd/libcsa.so.  Run as a
script (``python long_context_sparse_16_amd/build.py``) or through
``__graft_entry__.build()``; it imports nothing from the package, whose
import needs the library built here.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libcsa.so")

SOURCES = ["api.cpp", "compress.hip", "indexer.hip", "topk.hip", "attend.hip", "attend_bwd.hip",
           "scratch.hip"]
# Per-source additions.  The indexer's epilogue is pure VALU work next to
# the MFMAs: with IEEE mode off (its inputs never hold NaN) a ReLU is one
# v_max_f32 instead of a canonicalize plus max, and the VGPR form of MFMA
# keeps the accumulators out of AGPRs, saving one copy per value.
SOURCE_FLAGS = {
    "indexer.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    # the top-k kernels' per-thread atomics on one LDS counter (list slots):
    # the wave's values are summed with a DPP scan and one lane issues the
    # atomic, instead of a scalar loop over the active lanes
    "topk.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=DPP"],
}
HEADERS = ["common.h", "kernels.h", "select.h"]
PUBLIC_HEADER = os.path.join(ROOT, "include", "csa.h")
DIGEST_TAG = b"csa-source-digest:"

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # keep hipcc from forming packed fp32 instructions (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}",
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def source_digest() -> str:
    """sha256 over every source, header and compile flag the library is
    built from (embedded in the library, so a stale build is detectable)."""
    import hashlib
    h = hashlib.sha256()
    for f in [*SOURCES, *HEADERS]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    with open(PUBLIC_HEADER, "rb") as fh:
        h.update(fh.read())
    h.update(repr((FLAGS[:-1], SOURCE_FLAGS)).encode())
    return h.hexdigest()


def library_digest(path: str = LIB):
    """The source digest embedded in a built library (read from the file,
    without loading it), or None."""
    try:
        with open(path, "rb") as fh:
            data = fh.read()
    except OSError:
        return None
    i = data.find(DIGEST_TAG)
    if i < 0:
        return None
    return data[i + len(DIGEST_TAG):i + len(DIGEST_TAG) + 64].decode("ascii", "replace")


def ensure_current(verbose: bool = True) -> str:
    """Build the library when it is missing or was built from other sources
    than the ones in the tree."""
    want = source_digest()
    have = library_digest()
    if have != want:
        if verbose:
            print(f"libcsa.so {'missing' if have is None else 'stale'}: building", file=sys.stderr)
        build(verbose=verbose)
        if library_digest() != want:
            raise RuntimeError("libcsa.so does not carry the digest of its sources after a build")
    return LIB


def _compile(src: str, digest: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    extra = [f'-DCSA_SOURCE_DIGEST="{digest}"'] if src == "api.cpp" else []
    cmd = [hipcc(), *FLAGS, *SOURCE_FLAGS.get(src, []), *extra, *lang, "-c",
           os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = min(len(SOURCES), max(1, (os.cpu_count() or 2)))
    digest = source_digest()
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda src: _compile(src, digest), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
