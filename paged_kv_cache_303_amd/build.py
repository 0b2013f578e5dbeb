"""Build ``libpa.so`` for gfx950 with hipcc, in-tree.

Every source under ``csrc/`` is compiled for ``--offload-arch=gfx950`` (code
object v5, the version the HIP runtime bundled with PyTorch loads), objects go
to ``_build/`` and the shared library to ``paged_kv_cache_303_amd/libpa.so``.
Packed fp32 VALU ops are disabled for the device code.

    python -m paged_kv_cache_303_amd.build
"""

from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
ARCH = "gfx950"

COMMON = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++20",
    "-fPIC",
    "-mcode-object-version=5",
    "-Wall",
    "-Wno-unused-result",
    # No NaN semantics for float operations: max reductions and compares need
    # no quieting or canonicalising.  Nothing that keeps NaN-poisoned rows out
    # of the sums is a float operation (masks select integer bit patterns, and
    # gathers past a range's end are clamped to valid rows), so the flag
    # cannot fold them away.
    "-fno-honor-nans",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}",
]


def library_path() -> str:
    """The library the binding loads: ``$PA_LIBRARY`` if set, else the in-tree build."""
    return os.environ.get("PA_LIBRARY") or os.path.join(PKG, "libpa.so")


def _hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the HIP library cannot be built")
    return path


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def _compile(src: str, verbose: bool, defines=(), build_dir=BUILD_DIR) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *COMMON, *[f"-D{d}" for d in defines], "-c", src, "-o", obj]
    if not src.endswith(".hip"):
        cmd[1:1] = ["-x", "hip"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = False, defines=(), out: str | None = None) -> str:
    """Compile every source and link ``libpa.so``; returns its path.

    ``defines`` (``NAME=VALUE`` strings) override compile-time tuning
    parameters such as ``PA_TILE_TOKENS``; ``out`` places the library
    elsewhere (the binding loads it when ``PA_LIBRARY`` names it).
    """
    build_dir = BUILD_DIR if not defines else os.path.join(
        BUILD_DIR, "_".join(d.replace("=", "") for d in defines))
    os.makedirs(build_dir, exist_ok=True)
    srcs = sources()
    workers = min(len(srcs), max(1, (os.cpu_count() or 2) // 2), 8)
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, defines, build_dir), srcs))
    out = out or library_path()
    tmp = out + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, out)
    return out


def source_hash(source: str | None = None) -> str:
    """SHA-256 over the kernel sources and headers (ties measurements to a version).

    With ``source`` (a file name under csrc/, e.g. ``"pa_decode.hip"``) only that
    source and the headers count, so a measurement of its kernels stays current
    while other sources change."""
    import hashlib
    h = hashlib.sha256()
    srcs = sources() if source is None else [os.path.join(CSRC, source)]
    files = srcs + sorted(glob.glob(os.path.join(CSRC, "*.h")))
    files.append(os.path.join(ROOT, "include", "pa.h"))
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


if __name__ == "__main__":
    print(build(verbose=True))
