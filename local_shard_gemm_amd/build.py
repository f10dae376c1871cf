"""Build libshardmm.so in-tree with hipcc for gfx950.

Every source under csrc/ is compiled for gfx950 only, with packed-fp32
instruction generation disabled, and linked into
``local_shard_gemm_amd/libshardmm.so`` next to this file. The library is
stamped with a sha256 of its sources (``source_digest``), which the binding
compares before loading it, so a stale build is never used.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libshardmm.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (needed to build libshardmm for gfx950)")


COMMON = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-I" + INCLUDE,
    "-I" + CSRC,
    # Packed fp32 VALU ops are kept out of the generated code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.cpp")) + glob.glob(os.path.join(CSRC, "*.hip")))


DIGEST_MARKER = b"SM_SOURCE_DIGEST="


def digest_inputs(root: str = ROOT):
    """Files whose contents decide the built library: every source and
    header under csrc/, the public header, and this build script (flags)."""
    pkg = os.path.join(root, "local_shard_gemm_amd")
    files = []
    for pat in ("*.cpp", "*.hip", "*.h"):
        files += glob.glob(os.path.join(pkg, "csrc", pat))
    files.append(os.path.join(root, "include", "shardmm.h"))
    files.append(os.path.join(pkg, "build.py"))
    return sorted(files, key=lambda f: os.path.relpath(f, root))


def source_digest(root: str = ROOT) -> str:
    """sha256 over (relative path, contents) of digest_inputs(root)."""
    import hashlib

    h = hashlib.sha256()
    for f in digest_inputs(root):
        h.update(os.path.relpath(f, root).encode() + b"\0")
        with open(f, "rb") as fh:
            h.update(fh.read())
        h.update(b"\0")
    return h.hexdigest()


def library_digest(path: str = None):
    """The source digest stamped into a built library (None if absent)."""
    path = path or LIB
    try:
        with open(path, "rb") as f:
            data = f.read()
    except OSError:
        return None
    i = data.find(DIGEST_MARKER)
    if i < 0:
        return None
    d = data[i + len(DIGEST_MARKER):i + len(DIGEST_MARKER) + 64]
    return d.decode("ascii", "replace") if len(d) == 64 else None


def _compile(src: str, verbose: bool, digest: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), *COMMON, f'-DSM_SOURCE_DIGEST="{digest}"', "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err and verbose:
        print(err, flush=True)
    return obj


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    digest = source_digest()
    with ThreadPoolExecutor(max_workers=max(1, min(jobs, len(srcs)))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, digest), srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
