"""The library's source stamp: libshardmm.so carries a sha256 of the sources
it was built from, the binding compares it with the current sources before
loading, and a stale library is rebuilt or refused, never loaded."""
import os
import shutil

import pytest

import local_shard_gemm_amd as sm
from local_shard_gemm_amd import build


def test_library_carries_the_source_stamp():
    lib = sm.load()
    want = build.source_digest()
    assert build.library_digest() == want
    if sm.loaded_library_path() == sm.LIB_PATH:
        assert lib.sm_build_digest().decode() == want


def test_changed_source_changes_the_digest(tmp_path):
    root = str(tmp_path)
    for f in build.digest_inputs():
        dst = os.path.join(root, os.path.relpath(f, build.ROOT))
        os.makedirs(os.path.dirname(dst), exist_ok=True)
        shutil.copyfile(f, dst)
    d0 = build.source_digest(root)
    assert d0 == build.source_digest()
    src = os.path.join(root, "local_shard_gemm_amd", "csrc", "gemm_mfma.hip")
    with open(src, "ab") as f:
        f.write(b"\n")
    assert build.source_digest(root) != d0
    os.remove(src)  # a removed source changes it too
    assert build.source_digest(root) not in (d0, None)


def test_stale_library_refused_when_it_cannot_be_rebuilt(tmp_path, monkeypatch):
    stale = tmp_path / "libshardmm.so"
    stale.write_bytes(b"\x7fELF" + build.DIGEST_MARKER + b"0" * 64)
    assert build.library_digest(str(stale)) == "0" * 64

    def no_compiler(*a, **k):
        raise RuntimeError("hipcc not found (needed to build libshardmm for gfx950)")

    monkeypatch.setattr(build, "build", no_compiler)
    with pytest.raises(sm.ShardmmError) as ei:
        sm.ensure_fresh(str(stale))
    assert "older than its sources" in str(ei.value)
    with pytest.raises(sm.ShardmmError) as ei:
        sm.ensure_fresh(str(tmp_path / "missing.so"))
    assert "missing" in str(ei.value)
