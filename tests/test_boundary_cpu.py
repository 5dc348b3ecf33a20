"""The C-ABI boundary without a GPU: the library loads, exports every entry
point include/vpe.h declares, and rejects invalid arguments on the host before
any HIP call (these calls never reach a kernel launch)."""
import ctypes
import os
import re

import numpy as np
import pytest

import vocab_sharded_embedding_amd as vpe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vpe.h")

FAKE = 0x10000  # a non-null, 16-byte aligned address that is never dereferenced
F32, BF16, I32, I64 = vpe.VPE_F32, vpe.VPE_BF16, vpe.VPE_I32, vpe.VPE_I64


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:vpe_status|const char \*)\s*(vpe_\w+)\s*\(", text, re.M)))


def test_header_declares_the_calls():
    assert _declared() == sorted(["vpe_shard_range", "vpe_embed", "vpe_sum_partials",
                                  "vpe_last_token_select", "vpe_lmhead", "vpe_lmhead_prefill",
                                  "vpe_argmax_init", "vpe_lmhead_argmax",
                                  "vpe_lmhead_prefill_argmax", "vpe_argmax_decode",
                                  "vpe_argmax_decode_clear",
                                  "vpe_load_shard", "vpe_lmhead_logsumexp_workspace",
                                  "vpe_lmhead_logsumexp", "vpe_lmhead_prefill_logsumexp",
                                  "vpe_logsumexp_combine",
                                  "vpe_lmhead_logsumexp_noalloc", "vpe_status_string"])


def test_library_exports_every_declared_symbol():
    lib = vpe.load_library()
    for name in _declared():
        assert hasattr(lib, name), name
    assert set(_declared()) == set(vpe.EXPORTED_SYMBOLS)


def test_status_strings():
    names = ["VPE_OK", "VPE_ERR_NULL", "VPE_ERR_SHAPE", "VPE_ERR_DTYPE", "VPE_ERR_ALIGN",
             "VPE_ERR_SHARD", "VPE_ERR_LAUNCH", "VPE_ERR_RANGE"]
    for code, name in enumerate(names):
        assert vpe.status_name(code) == name


def test_shard_range():
    assert vpe.vpe_shard_range(151936, 2, 0) == (0, 75968)
    assert vpe.vpe_shard_range(151936, 2, 1) == (75968, 151936)
    assert vpe.vpe_shard_range(151936, 4, 2) == (75968, 113952)
    assert vpe.vpe_shard_range(12, 1, 0) == (0, 12)
    lib = vpe.load_library()
    s, e = ctypes.c_int64(), ctypes.c_int64()
    for args in [(10, 3, 0), (12, 2, 2), (12, 2, -1), (12, 0, 0), (0, 1, 0)]:
        assert lib.vpe_shard_range(*args, ctypes.byref(s), ctypes.byref(e)) == vpe.VPE_ERR_SHARD
    assert lib.vpe_shard_range(12, 2, 0, None, ctypes.byref(e)) == vpe.VPE_ERR_NULL


def test_embed_validation():
    lib = vpe.load_library()
    ok = dict(ids=FAKE, itype=I32, n=10, w=FAKE, dt=BF16, rows=100, dim=64, start=0, out=FAKE)

    def call(**kw):
        a = {**ok, **kw}
        return lib.vpe_embed(a["ids"], a["itype"], a["n"], a["w"], a["dt"], a["rows"], a["dim"],
                             a["start"], a["out"], None)

    assert call(dt=9) == vpe.VPE_ERR_DTYPE
    assert call(itype=5) == vpe.VPE_ERR_DTYPE
    assert call(n=-1) == vpe.VPE_ERR_SHAPE
    assert call(dim=0) == vpe.VPE_ERR_SHAPE
    assert call(rows=0) == vpe.VPE_ERR_SHAPE
    assert call(n=2 ** 40) == vpe.VPE_ERR_SHAPE
    assert call(ids=None) == vpe.VPE_ERR_NULL
    assert call(w=None) == vpe.VPE_ERR_NULL
    assert call(out=None) == vpe.VPE_ERR_NULL
    assert call(out=FAKE + 1) == vpe.VPE_ERR_ALIGN
    assert call(ids=FAKE + 2) == vpe.VPE_ERR_ALIGN
    assert call(itype=I64, ids=FAKE + 4) == vpe.VPE_ERR_ALIGN
    assert call(dt=F32, w=FAKE + 2) == vpe.VPE_ERR_ALIGN
    assert call(start=-1) == vpe.VPE_ERR_RANGE
    assert call(start=2 ** 63 - 100) == vpe.VPE_ERR_RANGE
    assert call(start=2 ** 63 - 101, n=0) == vpe.VPE_OK
    # empty input: valid, enqueues nothing, even with NULL pointers
    assert call(n=0, ids=None, w=None, out=None) == vpe.VPE_OK


def test_sum_partials_validation():
    lib = vpe.load_library()
    arr = (ctypes.c_void_p * 65)(*([FAKE] * 65))
    assert lib.vpe_sum_partials(arr, 0, 10, BF16, FAKE, None) == vpe.VPE_ERR_SHAPE
    assert lib.vpe_sum_partials(arr, 65, 10, BF16, FAKE, None) == vpe.VPE_ERR_SHAPE
    assert lib.vpe_sum_partials(arr, 2, -1, BF16, FAKE, None) == vpe.VPE_ERR_SHAPE
    assert lib.vpe_sum_partials(arr, 2, 10, 7, FAKE, None) == vpe.VPE_ERR_DTYPE
    assert lib.vpe_sum_partials(arr, 2, 10, BF16, None, None) == vpe.VPE_ERR_NULL
    assert lib.vpe_sum_partials(None, 2, 10, BF16, FAKE, None) == vpe.VPE_ERR_NULL
    bad = (ctypes.c_void_p * 2)(FAKE, None)
    assert lib.vpe_sum_partials(bad, 2, 10, BF16, FAKE, None) == vpe.VPE_ERR_NULL
    mis = (ctypes.c_void_p * 2)(FAKE, FAKE + 1)
    assert lib.vpe_sum_partials(mis, 2, 10, BF16, FAKE, None) == vpe.VPE_ERR_ALIGN
    assert lib.vpe_sum_partials(arr, 2, 10, F32, FAKE + 2, None) == vpe.VPE_ERR_ALIGN
    assert lib.vpe_sum_partials(arr, 2, 0, BF16, None, None) == vpe.VPE_OK


def test_select_validation():
    lib = vpe.load_library()
    f = lib.vpe_last_token_select
    assert f(FAKE, -1, 64, BF16, FAKE, 4, FAKE, None) == vpe.VPE_ERR_SHAPE
    assert f(FAKE, 100, 0, BF16, FAKE, 4, FAKE, None) == vpe.VPE_ERR_SHAPE
    assert f(FAKE, 100, 64, BF16, FAKE, -1, FAKE, None) == vpe.VPE_ERR_SHAPE
    assert f(FAKE, 2 ** 31, 64, BF16, FAKE, 4, FAKE, None) == vpe.VPE_ERR_SHAPE
    assert f(FAKE, 100, 64, 3, FAKE, 4, FAKE, None) == vpe.VPE_ERR_DTYPE
    assert f(FAKE, 100, 64, BF16, None, 4, FAKE, None) == vpe.VPE_ERR_NULL
    assert f(FAKE, 100, 64, BF16, FAKE + 2, 4, FAKE, None) == vpe.VPE_ERR_ALIGN
    assert f(FAKE, 100, 64, F32, FAKE, 4, FAKE + 2, None) == vpe.VPE_ERR_ALIGN
    assert f(None, 0, 64, BF16, FAKE, 0, None, None) == vpe.VPE_OK


def test_lmhead_validation():
    lib = vpe.load_library()
    ok = dict(x=FAKE, m=4, dim=64, w=FAKE, rows=100, dt=BF16, out=FAKE, ld=100, col=0)

    def call(**kw):
        a = {**ok, **kw}
        return lib.vpe_lmhead(a["x"], a["m"], a["dim"], a["w"], a["rows"], a["dt"], a["out"],
                              a["ld"], a["col"], None)

    assert call(dt=2) == vpe.VPE_ERR_DTYPE
    assert call(m=-1) == vpe.VPE_ERR_SHAPE
    assert call(dim=0) == vpe.VPE_ERR_SHAPE
    assert call(rows=0) == vpe.VPE_ERR_SHAPE
    assert call(m=2 ** 21 + 1) == vpe.VPE_ERR_SHAPE
    assert call(dim=2 ** 20 + 8) == vpe.VPE_ERR_SHAPE
    assert call(ld=99) == vpe.VPE_ERR_RANGE
    assert call(ld=150, col=51) == vpe.VPE_ERR_RANGE
    assert call(col=-1, ld=200) == vpe.VPE_ERR_RANGE
    assert call(x=None) == vpe.VPE_ERR_NULL
    assert call(out=None) == vpe.VPE_ERR_NULL
    assert call(x=FAKE + 1) == vpe.VPE_ERR_ALIGN
    assert call(dt=F32, out=FAKE + 2) == vpe.VPE_ERR_ALIGN
    assert call(m=0, x=None, w=None, out=None) == vpe.VPE_OK


def test_binding_rejects_host_tensors():
    torch = pytest.importorskip("torch")
    ids = torch.zeros(4, dtype=torch.int32)
    w = torch.zeros(8, 16)
    with pytest.raises(ValueError):
        vpe.vpe_embed(ids, w, 0)
    with pytest.raises(ValueError):
        vpe.vpe_lmhead(torch.zeros(2, 16), w)
    with pytest.raises(ValueError):
        vpe.vpe_sum_partials([w, w])
    with pytest.raises(ValueError):
        vpe.vpe_last_token_select(w, torch.zeros(2, dtype=torch.int32))


def test_product_package_does_not_import_the_oracle():
    pkg = os.path.dirname(vpe.__file__)
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, fn), encoding="utf-8").read()
                for bad in ("import oracle", "from oracle", "liboracle", "oracle.c"):
                    assert bad not in text, (fn, bad)


def test_lmhead_prefill_validation():
    lib = vpe.load_library()
    ok = dict(h=FAKE, t=100, dim=64, cu=FAKE, s=4, w=FAKE, rows=100, dt=BF16, out=FAKE, ld=100,
              col=0)

    def call(**kw):
        a = {**ok, **kw}
        return lib.vpe_lmhead_prefill(a["h"], a["t"], a["dim"], a["cu"], a["s"], a["w"],
                                      a["rows"], a["dt"], a["out"], a["ld"], a["col"], None)

    assert call(dt=5) == vpe.VPE_ERR_DTYPE
    assert call(t=-1) == vpe.VPE_ERR_SHAPE
    assert call(t=2 ** 31) == vpe.VPE_ERR_SHAPE
    assert call(s=-1) == vpe.VPE_ERR_SHAPE
    assert call(s=2 ** 21 + 1) == vpe.VPE_ERR_SHAPE
    assert call(dim=0) == vpe.VPE_ERR_SHAPE
    assert call(dim=2 ** 20 + 8) == vpe.VPE_ERR_SHAPE
    assert call(rows=0) == vpe.VPE_ERR_SHAPE
    assert call(ld=99) == vpe.VPE_ERR_RANGE
    assert call(col=1) == vpe.VPE_ERR_RANGE
    assert call(cu=None) == vpe.VPE_ERR_NULL
    assert call(h=None) == vpe.VPE_ERR_NULL
    assert call(cu=FAKE + 2) == vpe.VPE_ERR_ALIGN
    assert call(dt=F32, h=FAKE + 2) == vpe.VPE_ERR_ALIGN
    assert call(s=0, h=None, cu=None, w=None, out=None) == vpe.VPE_OK


def test_argmax_validation():
    lib = vpe.load_library()
    assert lib.vpe_argmax_init(FAKE, -1, None) == vpe.VPE_ERR_SHAPE
    assert lib.vpe_argmax_init(None, 4, None) == vpe.VPE_ERR_NULL
    assert lib.vpe_argmax_init(FAKE + 4, 4, None) == vpe.VPE_ERR_ALIGN
    assert lib.vpe_argmax_init(None, 0, None) == vpe.VPE_OK
    f = lib.vpe_lmhead_argmax
    assert f(FAKE, 4, 64, FAKE, 100, 9, 0, FAKE, None) == vpe.VPE_ERR_DTYPE
    assert f(FAKE, -1, 64, FAKE, 100, BF16, 0, FAKE, None) == vpe.VPE_ERR_SHAPE
    assert f(FAKE, 4, 0, FAKE, 100, BF16, 0, FAKE, None) == vpe.VPE_ERR_SHAPE
    assert f(FAKE, 4, 64, FAKE, 0, BF16, 0, FAKE, None) == vpe.VPE_ERR_SHAPE
    assert f(FAKE, 4, 64, FAKE, 100, BF16, -1, FAKE, None) == vpe.VPE_ERR_RANGE
    assert f(FAKE, 4, 64, FAKE, 100, BF16, 2 ** 32 - 100, FAKE, None) == vpe.VPE_ERR_RANGE
    assert f(FAKE, 4, 64, FAKE, 100, BF16, 0, None, None) == vpe.VPE_ERR_NULL
    assert f(FAKE, 4, 64, FAKE, 100, BF16, 0, FAKE + 4, None) == vpe.VPE_ERR_ALIGN
    assert f(None, 0, 64, None, 100, BF16, 0, None, None) == vpe.VPE_OK
    d = lib.vpe_argmax_decode
    assert d(FAKE, 4, None, None, None) == vpe.VPE_ERR_NULL
    assert d(FAKE, -1, FAKE, FAKE, None) == vpe.VPE_ERR_SHAPE
    assert d(FAKE, 4, FAKE + 2, FAKE, None) == vpe.VPE_ERR_ALIGN
    assert d(None, 0, None, None, None) == vpe.VPE_OK
    assert lib.vpe_argmax_init(FAKE, 2 ** 21 + 1, None) == vpe.VPE_ERR_SHAPE
    assert d(FAKE, 2 ** 21 + 1, FAKE, FAKE, None) == vpe.VPE_ERR_SHAPE
    c = lib.vpe_argmax_decode_clear
    assert c(FAKE, 4, None, None, None) == vpe.VPE_ERR_NULL
    assert c(None, 4, FAKE, FAKE, None) == vpe.VPE_ERR_NULL
    assert c(FAKE, -1, FAKE, FAKE, None) == vpe.VPE_ERR_SHAPE
    assert c(FAKE, 2 ** 21 + 1, FAKE, FAKE, None) == vpe.VPE_ERR_SHAPE
    assert c(FAKE + 4, 4, FAKE, FAKE, None) == vpe.VPE_ERR_ALIGN
    assert c(FAKE, 4, FAKE + 2, FAKE, None) == vpe.VPE_ERR_ALIGN
    assert c(None, 0, None, None, None) == vpe.VPE_OK
    assert f(FAKE, 2 ** 21 + 1, 64, FAKE, 100, BF16, 0, FAKE, None) == vpe.VPE_ERR_SHAPE


def test_prefill_argmax_validation():
    lib = vpe.load_library()
    f = lib.vpe_lmhead_prefill_argmax
    ok = dict(h=FAKE, t=1000, d=64, cu=FAKE, s=4, w=FAKE, rows=100, dt=BF16, start=0, best=FAKE)

    def call(**kw):
        a = {**ok, **kw}
        return f(a["h"], a["t"], a["d"], a["cu"], a["s"], a["w"], a["rows"], a["dt"], a["start"],
                 a["best"], None)

    assert call(dt=9) == vpe.VPE_ERR_DTYPE
    assert call(t=-1) == vpe.VPE_ERR_SHAPE
    assert call(t=2 ** 31) == vpe.VPE_ERR_SHAPE
    assert call(s=-1) == vpe.VPE_ERR_SHAPE
    assert call(s=2 ** 21 + 1) == vpe.VPE_ERR_SHAPE
    assert call(d=0) == vpe.VPE_ERR_SHAPE
    assert call(d=2 ** 20 + 8) == vpe.VPE_ERR_SHAPE
    assert call(rows=0) == vpe.VPE_ERR_SHAPE
    assert call(start=-1) == vpe.VPE_ERR_RANGE
    assert call(start=2 ** 32 - 100) == vpe.VPE_ERR_RANGE
    assert call(h=None) == vpe.VPE_ERR_NULL
    assert call(cu=None) == vpe.VPE_ERR_NULL
    assert call(best=None) == vpe.VPE_ERR_NULL
    assert call(cu=FAKE + 2) == vpe.VPE_ERR_ALIGN
    assert call(best=FAKE + 4) == vpe.VPE_ERR_ALIGN
    assert call(dt=F32, w=FAKE + 2) == vpe.VPE_ERR_ALIGN
    assert call(s=0, h=None, cu=None, w=None, best=None) == vpe.VPE_OK


def test_load_shard_validation():
    lib = vpe.load_library()
    f = lib.vpe_load_shard
    assert f(FAKE, 100, 8, 9, 2, 0, FAKE + 4096, None) == vpe.VPE_ERR_DTYPE
    assert f(FAKE, 100, 0, BF16, 2, 0, FAKE + 4096, None) == vpe.VPE_ERR_SHAPE
    assert f(FAKE, 0, 8, BF16, 2, 0, FAKE + 4096, None) == vpe.VPE_ERR_SHAPE
    assert f(FAKE, 2 ** 40, 2 ** 10, BF16, 2, 0, FAKE + 4096, None) == vpe.VPE_ERR_SHAPE
    assert f(FAKE, 101, 8, BF16, 2, 0, FAKE + 4096, None) == vpe.VPE_ERR_SHARD
    assert f(FAKE, 100, 8, BF16, 2, 2, FAKE + 4096, None) == vpe.VPE_ERR_SHARD
    assert f(FAKE, 100, 8, BF16, 0, 0, FAKE + 4096, None) == vpe.VPE_ERR_SHARD
    assert f(None, 100, 8, BF16, 2, 0, FAKE + 4096, None) == vpe.VPE_ERR_NULL
    assert f(FAKE, 100, 8, BF16, 2, 0, None, None) == vpe.VPE_ERR_NULL
    assert f(FAKE + 1, 100, 8, BF16, 2, 0, FAKE + 4096, None) == vpe.VPE_ERR_ALIGN
    assert f(FAKE, 100, 8, F32, 2, 0, FAKE + 4098, None) == vpe.VPE_ERR_ALIGN
    # rank 1's rows start at byte 50*8*2 = 800: a shard at FAKE + 1000 overlaps them
    assert f(FAKE, 100, 8, BF16, 2, 1, FAKE + 1000, None) == vpe.VPE_ERR_RANGE
    assert f(FAKE, 100, 8, BF16, 2, 0, FAKE + 16, None) == vpe.VPE_ERR_RANGE


# ---------------------------------------------------------------------------
# a library built from other sources is refused, not loaded silently
# ---------------------------------------------------------------------------
def test_built_library_matches_its_sources():
    from vocab_sharded_embedding_amd import build as vbuild
    assert vbuild.built_digest() == vbuild.source_digest()
    vpe.check_library_current()


def test_mismatched_digest_is_refused(tmp_path, monkeypatch):
    import shutil
    from vocab_sharded_embedding_amd import build as vbuild
    lib = tmp_path / "libvpe.so"
    shutil.copy(vpe.LIB_PATH, lib)
    # no digest recorded at all
    with pytest.raises(vpe.StaleLibraryError):
        vpe.check_library_current(str(lib))
    # a digest of other sources
    (tmp_path / "libvpe.so.sha256").write_text("0" * 64 + "\n")
    with pytest.raises(vpe.StaleLibraryError):
        vpe.check_library_current(str(lib))
    monkeypatch.setattr(vpe, "_lib", None)
    monkeypatch.delenv("VPE_REBUILD_STALE", raising=False)
    with pytest.raises(vpe.StaleLibraryError):
        vpe.load_library(str(lib))
    # the tree's own digest is accepted
    (tmp_path / "libvpe.so.sha256").write_text(vbuild.source_digest() + "\n")
    vpe.check_library_current(str(lib))


def test_source_edit_changes_the_digest(tmp_path, monkeypatch):
    from vocab_sharded_embedding_amd import build as vbuild
    files = vbuild.source_files()
    assert any(f.endswith("lmhead.hip") for f in files)
    assert any(f.endswith("vpe.h") for f in files)
    before = vbuild.source_digest()
    # the same file list with one kernel source edited by one byte
    edited = []
    for f in files:
        dst = tmp_path / os.path.basename(f)
        data = open(f, "rb").read()
        if f.endswith("gather.hip"):
            data += b" "
        dst.write_bytes(data)
        edited.append(str(dst))
    monkeypatch.setattr(vbuild, "source_files", lambda: edited)
    assert vbuild.source_digest() != before
