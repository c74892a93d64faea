"""The C-ABI library loads, exports every declared entry point, and rejects
bad arguments on the host before touching a device (CPU only: no call here
launches work)."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import compressed_kv_attention_amd as ada

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "ada.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", src)) - {"if", "sizeof"})


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert {"ada_encode", "rdr_pack", "ada_decode", "ada_decode_stream", "ada_decode_merge",
            "dense_decode", "dense_pack"} <= set(names)
    lib = C.CDLL(ada.lib_path())
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_version():
    L = ada.load()
    for st in range(6):
        assert L.ada_status_str(st)
    assert L.ada_status_str(99) == b"unknown status"
    assert L.ada_version() >= 100


def test_phase_trace_is_refused_by_the_product_build():
    """Only the tracing build records phase timestamps; the product library
    refuses the call and changes nothing (no device memory is touched)."""
    L = ada.load()
    assert L.ada_phase_trace(C.c_void_p(64), 4096) == ada.EUNSUPPORTED
    assert L.ada_phase_trace(None, 0) == ada.EUNSUPPORTED


def test_page_bytes_match_the_format():
    assert [ada.page_bytes(128, t) for t in range(4)] == [8192, 4480, 2304, 8192]
    assert [ada.page_bytes(64, t) for t in range(4)] == [4096, 2304, 1152, 4096]
    assert ada.page_bytes(96, 0) == 0 and ada.page_bytes(128, 4) == 0


def test_pack_page_count_and_workspace():
    g = ada.Geom(128, 32, 8)
    # config-2 mix at T=32768: 308 + 922 + 512 pages per kv-head
    assert ada.pack_num_pages(g, [0, 32768], [[1500, 6000, 8500]]) == 8 * 1742
    assert ada.pack_num_pages(g, [0, 0, 5], [[0, 0, 0], [10000, 10000, 10000]]) == 8
    assert ada.pack_workspace_size(g, 32768, 1) > 32768 * 8 * 4
    assert ada.decode_workspace_size(g, 1, 2000) >= 8 * ada.decode_default_splits(g, 1, 2000) * 4 * 130 * 4


def _bad(call):
    with pytest.raises(ada.AdaError) as e:
        call()
    return e.value.status


def test_host_argument_errors():
    L = ada.load()
    for bad in (ada.Geom(96, 32, 8), ada.Geom(128, 30, 8), ada.Geom(128, 32, 8, 32), ada.Geom(128, 0, 8)):
        assert L.rdr_pack_num_pages(C.byref(bad), 1, np.array([0, 16], np.int32).ctypes.data_as(C.c_void_p),
                                    np.array([5000, 5000, 5000], np.int32).ctypes.data_as(C.c_void_p),
                                    C.byref(C.c_int64())) == ada.EINVAL
    g = ada.Geom(128, 32, 8)
    # decreasing cumulative basis points / non-zero start / decreasing cu
    assert _bad(lambda: ada.pack_num_pages(g, [0, 16], [[5000, 4000, 9000]])) == ada.EINVAL
    assert _bad(lambda: ada.pack_num_pages(g, [1, 16], [[0, 0, 0]])) == ada.EINVAL
    assert _bad(lambda: ada.pack_num_pages(g, [0, 16, 8], [[0, 0, 0], [0, 0, 0]])) == ada.EINVAL
    # decode: null pointers and unsupported GQA ratios are refused before any launch
    view = ada._CacheView(0, 0, 0, 0, 0, 0, 0, 1, 4)
    assert L.ada_decode(C.byref(g), C.byref(view), None, None, None, 1.0, None, None, None, 0, None, 0,
                        None) == ada.EINVAL
    g3 = ada.Geom(128, 24, 8)  # GQA ratio 3 is not built
    view = ada._CacheView(16, 1, 16, 16, 16, 16, 0, 1, 4)
    assert L.ada_decode(C.byref(g3), C.byref(view), C.c_void_p(16), C.c_void_p(16), C.c_void_p(16), 1.0,
                        C.c_void_p(16), None, None, 0, C.c_void_p(256), 1 << 20, None) == ada.EUNSUPPORTED
    # too small a workspace
    view = ada._CacheView(16, 1, 16, 16, 16, 16, 0, 1, 4)
    assert L.ada_decode(C.byref(g), C.byref(view), C.c_void_p(16), C.c_void_p(16), C.c_void_p(16), 1.0,
                        C.c_void_p(16), None, None, 0, C.c_void_p(256), 8, None) == ada.EWORKSPACE
    # encode with no tokens is a no-op; negative counts are refused
    assert L.ada_encode(C.byref(g), 0, None, None, None, None, None, None, None) == ada.OK
    assert L.ada_encode(C.byref(g), -1, None, None, None, None, None, None, None) == ada.EINVAL
    # keys and both codebooks must be 16-byte aligned (staged with 16-byte loads)
    p16, p4 = C.c_void_p(256), C.c_void_p(260)
    for keys, cb8, cb4 in ((p4, p16, p16), (p16, p4, p16), (p16, p16, p4)):
        assert L.ada_encode(C.byref(g), 1, keys, cb8, cb4, p16, p16, p16, None) == ada.EINVAL


def test_pack_host_errors_leave_host_state_untouched():
    """Arena overflow and row-capacity errors come back before any device
    work, with the cursor and page counts unchanged (no device needed: the
    device pointers are never dereferenced on these paths)."""
    L = ada.load()
    g = ada.Geom(64, 4, 2)
    cu = np.array([0, 64], np.int32)
    bp = np.array([2500, 7500, 10000], np.int32)
    cursor = np.zeros(1, np.uint64)
    npages = np.zeros(2, np.int32)
    fake = C.c_void_p(256)

    def call(arena_units, maxp, protect=None, perm=None):
        view = ada._CacheView(256, arena_units, 256, 256, 256, 256, 0, 1, maxp)
        return L.rdr_pack(C.byref(g), C.byref(view), 1, cu.ctypes.data_as(C.c_void_p),
                          bp.ctypes.data_as(C.c_void_p), fake, fake, fake, fake, fake, fake,
                          None if protect is None else protect.ctypes.data_as(C.c_void_p),
                          None if perm is None else perm.ctypes.data_as(C.c_void_p), None,
                          cursor.ctypes.data_as(C.c_void_p), npages.ctypes.data_as(C.c_void_p),
                          C.c_void_p(1 << 20), 1 << 30, None)

    assert call(arena_units=10, maxp=64) == ada.ENOSPACE          # needs 2 * 36 units + more
    assert call(arena_units=1 << 20, maxp=3) == ada.EINVAL        # 4 pages per row needed
    prot = np.zeros((64, 2), np.uint8)
    prot[:17, 1] = 1                                              # 16 fp16 slots only
    assert call(arena_units=1 << 20, maxp=64, protect=prot) == ada.EINVAL
    bad_perm = np.zeros(8, np.uint32)
    assert call(arena_units=1 << 20, maxp=64, perm=bad_perm) == ada.EINVAL
    # misaligned keys / values (16-byte loads) or codes (4-byte loads)
    view = ada._CacheView(256, 1 << 20, 256, 256, 256, 256, 0, 1, 64)
    for k, v, c8, c4 in ((264, 256, 256, 256), (256, 264, 256, 256), (256, 256, 258, 256),
                         (256, 256, 256, 257)):
        assert L.rdr_pack(C.byref(g), C.byref(view), 1, cu.ctypes.data_as(C.c_void_p),
                          bp.ctypes.data_as(C.c_void_p), C.c_void_p(k), C.c_void_p(v), fake,
                          C.c_void_p(c8), C.c_void_p(c4), fake, None, None, None,
                          cursor.ctypes.data_as(C.c_void_p), npages.ctypes.data_as(C.c_void_p),
                          C.c_void_p(1 << 20), 1 << 30, None) == ada.EINVAL
    assert cursor[0] == 0 and not npages.any()


def test_rdr_entry_points_host_errors():
    """The budget solver, tier counts and tier-given pack refuse bad host
    arguments before any launch (device pointers are never dereferenced)."""
    L = ada.load()
    g = ada.Geom(64, 4, 2)
    names = _declared()
    assert {"ada_code_error", "rdr_solve", "rdr_tier_counts", "rdr_pack_tiers",
            "rdr_pack_tiers_num_pages"} <= set(names)
    cu = np.array([0, 10, 30], np.int32)
    fake = C.c_void_p(256)
    cup = cu.ctypes.data_as(C.c_void_p)

    def solve(budget, ws_bytes=1 << 20, ws=fake):
        b = np.asarray(budget, np.int64)
        return L.rdr_solve(C.byref(g), 2, cup, b.ctypes.data_as(C.c_void_p), fake, fake, fake, fake, None,
                           fake, None, ws, ws_bytes, None)

    assert solve([100, -1]) == ada.EINVAL
    assert solve([100, 100], ws_bytes=16) == ada.EWORKSPACE
    assert solve([100, 100], ws=C.c_void_p(257)) == ada.EWORKSPACE
    assert L.rdr_solve(C.byref(g), 2, cup, None, fake, fake, fake, fake, None, fake, None, fake, 1 << 20,
                       None) == ada.EINVAL
    assert ada.solve_workspace_size(g, 2, 30) >= 4 * 256 * 8 * 2
    # tier counts: null output, too small a workspace
    assert L.rdr_tier_counts(C.byref(g), 2, cup, fake, None, fake, 1 << 20, None) == ada.EINVAL
    out = np.zeros((4, 3), np.int32)
    assert L.rdr_tier_counts(C.byref(g), 2, cup, fake, out.ctypes.data_as(C.c_void_p), fake, 8,
                             None) == ada.EWORKSPACE
    # page count from row counts (host arithmetic only)
    rc = np.array([[3, 16, 17], [0, 0, 1], [16, 0, 0], [0, 0, 0]], np.int32)
    assert ada.pack_tiers_num_pages(g, rc) == 1 + 1 + 2 + 1 + 1
    # tier-given pack: a row whose counts exceed its tokens, negative counts
    cursor = np.zeros(1, np.uint64)
    npages = np.zeros(4, np.int32)
    view = ada._CacheView(256, 1 << 20, 256, 256, 256, 256, 0, 2, 64)

    def pack(counts):
        c = np.asarray(counts, np.int32)
        return L.rdr_pack_tiers(C.byref(g), C.byref(view), 2, cup, c.ctypes.data_as(C.c_void_p), fake,
                                fake, fake, fake, fake, fake, None, None,
                                cursor.ctypes.data_as(C.c_void_p), npages.ctypes.data_as(C.c_void_p),
                                C.c_void_p(1 << 20), 1 << 30, None)

    assert pack([[5, 5, 1], [0, 0, 0], [0, 0, 0], [0, 0, 0]]) == ada.EINVAL    # 11 > 10 tokens
    assert pack([[-1, 0, 0], [0, 0, 0], [0, 0, 0], [0, 0, 0]]) == ada.EINVAL
    assert cursor[0] == 0 and not npages.any()
    # code error: nothing to do for no tokens; negative counts refused
    assert L.ada_code_error(C.byref(g), 0, None, None, None, None, None, None, None, None) == ada.OK
    assert L.ada_code_error(C.byref(g), -2, None, None, None, None, None, None, None, None) == ada.EINVAL


def test_decode_refuses_a_split_count_whose_tables_overflow_lds():
    """GQA 8 at D = 128 keeps a 136 KiB LUT in LDS: one split over 8192 pages
    leaves no room for the page-table entries (refused on the host); the
    default split count always fits."""
    L = ada.load()
    g = ada.Geom(128, 8, 1)
    maxp = 8192
    view = ada._CacheView(256, 1 << 20, 256, 256, 256, 256, 0, 1, maxp)
    ws = ada.decode_workspace_size(g, 1, maxp, 1)
    fake = C.c_void_p(256)
    assert L.ada_decode(C.byref(g), C.byref(view), fake, fake, fake, 1.0, fake, None, None, 1,
                        C.c_void_p(1 << 20), ws, None) == ada.EINVAL
    ns = ada.decode_default_splits(g, 1, maxp)
    lut = 16 * 272 * 8 * 4
    assert lut + -(-maxp // ns) * 8 <= 160 * 1024 and ns <= 1024


def test_load_refuses_a_stale_library(monkeypatch):
    """The library carries the digest of the sources it was built from; a
    binding whose sources have changed since refuses to load it."""
    import compressed_kv_attention_amd as ada
    import compressed_kv_attention_amd.build as b
    assert ada.load().ada_build_id().decode() == b.source_digest()
    monkeypatch.setattr(ada, "_lib", None)
    monkeypatch.setattr(b, "source_digest", lambda: "0" * 64)
    with pytest.raises(ImportError, match="stale"):
        ada.load()


def test_cache_view_keeps_its_buffers_alive():
    """A view holds raw addresses; it must keep the tensors behind them alive
    (a freed arena copy read through a view would be a use after free)."""
    import gc
    import weakref

    import torch
    geom = ada.Geom(64, 4, 4)
    c = ada.Cache(geom, 1, 4, 4096, device="cpu")
    sub = torch.zeros_like(c.arena)
    ref = weakref.ref(sub)
    v = c.view(sub)
    del sub
    gc.collect()
    assert ref() is not None and v.arena == ref().data_ptr()
    del v
    gc.collect()
    assert ref() is None


def test_noalloc_decode_rejects_partials_beyond_its_array_on_the_host():
    """ada_decode_noalloc checks the step's partials against its fixed array
    before any device work: too many splits is ADA_EWORKSPACE."""
    lib = ada.load()
    geom = ada.Geom(128, 32, 8)
    need = ada.decode_workspace_size(geom, 64, 4200, 64)
    assert need > (8 << 20)
    view = ada._CacheView(1 << 20, 1, 1 << 21, 1 << 22, 1 << 23, 1 << 24, None, 64, 4200)
    st = lib.ada_decode_noalloc(C.byref(geom), C.byref(view), C.c_void_p(256), C.c_void_p(256),
                                C.c_void_p(256), 0.1, C.c_void_p(256), None, None, 64, None)
    assert st == ada.EWORKSPACE
    st = lib.ada_decode_noalloc(C.byref(geom), C.byref(view), C.c_void_p(256), C.c_void_p(256),
                                C.c_void_p(256), 0.1, C.c_void_p(256), None, None, 2000, None)
    assert st == ada.EINVAL
