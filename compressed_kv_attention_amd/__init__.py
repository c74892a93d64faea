"""ADA (Angle-Domain Attention) decode path for MI355X -- Python binding.

This module only marshals arguments into libada (include/ada.h): every step
of encode, pack and decode runs in the library's gfx950 kernels.  PyTorch
provides device memory and the current stream.  There is no fallback: if
libada.so is missing or fails to load, every call raises.

Method: SPHERICAL KV (arXiv 2605.18856) -- gist.science technical summary,
sections 2.1 (keys as radius + angle codes; logits from the codes without
rebuilding keys) and 2.2 (per-state keep/drop and tier; tier-homogeneous
pages).
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np
import torch

__all__ = [
    "AdaError", "Geom", "Cache", "load", "lib_path", "page_bytes", "encode", "pack_num_pages",
    "pack_workspace_size", "rdr_pack", "dense_pack", "decode_default_splits",
    "decode_workspace_size", "decode", "decode_stage", "dense_decode",
    "code_error", "solve_workspace_size", "rdr_solve", "tier_counts", "pack_tiers_num_pages",
    "rdr_pack_tiers", "rdr_pack_tiers_device", "AppendState", "append", "retier", "retier_plan",
    "decode_sym_workspace_size", "decode_sym", "decode_noalloc", "phase_trace", "use_tracing_build",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libada.so")
_lib = None

OK, EINVAL, EUNSUPPORTED, ENOSPACE, EWORKSPACE, EHIP = range(6)


class AdaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {load().ada_status_str(status).decode()} (status {status})")


class Geom(C.Structure):
    _fields_ = [("head_dim", C.c_int32), ("num_q_heads", C.c_int32),
                ("num_kv_heads", C.c_int32), ("page_size", C.c_int32)]

    def __init__(self, head_dim, num_q_heads, num_kv_heads, page_size=16):
        super().__init__(head_dim, num_q_heads, num_kv_heads, page_size)


class _CacheView(C.Structure):
    _fields_ = [("arena", C.c_void_p), ("arena_units", C.c_uint64),
                ("page_table", C.c_void_p), ("page_meta", C.c_void_p),
                ("num_pages", C.c_void_p), ("tier_tokens", C.c_void_p),
                ("slot_token", C.c_void_p), ("num_seqs", C.c_int32),
                ("max_pages_per_head", C.c_int32)]


def lib_path() -> str:
    return _LIB_PATH


def use_tracing_build():
    """Loads libada_trace.so instead of libada.so: the same sources built
    with per-wave phase timestamps in the page stream (`python -m
    compressed_kv_attention_amd.build --phase-trace`).  For profiling only;
    call it before anything loads the library."""
    global _LIB_PATH
    if _lib is not None:
        raise RuntimeError("the library is already loaded")
    _LIB_PATH = os.path.join(_HERE, "libada_trace.so")


def load():
    """Loads libada.so once; raises if it is not built, or if it was built
    from other sources than the ones beside it (a stale library)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"{_LIB_PATH} is missing: build it with "
                              "`python -m compressed_kv_attention_amd.build`")
        L = C.CDLL(_LIB_PATH)
        L.ada_build_id.restype = C.c_char_p
        from .build import source_digest
        built, now = L.ada_build_id().decode(), source_digest()
        if built != now:
            raise ImportError(f"{_LIB_PATH} is stale: built from sources {built[:16]}, the sources "
                              f"are now {now[:16]}; rebuild with "
                              "`python -m compressed_kv_attention_amd.build`")
        P, I32, I64, U64, SZ, F = C.c_void_p, C.c_int32, C.c_int64, C.c_uint64, C.c_size_t, C.c_float
        G = C.POINTER(Geom)
        CV = C.POINTER(_CacheView)
        L.ada_status_str.argtypes = [C.c_int]
        L.ada_status_str.restype = C.c_char_p
        L.ada_version.restype = C.c_int
        L.ada_page_bytes.argtypes = [I32, I32]
        L.ada_page_bytes.restype = SZ
        L.ada_encode.argtypes = [G, I64, P, P, P, P, P, P, P]
        L.ada_encode.restype = C.c_int
        L.rdr_pack_num_pages.argtypes = [G, I32, P, P, P]
        L.rdr_pack_num_pages.restype = C.c_int
        L.rdr_pack_workspace_size.argtypes = [G, I64, I32]
        L.rdr_pack_workspace_size.restype = SZ
        L.rdr_pack.argtypes = [G, CV, I32, P, P, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P]
        L.rdr_pack.restype = C.c_int
        L.dense_pack.argtypes = [G, CV, I32, P, P, P, P, P, P, P, SZ, P]
        L.dense_pack.restype = C.c_int
        L.ada_code_error.argtypes = [G, I64, P, P, P, P, P, P, P, P]
        L.ada_code_error.restype = C.c_int
        L.rdr_solve_workspace_size.argtypes = [G, I32, I64]
        L.rdr_solve_workspace_size.restype = SZ
        L.rdr_solve.argtypes = [G, I32, P, P, P, P, P, P, P, P, P, P, SZ, P]
        L.ada_append_state_bytes.argtypes = [G, I32]
        L.ada_append_state_bytes.restype = SZ
        L.ada_append.argtypes = [G, CV, P, P, P, P, P, P, P, P, P, P, P]
        L.ada_append.restype = C.c_int
        L.ada_retier.argtypes = [G, CV, P, P, I32, P, P, P, P, P]
        L.ada_retier.restype = C.c_int
        L.ada_retier_plan.argtypes = [G, I32, P, P, P, I32, I32, I32, P, P, P, P]
        L.ada_retier_plan.restype = C.c_int
        L.rdr_solve.restype = C.c_int
        L.rdr_tier_counts_workspace_size.argtypes = [G, I32]
        L.rdr_tier_counts_workspace_size.restype = SZ
        L.rdr_tier_counts.argtypes = [G, I32, P, P, P, P, SZ, P]
        L.rdr_tier_counts.restype = C.c_int
        L.rdr_pack_tiers_num_pages.argtypes = [G, I32, P, P]
        L.rdr_pack_tiers_num_pages.restype = C.c_int
        L.rdr_pack_tiers.argtypes = [G, CV, I32, P, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P]
        L.rdr_pack_tiers.restype = C.c_int
        L.rdr_pack_tiers_device.argtypes = [G, CV, I32, P, P, P, P, P, P, P, P, P, P, SZ, P]
        L.rdr_pack_tiers_device.restype = C.c_int
        L.ada_decode_default_splits.argtypes = [G, I32, I32]
        L.ada_decode_default_splits.restype = I32
        L.ada_decode_workspace_size.argtypes = [G, I32, I32, I32]
        L.ada_decode_workspace_size.restype = SZ
        L.ada_decode.argtypes = [G, CV, P, P, P, F, P, P, P, I32, P, SZ, P]
        L.ada_decode.restype = C.c_int
        L.dense_decode.argtypes = [G, CV, P, F, P, P, P, I32, P, SZ, P]
        L.dense_decode.restype = C.c_int
        L.ada_decode_stream.argtypes = [G, CV, P, P, P, F, P, P, P, I32, P, SZ, P]
        L.ada_decode_stream.restype = C.c_int
        L.ada_decode_sym.argtypes = [G, CV, P, P, P, F, P, P, P, I32, P, SZ, P]
        L.ada_decode_sym.restype = C.c_int
        L.ada_decode_sym_workspace_size.argtypes = [G, I32, I32, I32]
        L.ada_decode_sym_workspace_size.restype = SZ
        L.ada_decode_noalloc.argtypes = [G, CV, P, P, P, F, P, P, P, I32, P]
        L.ada_decode_noalloc.restype = C.c_int
        L.ada_phase_trace.argtypes = [P, SZ]
        L.ada_phase_trace.restype = C.c_int
        L.ada_decode_merge.argtypes = [G, CV, P, P, P, F, P, P, I32, P, SZ, P]
        L.ada_decode_merge.restype = C.c_int
        _lib = L
    return _lib


def _check(status: int, what: str):
    if status != OK:
        raise AdaError(status, what)


def _dev(t: torch.Tensor | None, name: str, dtypes=None, device=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return C.c_void_p(t.data_ptr())


def _host(a, dtype, name: str):
    if a is None:
        return None, None
    arr = np.ascontiguousarray(a, dtype=dtype)
    return arr, arr.ctypes.data_as(C.c_void_p)


def _stream(stream) -> C.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


def page_bytes(head_dim: int, tier: int) -> int:
    return int(load().ada_page_bytes(head_dim, tier))


class Cache:
    """One layer's paged cache on a device, allocated with torch, plus the
    host-side allocator state (arena cursor, per-row page counts) that pack
    calls advance.  `view()` gives the C struct the library reads."""

    def __init__(self, geom: Geom, num_seqs: int, max_pages_per_head: int, arena_bytes: int,
                 device="cuda", slot_tokens: bool = False):
        self.geom = geom
        self.num_seqs = num_seqs
        self.maxp = max_pages_per_head
        rows = num_seqs * geom.num_kv_heads
        arena_bytes = (arena_bytes + 127) // 128 * 128
        dev = torch.device(device)
        self.arena = torch.zeros(arena_bytes, dtype=torch.uint8, device=dev)
        self.page_table = torch.zeros((rows, max(1, max_pages_per_head)), dtype=torch.int32, device=dev)
        self.page_meta = torch.zeros((rows, max(1, max_pages_per_head)), dtype=torch.uint8, device=dev)
        self.num_pages = torch.zeros(max(1, rows), dtype=torch.int32, device=dev)
        self.tier_tokens = torch.zeros((max(1, rows), 3), dtype=torch.int32, device=dev)
        self.slot_token = (torch.full((rows, max(1, max_pages_per_head), 16), -1, dtype=torch.int32,
                                      device=dev) if slot_tokens else None)
        self.cursor = np.zeros(1, dtype=np.uint64)
        self.num_pages_host = np.zeros(max(1, rows), dtype=np.int32)

    @property
    def arena_units(self) -> int:
        return self.arena.numel() // 128

    def used_bytes(self) -> int:
        return int(self.cursor[0]) * 128

    def view(self, arena: torch.Tensor | None = None) -> _CacheView:
        """C view; `arena` may substitute a same-size copy of the arena
        (same page table), e.g. to rotate copies in a benchmark."""
        ar = self.arena if arena is None else arena
        if ar.numel() != self.arena.numel():
            raise ValueError("substitute arena must have the same size")
        v = _CacheView(ar.data_ptr(), ar.numel() // 128, self.page_table.data_ptr(),
                       self.page_meta.data_ptr(), self.num_pages.data_ptr(),
                       self.tier_tokens.data_ptr(),
                       self.slot_token.data_ptr() if self.slot_token is not None else None,
                       self.num_seqs, self.maxp)
        # the view holds raw device addresses: it keeps the tensors behind
        # them alive for as long as it exists
        v._keep = (ar, self.page_table, self.page_meta, self.num_pages, self.tier_tokens, self.slot_token)
        return v


def encode(geom: Geom, keys, cb8, cb4, radius, codes8, codes4, stream=None):
    """keys [N][Hkv][D] fp16 -> radius [N][Hkv] fp16 bits, codes8 [N][Hkv][G]
    u8, codes4 [N][Hkv][G/2] u8 (outputs preallocated)."""
    n = keys.shape[0]
    H, D = geom.num_kv_heads, geom.head_dim
    if tuple(keys.shape) != (n, H, D):
        raise ValueError(f"keys shape {tuple(keys.shape)} != {(n, H, D)}")
    for t, shape, name in ((radius, (n, H), "radius"), (codes8, (n, H, D // 8), "codes8"),
                           (codes4, (n, H, D // 16), "codes4"),
                           (cb8, (H, D // 8, 256, 8), "cb8"), (cb4, (H, D // 8, 16, 8), "cb4")):
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} shape {tuple(t.shape)} != {shape}")
    st = load().ada_encode(C.byref(geom), n, _dev(keys, "keys", (torch.float16,)),
                           _dev(cb8, "cb8", (torch.float32,)), _dev(cb4, "cb4", (torch.float32,)),
                           _dev(radius, "radius", (torch.float16, torch.int16)),
                           _dev(codes8, "codes8", (torch.uint8,)), _dev(codes4, "codes4", (torch.uint8,)),
                           _stream(stream))
    _check(st, "ada_encode")


def pack_num_pages(geom: Geom, cu_tokens, tier_cum_bp) -> int:
    cu, cup = _host(cu_tokens, np.int32, "cu_tokens")
    bp, bpp = _host(tier_cum_bp, np.int32, "tier_cum_bp")
    out = C.c_int64(0)
    _check(load().rdr_pack_num_pages(C.byref(geom), len(cu) - 1, cup, bpp, C.byref(out)),
           "rdr_pack_num_pages")
    return out.value


def pack_workspace_size(geom: Geom, n_tokens: int, num_seqs: int) -> int:
    return int(load().rdr_pack_workspace_size(C.byref(geom), n_tokens, num_seqs))


def _workspace(nbytes: int, device, stream=None) -> torch.Tensor:
    """A workspace for a call enqueued on `stream` (None = the current
    stream).  It is allocated, and zero-filled, on that stream, so torch's
    caching allocator orders any reuse of its memory after the call even if
    the caller drops the tensor while the call still runs."""
    # (every entry point writes what it reads; zero-filled only so that a
    # workspace never holds stale data from elsewhere)
    if stream is None:
        return torch.zeros(max(256, nbytes), dtype=torch.uint8, device=device)
    with torch.cuda.stream(stream):
        return torch.zeros(max(256, nbytes), dtype=torch.uint8, device=device)


def rdr_pack(geom: Geom, cache: Cache, cu_tokens, tier_cum_bp, keys, values, radius, codes8, codes4,
             scores, protect=None, place_perm=None, pos_base=None, ws=None, stream=None):
    """Appends one call's tokens to `cache` (see rdr_pack in include/ada.h).
    cu_tokens / tier_cum_bp / protect / place_perm / pos_base are host arrays."""
    cu, cup = _host(cu_tokens, np.int32, "cu_tokens")
    bp, bpp = _host(tier_cum_bp, np.int32, "tier_cum_bp")
    n = int(cu[-1])
    pr, prp = _host(protect, np.uint8, "protect")
    pp, ppp = _host(place_perm, np.uint32, "place_perm")
    pb, pbp = _host(pos_base, np.int64, "pos_base")
    if ws is None:
        ws = _workspace(pack_workspace_size(geom, n, len(cu) - 1), cache.arena.device, stream)
    view = cache.view()
    st = load().rdr_pack(
        C.byref(geom), C.byref(view), len(cu) - 1, cup, bpp,
        _dev(keys, "keys", (torch.float16,)), _dev(values, "values", (torch.bfloat16,)),
        _dev(radius, "radius", (torch.float16, torch.int16)), _dev(codes8, "codes8", (torch.uint8,)),
        _dev(codes4, "codes4", (torch.uint8,)), _dev(scores, "scores", (torch.float32,)),
        prp, ppp, pbp, cache.cursor.ctypes.data_as(C.c_void_p),
        cache.num_pages_host.ctypes.data_as(C.c_void_p), _dev(ws, "ws"), ws.numel(), _stream(stream))
    _check(st, "rdr_pack")
    return ws


def code_error(geom: Geom, keys, cb8, cb4, codes8, codes4, err8, err4, stream=None):
    """Squared chord error of each (token, head)'s 8-bit and 4-bit codes:
    err8 / err4 [N][Hkv] f32 (preallocated).  See ada_code_error."""
    n = keys.shape[0]
    H, D = geom.num_kv_heads, geom.head_dim
    for t, shape, name in ((keys, (n, H, D), "keys"), (codes8, (n, H, D // 8), "codes8"),
                           (codes4, (n, H, D // 16), "codes4"), (err8, (n, H), "err8"),
                           (err4, (n, H), "err4"), (cb8, (H, D // 8, 256, 8), "cb8"),
                           (cb4, (H, D // 8, 16, 8), "cb4")):
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} shape {tuple(t.shape)} != {shape}")
    st = load().ada_code_error(C.byref(geom), n, _dev(keys, "keys", (torch.float16,)),
                               _dev(cb8, "cb8", (torch.float32,)), _dev(cb4, "cb4", (torch.float32,)),
                               _dev(codes8, "codes8", (torch.uint8,)), _dev(codes4, "codes4", (torch.uint8,)),
                               _dev(err8, "err8", (torch.float32,)), _dev(err4, "err4", (torch.float32,)),
                               _stream(stream))
    _check(st, "ada_code_error")


def solve_workspace_size(geom: Geom, num_seqs: int, n_tokens: int) -> int:
    return int(load().rdr_solve_workspace_size(C.byref(geom), num_seqs, n_tokens))


def rdr_solve(geom: Geom, cu_tokens, budget_bytes, radius, err8, err4, scores, tiers, protect=None,
              threshold=None, ws=None, stream=None):
    """Tier of every (token, head) under a byte budget per sequence (see
    rdr_solve in include/ada.h).  cu_tokens / budget_bytes are host arrays;
    radius, err8, err4, scores, protect (u8 or None) and tiers (u8 out,
    [N][Hkv]) are device tensors."""
    cu, cup = _host(cu_tokens, np.int32, "cu_tokens")
    bud, budp = _host(budget_bytes, np.int64, "budget_bytes")
    if len(bud) != len(cu) - 1:
        raise ValueError("one budget per sequence")
    n = int(cu[-1])
    H = geom.num_kv_heads
    for t, name in ((radius, "radius"), (err8, "err8"), (err4, "err4"), (scores, "scores"),
                    (tiers, "tiers")) + (((protect, "protect"),) if protect is not None else ()):
        if tuple(t.shape) != (n, H):
            raise ValueError(f"{name} shape {tuple(t.shape)} != {(n, H)}")
    if ws is None:
        ws = _workspace(solve_workspace_size(geom, len(cu) - 1, n), tiers.device, stream)
    st = load().rdr_solve(C.byref(geom), len(cu) - 1, cup, budp,
                          _dev(radius, "radius", (torch.float16, torch.int16)),
                          _dev(err8, "err8", (torch.float32,)), _dev(err4, "err4", (torch.float32,)),
                          _dev(scores, "scores", (torch.float32,)), _dev(protect, "protect", (torch.uint8,)),
                          _dev(tiers, "tiers", (torch.uint8,)), _dev(threshold, "threshold", (torch.float32,)),
                          _dev(ws, "ws"), ws.numel(), _stream(stream))
    _check(st, "rdr_solve")
    return ws


class AppendState:
    """Device state of the decode-step append (ada_append) for one cache:
    the arena cursor, sticky status bits and each row's open pages."""

    def __init__(self, geom: Geom, cache: "Cache"):
        n = int(load().ada_append_state_bytes(C.byref(geom), cache.num_seqs))
        self.buf = torch.zeros(n, dtype=torch.uint8, device=cache.arena.device)
        self.cache = cache
        self.push_cursor()

    def push_cursor(self, stream=None):
        """Host cursor -> device (before appending after host-planned packs),
        ordered on `stream` (None = the current stream)."""
        src = torch.from_numpy(self.cache.cursor.view(np.uint8).copy())
        with torch.cuda.stream(torch.cuda.current_stream() if stream is None else stream):
            self.buf[:8].copy_(src)

    def pull(self, stream=None) -> int:
        """Device cursor and page counts -> the cache's host copies (before a
        host-planned pack), after the work enqueued on `stream` (None = the
        current stream); returns the status bits.  Synchronizes that stream."""
        with torch.cuda.stream(torch.cuda.current_stream() if stream is None else stream):
            c = self.buf[:16].cpu().numpy()
            rows = self.cache.num_pages_host.shape[0]
            npg = self.cache.num_pages[:rows].cpu().numpy()
        self.cache.cursor[:] = c[:8].view(np.uint64)
        self.cache.num_pages_host[:] = npg
        return int(c[8:12].view(np.uint32)[0])


def append(geom: Geom, cache: Cache, state: AppendState, cb8, cb4, keys, values, scores, threshold, pos,
           protect=None, tiers=None, stream=None):
    """One decode step's append (ada_append): keys / values [S][Hkv][D],
    scores [S][Hkv], threshold f32 [S], pos int64 [S], all device tensors."""
    S, H, D = cache.num_seqs, geom.num_kv_heads, geom.head_dim
    for t, shape, name in ((keys, (S, H, D), "keys"), (values, (S, H, D), "values"), (scores, (S, H), "scores"),
                           (threshold, (S,), "threshold"), (pos, (S,), "pos")):
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} shape {tuple(t.shape)} != {shape}")
    view = cache.view()
    st = load().ada_append(C.byref(geom), C.byref(view), _dev(cb8, "cb8", (torch.float32,)),
                           _dev(cb4, "cb4", (torch.float32,)), _dev(keys, "keys", (torch.float16,)),
                           _dev(values, "values", (torch.bfloat16,)), _dev(scores, "scores", (torch.float32,)),
                           _dev(protect, "protect", (torch.uint8,)), _dev(threshold, "threshold", (torch.float32,)),
                           _dev(pos, "pos", (torch.int64,)), _dev(tiers, "tiers", (torch.uint8,)),
                           _dev(state.buf, "state"), _stream(stream))
    _check(st, "ada_append")


def retier(geom: Geom, cache: Cache, state: AppendState, cb8, cb4, rows, pages, target, stream=None):
    """Demote (target 1 / 2) or evict (3) listed pages in place (ada_retier).
    rows / pages int32 and target uint8 are device tensors of one length."""
    n = int(rows.numel())
    if pages.numel() != n or target.numel() != n:
        raise ValueError("rows, pages and target must have one length")
    view = cache.view()
    st = load().ada_retier(C.byref(geom), C.byref(view), _dev(cb8, "cb8", (torch.float32,)),
                           _dev(cb4, "cb4", (torch.float32,)), n, _dev(rows, "rows", (torch.int32,)),
                           _dev(pages, "pages", (torch.int32,)), _dev(target, "target", (torch.uint8,)),
                           _dev(state.buf, "state"), _stream(stream))
    _check(st, "ada_retier")


def retier_plan(geom: Geom, budget_bytes, num_pages_host, page_meta_host, demote_to: int = 2,
                cap: int = 1 << 20):
    """The age-ordered re-tiering policy (ada_retier_plan) on host copies of
    the tables: (rows, pages, target) numpy arrays."""
    bud, budp = _host(budget_bytes, np.int64, "budget_bytes")
    npg, npgp = _host(num_pages_host, np.int32, "num_pages")
    pm, pmp = _host(page_meta_host, np.uint8, "page_meta")
    rows = np.zeros(cap, np.int32)
    pages = np.zeros(cap, np.int32)
    tgt = np.zeros(cap, np.uint8)
    n = C.c_int32(0)
    _check(load().ada_retier_plan(C.byref(geom), len(bud), budp, npgp, pmp, pm.shape[1], demote_to, cap,
                                  rows.ctypes.data_as(C.c_void_p), pages.ctypes.data_as(C.c_void_p),
                                  tgt.ctypes.data_as(C.c_void_p), C.byref(n)), "ada_retier_plan")
    return rows[:n.value], pages[:n.value], tgt[:n.value]


def tier_counts(geom: Geom, cu_tokens, tiers, stream=None) -> np.ndarray:
    """Tokens of tier 0, 1, 2 per row: int32 [S*Hkv][3] on the host
    (synchronizes the stream)."""
    cu, cup = _host(cu_tokens, np.int32, "cu_tokens")
    S = len(cu) - 1
    # page-locked result buffer (from torch's caching host allocator): the
    # device-to-host copy then needs no staging
    out = torch.zeros((max(1, S * geom.num_kv_heads), 3), dtype=torch.int32, pin_memory=True)
    ws = _workspace(int(load().rdr_tier_counts_workspace_size(C.byref(geom), S)), tiers.device, stream)
    st = load().rdr_tier_counts(C.byref(geom), S, cup, _dev(tiers, "tiers", (torch.uint8,)),
                                C.c_void_p(out.data_ptr()), _dev(ws, "ws"), ws.numel(), _stream(stream))
    _check(st, "rdr_tier_counts")
    return out.numpy()[: S * geom.num_kv_heads].copy()


def pack_tiers_num_pages(geom: Geom, row_counts) -> int:
    rc, rcp = _host(row_counts, np.int32, "row_counts")
    out = C.c_int64(0)
    _check(load().rdr_pack_tiers_num_pages(C.byref(geom), rc.shape[0] // max(1, geom.num_kv_heads), rcp,
                                           C.byref(out)), "rdr_pack_tiers_num_pages")
    return out.value


def rdr_pack_tiers(geom: Geom, cache: Cache, cu_tokens, row_counts, tiers, keys, values, radius, codes8,
                   codes4, place_perm=None, pos_base=None, ws=None, stream=None):
    """rdr_pack with the tier of every (token, head) given (see rdr_pack_tiers
    in include/ada.h).  row_counts = tier_counts(geom, cu_tokens, tiers)."""
    cu, cup = _host(cu_tokens, np.int32, "cu_tokens")
    rc, rcp = _host(row_counts, np.int32, "row_counts")
    n = int(cu[-1])
    if rc.shape != ((len(cu) - 1) * geom.num_kv_heads, 3):
        raise ValueError("row_counts must be [S*Hkv][3]")
    pp, ppp = _host(place_perm, np.uint32, "place_perm")
    pb, pbp = _host(pos_base, np.int64, "pos_base")
    if ws is None:
        ws = _workspace(pack_workspace_size(geom, n, len(cu) - 1), cache.arena.device, stream)
    view = cache.view()
    st = load().rdr_pack_tiers(
        C.byref(geom), C.byref(view), len(cu) - 1, cup, rcp, _dev(tiers, "tiers", (torch.uint8,)),
        _dev(keys, "keys", (torch.float16,)), _dev(values, "values", (torch.bfloat16,)),
        _dev(radius, "radius", (torch.float16, torch.int16)), _dev(codes8, "codes8", (torch.uint8,)),
        _dev(codes4, "codes4", (torch.uint8,)), ppp, pbp, cache.cursor.ctypes.data_as(C.c_void_p),
        cache.num_pages_host.ctypes.data_as(C.c_void_p), _dev(ws, "ws"), ws.numel(), _stream(stream))
    _check(st, "rdr_pack_tiers")
    return ws


def rdr_pack_tiers_device(geom: Geom, cache: Cache, state: "AppendState", cu_tokens, tiers, keys, values,
                          radius, codes8, codes4, pos_base=None, ws=None, stream=None):
    """rdr_pack_tiers with the page plan made on the device (see
    rdr_pack_tiers_device in include/ada.h): no tier counts on the host and
    no synchronization.  The arena space comes from `state`'s device cursor;
    call state.pull() before the next host-planned pack."""
    cu, cup = _host(cu_tokens, np.int32, "cu_tokens")
    n = int(cu[-1])
    pb, pbp = _host(pos_base, np.int64, "pos_base")
    if ws is None:
        ws = _workspace(pack_workspace_size(geom, n, len(cu) - 1), cache.arena.device, stream)
    view = cache.view()
    st = load().rdr_pack_tiers_device(
        C.byref(geom), C.byref(view), len(cu) - 1, cup, _dev(tiers, "tiers", (torch.uint8,)),
        _dev(keys, "keys", (torch.float16,)), _dev(values, "values", (torch.bfloat16,)),
        _dev(radius, "radius", (torch.float16, torch.int16)), _dev(codes8, "codes8", (torch.uint8,)),
        _dev(codes4, "codes4", (torch.uint8,)), pbp, _dev(state.buf, "state"), _dev(ws, "ws"), ws.numel(),
        _stream(stream))
    _check(st, "rdr_pack_tiers_device")
    return ws


def dense_pack(geom: Geom, cache: Cache, cu_tokens, keys, values, place_perm=None, ws=None, stream=None):
    cu, cup = _host(cu_tokens, np.int32, "cu_tokens")
    n = int(cu[-1])
    pp, ppp = _host(place_perm, np.uint32, "place_perm")
    if ws is None:
        ws = _workspace(pack_workspace_size(geom, n, len(cu) - 1), cache.arena.device, stream)
    view = cache.view()
    st = load().dense_pack(C.byref(geom), C.byref(view), len(cu) - 1, cup,
                           _dev(keys, "keys", (torch.float16,)), _dev(values, "values", (torch.bfloat16,)),
                           ppp, cache.cursor.ctypes.data_as(C.c_void_p),
                           cache.num_pages_host.ctypes.data_as(C.c_void_p), _dev(ws, "ws"), ws.numel(),
                           _stream(stream))
    _check(st, "dense_pack")
    return ws


def decode_default_splits(geom: Geom, num_seqs: int, max_pages_per_head: int) -> int:
    return int(load().ada_decode_default_splits(C.byref(geom), num_seqs, max_pages_per_head))


def decode_workspace_size(geom: Geom, num_seqs: int, max_pages_per_head: int, num_splits: int = 0) -> int:
    return int(load().ada_decode_workspace_size(C.byref(geom), num_seqs, max_pages_per_head, num_splits))


def _decode_shapes(geom, cache, q, out, lse, logits):
    S, Hq, D = cache.num_seqs, geom.num_q_heads, geom.head_dim
    if tuple(q.shape) != (S, Hq, D) or tuple(out.shape) != (S, Hq, D):
        raise ValueError("q and out must be [S][Hq][D]")
    if lse is not None and tuple(lse.shape) != (S, Hq):
        raise ValueError("lse must be [S][Hq]")
    if logits is not None and tuple(logits.shape) != (S, Hq, cache.maxp * 16):
        raise ValueError("logits must be [S][Hq][max_pages_per_head*16]")


def _decode_args(geom, cache, q, out, lse, logits, ws, num_splits, stream=None):
    _decode_shapes(geom, cache, q, out, lse, logits)
    S = cache.num_seqs
    if ws is None:
        ws = _workspace(decode_workspace_size(geom, S, cache.maxp, num_splits), q.device, stream)
    return ws


def decode(geom: Geom, cache: Cache, cb8, cb4, q, softmax_scale: float, out, lse=None, logits=None,
           num_splits: int = 0, ws=None, stream=None, view=None):
    """One ADA decode step (ada_decode).  `view` may pass a prebuilt
    cache.view(...) (e.g. with a rotated arena)."""
    ws = _decode_args(geom, cache, q, out, lse, logits, ws, num_splits, stream)
    v = cache.view() if view is None else view
    st = load().ada_decode(C.byref(geom), C.byref(v), _dev(cb8, "cb8", (torch.float32,)),
                           _dev(cb4, "cb4", (torch.float32,)), _dev(q, "q", (torch.bfloat16,)),
                           float(softmax_scale), _dev(out, "out", (torch.float32,)),
                           _dev(lse, "lse", (torch.float32,)), _dev(logits, "logits", (torch.float32,)),
                           num_splits, _dev(ws, "ws"), ws.numel(), _stream(stream))
    _check(st, "ada_decode")
    return ws


def phase_trace(buf: torch.Tensor | None):
    """ada_phase_trace: decode calls record per-wave phase timestamps into
    buf (a device tensor the caller keeps alive; None stops).  Only the
    tracing build records them; any other raises AdaError(EUNSUPPORTED)."""
    if buf is None:
        _check(load().ada_phase_trace(None, 0), "ada_phase_trace")
        return
    _check(load().ada_phase_trace(_dev(buf, "buf"), buf.numel() * buf.element_size()), "ada_phase_trace")


def decode_noalloc(geom: Geom, cache: Cache, cb8, cb4, q, softmax_scale: float, out, lse=None, logits=None,
                   num_splits: int = 0, stream=None, view=None):
    """ada_decode_noalloc: one decode step that allocates nothing (the split
    partials live in the library's own device array; overlapping calls on
    one GPU race)."""
    _decode_shapes(geom, cache, q, out, lse, logits)
    v = cache.view() if view is None else view
    st = load().ada_decode_noalloc(C.byref(geom), C.byref(v), _dev(cb8, "cb8", (torch.float32,)),
                                   _dev(cb4, "cb4", (torch.float32,)), _dev(q, "q", (torch.bfloat16,)),
                                   float(softmax_scale), _dev(out, "out", (torch.float32,)),
                                   _dev(lse, "lse", (torch.float32,)), _dev(logits, "logits", (torch.float32,)),
                                   num_splits, _stream(stream))
    _check(st, "ada_decode_noalloc")


def decode_sym_workspace_size(geom: Geom, num_seqs: int, max_pages_per_head: int, num_splits: int = 0) -> int:
    return int(load().ada_decode_sym_workspace_size(C.byref(geom), num_seqs, max_pages_per_head, num_splits))


def decode_sym(geom: Geom, cache: Cache, cb8, cb4, q, softmax_scale: float, out, lse=None, logits=None,
               num_splits: int = 0, ws=None, stream=None, view=None):
    """One decode step with the symmetric angle-code logit (ada_decode_sym)."""
    if ws is None:
        ws = _workspace(decode_sym_workspace_size(geom, cache.num_seqs, cache.maxp, num_splits), q.device,
                        stream)
    ws = _decode_args(geom, cache, q, out, lse, logits, ws, num_splits, stream)
    v = cache.view() if view is None else view
    st = load().ada_decode_sym(C.byref(geom), C.byref(v), _dev(cb8, "cb8", (torch.float32,)),
                               _dev(cb4, "cb4", (torch.float32,)), _dev(q, "q", (torch.bfloat16,)),
                               float(softmax_scale), _dev(out, "out", (torch.float32,)),
                               _dev(lse, "lse", (torch.float32,)), _dev(logits, "logits", (torch.float32,)),
                               num_splits, _dev(ws, "ws"), ws.numel(), _stream(stream))
    _check(st, "ada_decode_sym")
    return ws


def decode_stage(stage: str, geom: Geom, cache: Cache, cb8, cb4, q, softmax_scale: float, out,
                 lse=None, logits=None, num_splits: int = 0, ws=None, stream=None, view=None):
    """One stage of ada_decode: "stream" or "merge" (ada_decode_stream /
    ada_decode_merge).  The stages share `ws`."""
    ws = _decode_args(geom, cache, q, out, lse, logits, ws, num_splits, stream)
    v = cache.view() if view is None else view
    L = load()
    g, cv = C.byref(geom), C.byref(v)
    c8, c4 = _dev(cb8, "cb8", (torch.float32,)), _dev(cb4, "cb4", (torch.float32,))
    qq, oo = _dev(q, "q", (torch.bfloat16,)), _dev(out, "out", (torch.float32,))
    ll = _dev(lse, "lse", (torch.float32,))
    if stage == "stream":
        st = L.ada_decode_stream(g, cv, c8, c4, qq, float(softmax_scale), oo, ll,
                                 _dev(logits, "logits", (torch.float32,)), num_splits, _dev(ws, "ws"),
                                 ws.numel(), _stream(stream))
    elif stage == "merge":
        st = L.ada_decode_merge(g, cv, c8, c4, qq, float(softmax_scale), oo, ll, num_splits, _dev(ws, "ws"),
                                ws.numel(), _stream(stream))
    else:
        raise ValueError(f"unknown decode stage {stage!r}")
    _check(st, f"ada_decode_{stage}")
    return ws


def dense_decode(geom: Geom, cache: Cache, q, softmax_scale: float, out, lse=None, logits=None,
                 num_splits: int = 0, ws=None, stream=None, view=None):
    ws = _decode_args(geom, cache, q, out, lse, logits, ws, num_splits, stream)
    v = cache.view() if view is None else view
    st = load().dense_decode(C.byref(geom), C.byref(v), _dev(q, "q", (torch.bfloat16,)),
                             float(softmax_scale), _dev(out, "out", (torch.float32,)),
                             _dev(lse, "lse", (torch.float32,)), _dev(logits, "logits", (torch.float32,)),
                             num_splits, _dev(ws, "ws"), ws.numel(), _stream(stream))
    _check(st, "dense_decode")
    return ws
