"""CPU oracle for the ADA decode path -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package.  The product (compressed_kv_attention_amd) never does, and it
shares no code with this package.

The arithmetic lives in oracle.c (plain C, double precision); this file only
builds it with gcc, loads it with ctypes and marshals numpy arrays.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

UNIT = 128
SLOTS = 16


def build() -> str:
    """Compile oracle.c into liboracle.so (IEEE arithmetic: no fast-math, no
    contraction of multiply-add)."""
    cmd = ["gcc", "-O2", "-std=c99", "-D_GNU_SOURCE", "-Wall", "-ffp-contract=off",
           "-fno-fast-math", "-fPIC", "-shared", "-o", _LIB + ".tmp", _SRC, "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = C.CDLL(_LIB)
        P, I, I64, U64, D_, SZ = C.c_void_p, C.c_int, C.c_int64, C.c_uint64, C.c_double, C.c_size_t
        L.oracle_page_bytes.argtypes = [I, I]
        L.oracle_page_bytes.restype = SZ
        L.oracle_encode.argtypes = [I, I, I64, P, P, P, P, P, P, P, P, I]
        L.oracle_encode.restype = I
        L.oracle_tier_counts.argtypes = [I64, P, P]
        L.oracle_pack.argtypes = [I, I, I, P, P, P, P, P, P, P, P, P, P, P, P, U64, P, P, P, P,
                                  P, P, I]
        L.oracle_pack.restype = I
        L.oracle_code_error.argtypes = [I, I, I64, P, P, P, P, P, P, P]
        L.oracle_code_error.restype = I
        L.oracle_rdr_solve.argtypes = [I, I, I, P, P, P, P, P, P, P, P, P]
        L.oracle_rdr_solve.restype = I
        L.oracle_pack_tiers.argtypes = [I, I, I, P, P, P, P, P, P, P, P, P, P, U64, P, P, P, P, P,
                                        P, I]
        L.oracle_pack_tiers.restype = I
        L.oracle_append.argtypes = [I, I, I, P, P, P, P, P, P, P, P, P, U64, P, P, P, P, P, P, I, P, P, P]
        L.oracle_append.restype = I
        L.oracle_retier.argtypes = [I, I, I, I, P, P, P, P, P, P, U64, P, P, P, P, P, P, I, P, P]
        L.oracle_retier.restype = I
        L.oracle_retier_plan.argtypes = [I, I, I, P, P, P, I, I, I, P, P, P]
        L.oracle_retier_plan.restype = I
        L.oracle_dense_pack.argtypes = [I, I, I, P, P, P, P, P, U64, P, P, P, P, I]
        L.oracle_dense_pack.restype = I
        L.oracle_decode.argtypes = [I, I, I, I, I, P, P, P, P, P, P, P, D_, P, P, P, P, I64, I64, I]
        L.oracle_decode.restype = I
        L.oracle_decode_sym.argtypes = L.oracle_decode.argtypes
        L.oracle_decode_sym.restype = I
        L.oracle_query_codes.argtypes = [I, I, I, I, P, P, P, P, P, P]
        L.oracle_query_codes.restype = I
        L.oracle_dense_attention.argtypes = [I, I64, P, P, P, D_, P, P]
        L.oracle_f16_to_double.argtypes = [C.c_uint16]
        L.oracle_f16_to_double.restype = D_
        L.oracle_double_to_f16.argtypes = [D_]
        L.oracle_double_to_f16.restype = C.c_uint16
        L.oracle_bf16_to_double.argtypes = [C.c_uint16]
        L.oracle_bf16_to_double.restype = D_
        L.oracle_double_to_bf16.argtypes = [D_]
        L.oracle_double_to_bf16.restype = C.c_uint16
        L.oracle_quant_v.argtypes = [I, P, P, P]
        for f in (L.oracle_row_off, L.oracle_col_off, L.oracle_col8_off):
            f.argtypes = [I, I]
            f.restype = SZ
        _lib = L
    return _lib


def _u16(x) -> np.ndarray:
    """fp16 / bf16 data (torch tensor or numpy array) -> contiguous uint16 bits."""
    if hasattr(x, "detach"):
        import torch
        x = x.detach().cpu().contiguous()
        if x.dtype in (torch.float16, torch.bfloat16):
            return x.view(torch.int16).numpy().view(np.uint16)
        return np.ascontiguousarray(x.numpy())
    x = np.ascontiguousarray(x)
    if x.dtype == np.float16:
        return x.view(np.uint16)
    return x.astype(np.uint16, copy=False)


def _np(x, dtype) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().cpu().contiguous().numpy()
    return np.ascontiguousarray(x, dtype=dtype)


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def page_bytes(D: int, tier: int) -> int:
    return int(lib().oracle_page_bytes(D, tier))


def f16_to_double(h: int) -> float:
    return lib().oracle_f16_to_double(h)


def double_to_f16(x: float) -> int:
    return lib().oracle_double_to_f16(x)


def bf16_to_double(b: int) -> float:
    return lib().oracle_bf16_to_double(b)


def double_to_bf16(x: float) -> int:
    return lib().oracle_double_to_bf16(x)


def row_off(t, d) -> int:
    return int(lib().oracle_row_off(t, d))


def col_off(t, d) -> int:
    return int(lib().oracle_col_off(t, d))


def col8_off(t, d) -> int:
    return int(lib().oracle_col8_off(t, d))


def quant_v(v_bf16) -> tuple[np.ndarray, int]:
    v = _u16(v_bf16)
    D = v.shape[-1]
    q = np.zeros(D, dtype=np.int8)
    sc = np.zeros(1, dtype=np.uint16)
    lib().oracle_quant_v(D, _p(v), _p(q), _p(sc))
    return q, int(sc[0])


def tier_counts(T: int, bp) -> np.ndarray:
    bp = np.ascontiguousarray(bp, dtype=np.int32)
    out = np.zeros(3, dtype=np.int64)
    lib().oracle_tier_counts(int(T), _p(bp), _p(out))
    return out


def encode(keys, cb8, cb4, with_dist: bool = False, nthreads: int = 1):
    """keys [N][Hkv][D] fp16 -> (radius u16 [N][Hkv], codes8 [N][Hkv][G],
    codes4 [N][Hkv][G/2]) (+ dist8, dist4 when with_dist)."""
    k = _u16(keys)
    N, H, D = k.shape
    G = D // 8
    c8, c4 = _np(cb8, np.float32), _np(cb4, np.float32)
    assert c8.shape == (H, G, 256, 8) and c4.shape == (H, G, 16, 8)
    r = np.zeros((N, H), dtype=np.uint16)
    k8 = np.zeros((N, H, G), dtype=np.uint8)
    k4 = np.zeros((N, H, G // 2), dtype=np.uint8)
    d8 = np.zeros((N, H, G, 256)) if with_dist else None
    d4 = np.zeros((N, H, G, 16)) if with_dist else None
    rc = lib().oracle_encode(D, H, N, _p(k), _p(c8), _p(c4), _p(r), _p(k8), _p(k4), _p(d8), _p(d4),
                             nthreads)
    assert rc == 0
    return (r, k8, k4, d8, d4) if with_dist else (r, k8, k4)


class HostCache:
    """A cache view in host memory, in the same format the library uses."""

    def __init__(self, D, Hkv, S, maxp, arena_bytes, slot_tokens=True):
        self.D, self.Hkv, self.S, self.maxp = D, Hkv, S, maxp
        self.arena = np.zeros(arena_bytes, dtype=np.uint8)
        self.arena_units = arena_bytes // UNIT
        self.cursor = np.zeros(1, dtype=np.uint64)
        self.page_table = np.zeros((S * Hkv, maxp), dtype=np.uint32)
        self.page_meta = np.zeros((S * Hkv, maxp), dtype=np.uint8)
        self.num_pages = np.zeros(S * Hkv, dtype=np.int32)
        self.tier_tokens = np.zeros((S * Hkv, 3), dtype=np.int32)
        self.slot_token = np.full((S * Hkv, maxp, SLOTS), -1, dtype=np.int32) if slot_tokens else None

    def page(self, row, p) -> np.ndarray:
        off = int(self.page_table[row, p]) * UNIT
        tier = int(self.page_meta[row, p]) & 3
        return self.arena[off: off + page_bytes(self.D, tier)]


def pack(cache: HostCache, cu_tokens, tier_cum_bp, keys, values, radius, codes8, codes4, scores,
         protect=None, place_perm=None, pos_base=None) -> int:
    """Append one call's tokens to `cache` (in place).  Returns the status
    (0 ok, 1 invalid, 3 no arena space)."""
    cu = _np(cu_tokens, np.int32)
    bp = _np(tier_cum_bp, np.int32)
    k, v = _u16(keys), _u16(values)
    r = _u16(radius)
    c8, c4 = _np(codes8, np.uint8), _np(codes4, np.uint8)
    sc = _np(scores, np.float32)
    pr = None if protect is None else _np(protect, np.uint8)
    pp = None if place_perm is None else _np(place_perm, np.uint32)
    pb = None if pos_base is None else _np(pos_base, np.int64)
    S = len(cu) - 1
    assert S == cache.S
    return lib().oracle_pack(cache.D, cache.Hkv, S, _p(cu), _p(bp), _p(k), _p(v), _p(r), _p(c8),
                             _p(c4), _p(sc), _p(pr), _p(pp), _p(pb), _p(cache.arena),
                             cache.arena_units, _p(cache.cursor), _p(cache.page_table),
                             _p(cache.page_meta), _p(cache.num_pages), _p(cache.tier_tokens),
                             _p(cache.slot_token), cache.maxp)


def code_error(keys, cb8, cb4, codes8, codes4):
    """Squared chord error of each (token, head)'s 8-bit and 4-bit code
    reconstruction: (err8, err4) f32 [N][Hkv]."""
    k = _u16(keys)
    N, H, D = k.shape
    c8, c4 = _np(cb8, np.float32), _np(cb4, np.float32)
    k8, k4 = _np(codes8, np.uint8), _np(codes4, np.uint8)
    e8 = np.zeros((N, H), dtype=np.float32)
    e4 = np.zeros((N, H), dtype=np.float32)
    rc = lib().oracle_code_error(D, H, N, _p(k), _p(c8), _p(c4), _p(k8), _p(k4), _p(e8), _p(e4))
    assert rc == 0
    return e8, e4


def rdr_solve(D, cu_tokens, budget_bytes, radius, err8, err4, scores, protect=None, with_threshold=False):
    """Tier of every (token, head) under a per-sequence byte budget:
    u8 [N][Hkv], 0-2 kept tier, 3 dropped (and each sequence's slope
    threshold s*, f32 [S], when with_threshold)."""
    cu = _np(cu_tokens, np.int32)
    bud = _np(budget_bytes, np.int64)
    r = _u16(radius)
    N, H = r.shape
    e8, e4 = _np(err8, np.float32), _np(err4, np.float32)
    sc = _np(scores, np.float32)
    pr = None if protect is None else _np(protect, np.uint8)
    t = np.zeros((N, H), dtype=np.uint8)
    th = np.zeros(len(cu) - 1, dtype=np.float32)
    rc = lib().oracle_rdr_solve(D, H, len(cu) - 1, _p(cu), _p(bud), _p(r), _p(e8), _p(e4), _p(sc),
                                _p(pr), _p(t), _p(th))
    assert rc == 0, rc
    return (t, th) if with_threshold else t


def pack_tiers(cache: HostCache, cu_tokens, tiers, keys, values, radius, codes8, codes4,
               place_perm=None, pos_base=None) -> int:
    """pack() with the tier of every (token, head) given (0-2 kept, 3 dropped)."""
    cu = _np(cu_tokens, np.int32)
    t = _np(tiers, np.uint8)
    k, v = _u16(keys), _u16(values)
    r = _u16(radius)
    c8, c4 = _np(codes8, np.uint8), _np(codes4, np.uint8)
    pp = None if place_perm is None else _np(place_perm, np.uint32)
    pb = None if pos_base is None else _np(pos_base, np.int64)
    S = len(cu) - 1
    assert S == cache.S
    return lib().oracle_pack_tiers(cache.D, cache.Hkv, S, _p(cu), _p(t), _p(k), _p(v), _p(r),
                                   _p(c8), _p(c4), _p(pp), _p(pb), _p(cache.arena),
                                   cache.arena_units, _p(cache.cursor), _p(cache.page_table),
                                   _p(cache.page_meta), _p(cache.num_pages),
                                   _p(cache.tier_tokens), _p(cache.slot_token), cache.maxp)


def append(cache: HostCache, keys, values, scores, cb8, cb4, threshold, pos, open_page, protect=None):
    """One decode-step append: one new token per sequence (keys fp16 /
    values bf16 [S][Hkv][D], scores f32 [S][Hkv], threshold f32 [S], pos
    int64 [S]); open_page int32 [S*Hkv][3] is updated in place.  Returns
    (tiers u8 [S][Hkv], status bits)."""
    k, v = _u16(keys), _u16(values)
    S, H, D = k.shape
    sc = _np(scores, np.float32)
    c8, c4 = _np(cb8, np.float32), _np(cb4, np.float32)
    th = _np(threshold, np.float32)
    ps = _np(pos, np.int64)
    pr = None if protect is None else _np(protect, np.uint8)
    assert open_page.dtype == np.int32 and open_page.shape == (S * H, 3) and open_page.flags.c_contiguous
    tiers = np.zeros((S, H), np.uint8)
    status = np.zeros(1, np.int32)
    rc = lib().oracle_append(D, H, S, _p(k), _p(v), _p(sc), _p(pr), _p(c8), _p(c4), _p(th), _p(ps),
                             _p(cache.arena), cache.arena_units, _p(cache.cursor), _p(cache.page_table),
                             _p(cache.page_meta), _p(cache.num_pages), _p(cache.tier_tokens),
                             _p(cache.slot_token), cache.maxp, _p(open_page), _p(tiers), _p(status))
    assert rc == 0
    return tiers, int(status[0])


def retier(cache: HostCache, cb8, cb4, rows, pages, target, open_page) -> int:
    """Demote (target 1 / 2) or evict (3) the listed pages in place; returns
    the status bits.  open_page int32 [S*Hkv][3] is updated in place."""
    r = np.ascontiguousarray(rows, np.int32)
    p = np.ascontiguousarray(pages, np.int32)
    t = np.ascontiguousarray(target, np.uint8)
    c8, c4 = _np(cb8, np.float32), _np(cb4, np.float32)
    status = np.zeros(1, np.int32)
    rc = lib().oracle_retier(cache.D, cache.Hkv, cache.S, len(r), _p(r), _p(p), _p(t), _p(c8), _p(c4), _p(cache.arena),
                             cache.arena_units, _p(cache.cursor), _p(cache.page_table), _p(cache.page_meta),
                             _p(cache.num_pages), _p(cache.tier_tokens), _p(cache.slot_token), cache.maxp,
                             _p(open_page), _p(status))
    assert rc == 0
    return int(status[0])


def retier_plan(cache: HostCache, budget_bytes, demote_to=2, cap=1 << 20):
    """The re-tiering policy: (rows, pages, target) arrays."""
    bud = np.ascontiguousarray(budget_bytes, np.int64)
    rows = np.zeros(cap, np.int32)
    pages = np.zeros(cap, np.int32)
    tgt = np.zeros(cap, np.uint8)
    n = lib().oracle_retier_plan(cache.D, cache.Hkv, cache.S, _p(bud), _p(cache.num_pages), _p(cache.page_meta),
                                 cache.maxp, demote_to, cap, _p(rows), _p(pages), _p(tgt))
    return rows[:n], pages[:n], tgt[:n]


def row_tier_counts(cu_tokens, tiers) -> np.ndarray:
    """Tokens of each kept tier per (sequence, head) row: int32 [S*Hkv][3]."""
    cu = np.asarray(cu_tokens)
    t = np.asarray(tiers)
    H = t.shape[1]
    out = np.zeros((len(cu) - 1, H, 3), dtype=np.int32)
    for s in range(len(cu) - 1):
        seg = t[cu[s]:cu[s + 1]]
        for k in range(3):
            out[s, :, k] = (seg == k).sum(axis=0)
    return out.reshape(-1, 3)


def dense_pack(cache: HostCache, cu_tokens, keys, values, place_perm=None) -> int:
    cu = _np(cu_tokens, np.int32)
    k, v = _u16(keys), _u16(values)
    pp = None if place_perm is None else _np(place_perm, np.uint32)
    return lib().oracle_dense_pack(cache.D, cache.Hkv, len(cu) - 1, _p(cu), _p(k), _p(v), _p(pp),
                                   _p(cache.arena), cache.arena_units, _p(cache.cursor),
                                   _p(cache.page_table), _p(cache.page_meta),
                                   _p(cache.num_pages), cache.maxp)


def decode(cache: HostCache, cb8, cb4, q, sigma, units=None, logits=False, nthreads=1, sym=False):
    """One decode step.  q [S][Hq][D] bf16.  Returns dict(out [S][Hq][D],
    lse [S][Hq]) (+ logits, logits_explicit [S][Hq][maxp*16], NaN where no
    retained slot) in double.  `units` = (begin, end) range of s*Hq + hq.
    sym: the symmetric variant (the query's direction quantized too)."""
    qq = _u16(q)
    S, Hq, D = qq.shape
    c8 = _np(cb8, np.float32) if cb8 is not None else np.zeros((cache.Hkv, D // 8, 256, 8), np.float32)
    c4 = _np(cb4, np.float32) if cb4 is not None else np.zeros((cache.Hkv, D // 8, 16, 8), np.float32)
    out = np.zeros((S, Hq, D))
    lse = np.full((S, Hq), np.nan)
    lg = np.full((S, Hq, cache.maxp * SLOTS), np.nan) if logits else None
    lx = np.full((S, Hq, cache.maxp * SLOTS), np.nan) if logits else None
    b, e = units if units is not None else (0, S * Hq)
    fn = lib().oracle_decode_sym if sym else lib().oracle_decode
    rc = fn(D, Hq, cache.Hkv, S, cache.maxp, _p(cache.arena), _p(cache.page_table),
            _p(cache.page_meta), _p(cache.num_pages), _p(c8), _p(c4), _p(qq), float(sigma), _p(out),
            _p(lse), _p(lg), _p(lx), b, e, nthreads)
    assert rc == 0
    res = {"out": out, "lse": lse}
    if logits:
        res["logits"], res["logits_explicit"] = lg, lx
    return res


def query_codes(q, cb8, cb4):
    """Symmetric variant: the query codes (qc8, qc4 int32 [S][Hq][G]) and
    |q| [S][Hq] of every (sequence, q-head)."""
    qq = _u16(q)
    S, Hq, D = qq.shape
    c8, c4 = _np(cb8, np.float32), _np(cb4, np.float32)
    Hkv = c8.shape[0]
    qc8 = np.zeros((S, Hq, D // 8), np.int32)
    qc4 = np.zeros((S, Hq, D // 8), np.int32)
    qn = np.zeros((S, Hq))
    assert lib().oracle_query_codes(D, Hq, Hkv, S, _p(qq), _p(c8), _p(c4), _p(qc8), _p(qc4), _p(qn)) == 0
    return qc8, qc4, qn


def dense_attention(q, K, V, sigma):
    """softmax(sigma q K^T) V for one query over explicit rows, in double."""
    q = np.ascontiguousarray(q, dtype=np.float64)
    K = np.ascontiguousarray(K, dtype=np.float64)
    V = np.ascontiguousarray(V, dtype=np.float64)
    D = q.shape[0]
    out = np.zeros(D)
    lse = np.zeros(1)
    lib().oracle_dense_attention(D, K.shape[0], _p(q), _p(K), _p(V), float(sigma), _p(out), _p(lse))
    return out, float(lse[0])


def num_pages_of_call(D, Hkv, cu_tokens, tier_cum_bp) -> int:
    """Number of pages one pack call creates (for building a placement order)."""
    cu = np.asarray(cu_tokens)
    n = 0
    for s in range(len(cu) - 1):
        T = int(cu[s + 1] - cu[s])
        c = tier_counts(T, tier_cum_bp[s])
        per = [c[0], c[1] - c[0], c[2] - c[1]]
        n += Hkv * sum((x + SLOTS - 1) // SLOTS for x in per)
    return int(n)
