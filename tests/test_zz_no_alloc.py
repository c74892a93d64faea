"""ada_decode_noalloc, the decode entry point that allocates nothing, called
through the C ABI: two calls in a row (the second on a smaller cache, so
the library's array still holds the first call's partials) each give
exactly ada_decode's outputs on the same inputs."""
import ctypes as C

import numpy as np
import pytest
import torch

import compressed_kv_attention_amd as ada
import synth
from gpu_util import flush, gpu_encode

pytestmark = pytest.mark.gpu


def _layer(number, T=None):
    cfg = synth.WORKLOADS[number]
    H, D = cfg.num_kv_heads, cfg.head_dim
    geom = ada.Geom(D, cfg.num_q_heads, H)
    lens = synth.seq_lens(cfg) if T is None else np.full(cfg.num_seqs, T, np.int64)
    cu = synth.cu_tokens(lens)
    N = int(cu[-1])
    bp = synth.tier_mix(cfg)
    keys = synth.keys(cfg, 0, N, "cuda")
    vals = synth.values(cfg, 0, N, "cuda")
    cb8, cb4 = (t.cuda() for t in synth.codebooks(cfg, 0))
    r, c8, c4 = gpu_encode(geom, keys, cb8, cb4)
    maxp = int(max(lens)) // 16 + 4
    dc = ada.Cache(geom, cfg.num_seqs, maxp, N * H * 512 + (1 << 20))
    ada.rdr_pack(geom, dc, cu, bp, keys, vals, r, c8, c4, synth.scores(cfg, 0, N).cuda())
    torch.cuda.synchronize()
    return cfg, geom, dc, cb8, cb4, synth.queries(cfg, 0, "cuda")


def _noalloc(geom, dc, cb8, cb4, q, sigma, out, lse, splits):
    """Straight through ctypes: the C entry point itself, no binding logic."""
    L = C.CDLL(ada.lib_path())
    fn = L.ada_decode_noalloc
    P = C.c_void_p
    fn.argtypes = [C.POINTER(ada.Geom), C.c_void_p, P, P, P, C.c_float, P, P, P, C.c_int32, P]
    fn.restype = C.c_int
    v = dc.view()
    return fn(C.byref(geom), C.addressof(v), P(cb8.data_ptr()), P(cb4.data_ptr()), P(q.data_ptr()),
              float(sigma), P(out.data_ptr()), P(lse.data_ptr()), None, splits,
              P(torch.cuda.current_stream().cuda_stream))


@pytest.mark.parametrize("splits", [0, 3])
def test_noalloc_decode_equals_decode_twice_second_smaller(splits):
    first = _layer(3)             # 4 x 131072 tokens (identity placement here)
    second = _layer(2, T=5000)    # 1 x 5000 tokens
    for label, (cfg, geom, dc, cb8, cb4, q) in (("first", first), ("second", second)):
        S, Hq, D = cfg.num_seqs, cfg.num_q_heads, cfg.head_dim
        o_ref = torch.empty((S, Hq, D), device="cuda")
        l_ref = torch.empty((S, Hq), device="cuda")
        ada.decode(geom, dc, cb8, cb4, q, cfg.sigma, o_ref, l_ref, num_splits=splits)
        o = torch.full((S, Hq, D), float("nan"), device="cuda")
        l = torch.full((S, Hq), float("nan"), device="cuda")
        assert _noalloc(geom, dc, cb8, cb4, q, cfg.sigma, o, l, splits) == 0
        torch.cuda.synchronize()
        err = float((o.double() - o_ref.double()).abs().max())
        assert err <= 1e-2 and torch.equal(o, o_ref) and torch.equal(l, l_ref), (label, err)
        flush(f"[noalloc] {label} call ({cfg.name}, splits={splits}): equal to ada_decode")


def test_noalloc_rejects_partials_beyond_its_array():
    cfg = synth.WORKLOADS[2]
    geom = ada.Geom(128, 32, 8)
    dc = ada.Cache(geom, 64, 4200, 1 << 20)
    q = torch.zeros((64, 32, 128), dtype=torch.bfloat16, device="cuda")
    o = torch.zeros((64, 32, 128), device="cuda")
    l = torch.zeros((64, 32), device="cuda")
    cb8 = torch.zeros((8, 16, 256, 8), device="cuda")
    cb4 = torch.zeros((8, 16, 16, 8), device="cuda")
    need = ada.decode_workspace_size(geom, 64, 4200, 64)
    assert need > (8 << 20)
    assert _noalloc(geom, dc, cb8, cb4, q, cfg.sigma, o, l, 64) == ada.EWORKSPACE
    assert not o.any()
