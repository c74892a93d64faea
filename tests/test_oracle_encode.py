"""Pins for the oracle's encoder (radius + per-group nearest codeword), CPU only.

The encoder's definition is an exhaustive argmin, so it is pinned by brute
force: distances recomputed here from the keys, the exhaustive minimum, the tie
rule, the closed-form radius and the special cases below."""
import numpy as np
import torch

import oracle
import synth
from helpers import f16_bits_to_f64, make_case, small_workload


def _directions(keys_u16):
    k = f16_bits_to_f64(keys_u16)
    r = np.sqrt((k * k).sum(-1))
    u = np.divide(k, r[..., None], out=np.zeros_like(k), where=r[..., None] > 0)
    return k, r, u


def test_encode_is_exhaustive_nearest_codeword():
    cfg = small_workload(D=64, Hkv=2, T=96, seed=1)
    case = make_case(cfg)
    r, c8, c4, d8, d4 = oracle.encode(case["keys"], case["cb8"], case["cb4"], with_dist=True)
    k, rr, u = _directions(case["keys"].view(torch.int16).numpy().view(np.uint16))
    N, H, D = k.shape
    G = D // 8
    ug = u.reshape(N, H, G, 1, 8)
    cb8 = case["cb8"].double().numpy()  # [H][G][256][8]
    cb4 = case["cb4"].double().numpy()
    ref8 = ((ug - cb8[None]) ** 2).sum(-1)  # [N][H][G][256]
    ref4 = ((ug - cb4[None]) ** 2).sum(-1)
    assert np.allclose(d8, ref8, rtol=0, atol=1e-13)
    assert np.allclose(d4, ref4, rtol=0, atol=1e-13)
    # the chosen code reaches the minimum; every strictly smaller index is worse
    assert np.array_equal(c8, ref8.argmin(-1))
    lo4 = ref4.argmin(-1)
    packed = (lo4[..., 0::2] | (lo4[..., 1::2] << 4)).astype(np.uint8)
    assert np.array_equal(c4, packed)
    # radius: the fp16 rounding of the exact norm
    assert np.array_equal(r, rr.astype(np.float16).view(np.uint16))


def test_encode_ties_take_lowest_index_and_zero_key():
    H, D, G = 1, 64, 8
    cb8 = np.zeros((H, G, 256, 8), np.float32)
    cb4 = np.zeros((H, G, 16, 8), np.float32)
    # codewords 3 and 7 identical and nearest to e0; all others far away
    cb8[..., :, 0] = 5.0
    cb8[..., 3, :] = 0
    cb8[..., 7, :] = 0
    cb8[..., 3, 0] = 1.0
    cb8[..., 7, 0] = 1.0
    cb4[..., :, 1] = 3.0
    cb4[..., 9, :] = 0.0
    cb4[..., 12, :] = 0.0
    keys = np.zeros((2, H, D), np.float16)
    keys[0, 0, ::8] = 2.0  # every group points along its first axis
    r, c8, c4 = oracle.encode(keys, cb8, cb4)
    assert oracle.f16_to_double(int(r[0, 0])) == float(np.float16(np.sqrt(8 * 4.0)))
    assert (c8[0] == 3).all()
    assert (c4[0] == (9 | (9 << 4))).all()
    # zero key: radius 0, u = 0, nearest = smallest-norm codeword (lowest index)
    assert r[1, 0] == 0
    assert (c8[1] == 3).all()
    assert (c4[1] == (9 | (9 << 4))).all()


def test_codebook_holding_exact_directions_gives_zero_error():
    cfg = small_workload(D=128, Hkv=1, T=64, seed=2)
    case = make_case(cfg)
    k16 = case["keys"].view(torch.int16).numpy().view(np.uint16)
    _, _, u = _directions(k16)
    N, H, D = u.shape
    G = D // 8
    cb8 = np.zeros((H, G, 256, 8), np.float32)
    perm = np.random.default_rng(0).permutation(256)[:N]
    for t in range(N):
        cb8[0, :, perm[t], :] = u[t, 0].reshape(G, 8)
    cb4 = np.full((H, G, 16, 8), 9.0, np.float32)
    r, c8, c4, d8, _ = oracle.encode(k16, cb8, cb4, with_dist=True)
    for t in range(N):
        assert (c8[t, 0] == perm[t]).all()
        assert d8[t, 0, np.arange(G), perm[t]].max() < 1e-13


def test_synthetic_codebooks_are_deterministic_and_unit_scale():
    cfg = small_workload(D=64, Hkv=2, seed=3)
    a8, a4 = synth.codebooks(cfg, 0)
    synth._CB_CACHE.clear()
    b8, b4 = synth.codebooks(cfg, 0)
    assert torch.equal(a8, b8) and torch.equal(a4, b4)
    # a centroid is a mean of sub-vectors of unit vectors: its norm is <= 1
    assert float(a8.norm(dim=-1).max()) <= 1.0 + 1e-6
    assert float(a4.norm(dim=-1).max()) <= 1.0 + 1e-6
