"""Pins for the oracle's number formats, page-section layouts and the int8
value quantiser (CPU only)."""
import json
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_f16_decode_exhaustive_matches_numpy():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_double(int(b)) for b in bits])
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(np.isinf(got), np.isinf(ref))


def test_f16_encode_round_to_nearest_even_matches_numpy():
    rng = np.random.default_rng(0)
    # random magnitudes across subnormal .. overflow-free range, plus exact ties
    x = np.concatenate([
        rng.standard_normal(20000) * np.exp2(rng.integers(-26, 16, 20000)),
        (np.arange(-3000, 3000) + 0.5) * 2.0 ** -24,           # subnormal ties
        (np.arange(1024, 2048) + 0.5) * 2.0 ** -10,            # ties in [1, 2)
        np.array([0.0, -0.0, 65504.0, 65519.99, -65504.0]),
    ])
    x = x[np.abs(x) < 65520.0]  # beyond this numpy gives inf, the oracle saturates
    got = np.array([oracle.double_to_f16(float(v)) for v in x], dtype=np.uint16)
    ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


def test_f16_encode_saturates_instead_of_inf():
    assert oracle.double_to_f16(65520.0) == 0x7BFF
    assert oracle.double_to_f16(1e30) == 0x7BFF
    assert oracle.double_to_f16(-1e30) == 0xFBFF


def test_bf16_round_trip_matches_torch():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(5000) * np.exp2(rng.integers(-20, 20, 5000))).astype(np.float16)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.double_to_bf16(float(v)) for v in x], dtype=np.uint16)
    assert np.array_equal(got, ref)
    back = np.array([oracle.bf16_to_double(int(b)) for b in ref])
    assert np.array_equal(back, torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).double().numpy())


@pytest.mark.parametrize("D", [64, 128])
def test_row_and_column_sections_are_lane_chunked_bijections(D):
    t, d = np.meshgrid(np.arange(16), np.arange(D), indexing="ij")
    rows = np.array([[oracle.row_off(a, b) for b in range(D)] for a in range(16)])
    cols = np.array([[oracle.col_off(a, b) for b in range(D)] for a in range(16)])
    cols8 = np.array([[oracle.col8_off(a, b) for b in range(D)] for a in range(16)])
    assert sorted(rows.ravel()) == list(range(0, 32 * D, 2))
    assert sorted(cols.ravel()) == list(range(0, 32 * D, 2))
    assert sorted(cols8.ravel()) == list(range(16 * D))
    blk = d // 16
    # the lane (16-byte column of a KiB) and the 8-byte half / 4-byte quarter
    assert np.array_equal((rows % 1024) // 16, t + 16 * ((d % 16) // 4))
    assert np.array_equal((cols % 1024) // 16, d % 16 + 16 * (t // 4))
    assert np.array_equal((cols8 % 1024) // 16, d % 16 + 16 * (t // 4))
    assert np.array_equal(rows // 1024, blk // 2) and np.array_equal(cols // 1024, blk // 2)
    assert np.array_equal(cols8 // 1024, blk // 4)
    assert np.array_equal((rows % 16) // 8, blk % 2) and np.array_equal((rows % 8) // 2, d % 4)
    assert np.array_equal((cols % 16) // 8, blk % 2) and np.array_equal((cols % 8) // 2, t % 4)
    assert np.array_equal((cols8 % 16) // 4, blk % 4) and np.array_equal(cols8 % 4, t % 4)
    # spot values: slot 5, dim 22 (block 1)
    assert oracle.row_off(5, 22) == 0 * 1024 + (5 + 16 * 1) * 16 + 8 + 2 * 2
    assert oracle.col_off(5, 22) == 0 * 1024 + (6 + 16 * 1) * 16 + 8 + 1 * 2
    assert oracle.col8_off(5, 22) == 0 * 1024 + (6 + 16 * 1) * 16 + 4 + 1


def test_page_sizes():
    assert [oracle.page_bytes(128, t) for t in range(4)] == [8192, 4480, 2304, 8192]
    assert [oracle.page_bytes(64, t) for t in range(4)] == [4096, 2304, 1152, 4096]


def test_quant_v_golden():
    with open(os.path.join(GOLDEN, "quant_v.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        v = torch.zeros(64)
        v[:3] = torch.tensor(case["v"])
        q, sc = oracle.quant_v(v.to(torch.bfloat16))
        assert sc == case["scale_bits"]
        assert oracle.f16_to_double(sc) == case["scale"]
        assert list(q[:3]) == case["q"] and not q[3:].any()


def test_quant_v_error_bound_random():
    rng = np.random.default_rng(2)
    for i in range(300):
        D = 128 if i % 2 else 64
        v = torch.from_numpy(rng.standard_normal(D) * np.exp2(rng.integers(-12, 12))).to(torch.bfloat16)
        q, sc = oracle.quant_v(v)
        s = oracle.f16_to_double(sc)
        vf = v.double().numpy()
        amax = np.abs(vf).max()
        assert np.abs(q.astype(int)).max() <= 127
        # the scale is amax/127 rounded (twice) to fp16, so 127*s is within
        # 2^-10 (relative) of amax; rounding to the integer grid adds s/2
        err = np.abs(vf - q * s)
        assert err.max() <= s * 0.5 + amax * 2.0 ** -10 + 1e-30
        # the largest |v| lands on +-127 or +-126 (fp16 scale rounding)
        assert np.abs(q).max() >= 126
