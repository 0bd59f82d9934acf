"""Pins of the MoE expert oracle (MXFP4 -> FP8 conversion and the expert
product) to things other than itself: the MX specification's E2M1 table and
a hand-worked block (tests/golden/mxfp4_e2m1_values.json), torch's own E8M0
and E4M3 conversions (library routines, round to nearest even), the closed
form of saturation, and numpy matrix products of the decoded values."""
import json
import os

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mxfp4_e2m1_values.json")


def test_fp4_table_and_sign(oracle_lib):
    g = json.load(open(GOLDEN))
    for c, v in enumerate(g["fp4_codes_0_to_7"]):
        assert oracle_lib.fp4_value(c) == v
        assert oracle_lib.fp4_value(c | g["fp4_sign_bit"]) == -v


def test_e8m0_matches_torch(oracle_lib):
    codes = torch.arange(255, dtype=torch.uint8)
    ref = codes.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = np.array([oracle_lib.e8m0_value(int(c)) for c in codes])
    np.testing.assert_array_equal(got, ref)
    assert np.isnan(oracle_lib.e8m0_value(255))


def test_e4m3_decode_matches_torch(oracle_lib):
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle_lib.e4m3_value(int(c)) for c in codes])
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(got[ok], ref[ok])


def test_e4m3_encode_matches_torch_below_saturation(oracle_lib):
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.normal(size=4000) * 50, rng.normal(size=2000) * 1e-2, rng.normal(size=1000) * 1e-3,
        np.array([0.0, -0.0, 448.0, 463.99, -463.99, 2.0**-9, 1.5 * 2.0**-9, 2.0**-10]),
        # exact midpoints between neighbouring E4M3 values (ties to even)
        np.array([(torch.tensor([c], dtype=torch.uint8).view(torch.float8_e4m3fn).double().item() +
                   torch.tensor([c + 1], dtype=torch.uint8).view(torch.float8_e4m3fn).double().item()) / 2
                  for c in range(0, 125)]),
    ])
    x = x[np.abs(x) < 464.0]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle_lib.e4m3_encode(v) for v in x], dtype=np.uint8)
    np.testing.assert_array_equal(got, ref)


def test_e4m3_encode_saturates(oracle_lib):
    # OCP "satfinite": every finite value beyond the largest E4M3 (448) -> +-448
    for v in (464.0, 480.0, 1e6, 1e300):
        assert oracle_lib.e4m3_encode(v) == 0x7E
        assert oracle_lib.e4m3_encode(-v) == 0xFE
    assert oracle_lib.e4m3_encode(float("nan")) == 0x7F


def test_hand_worked_block(oracle_lib):
    h = json.load(open(GOLDEN))["hand_worked"]
    codes = np.zeros((1, 1, 16), np.uint8)
    codes[0, 0, :2] = h["bytes"]
    scales = np.array([[[h["scale"]]]], np.uint8)
    w8 = oracle_lib.mxfp4_to_fp8(codes, scales, [0], 1, 32)
    assert w8[0, 0, :4].tolist() == h["e4m3"]
    assert [oracle_lib.e4m3_value(int(c)) for c in w8[0, 0, :4]] == h["values"]
    assert (w8[0, 0, 4:] == 0).all()  # code 0 -> +0


def _random_mxfp4(rng, experts, N, K, scale_lo=119, scale_hi=133):
    codes = rng.integers(0, 256, (experts, N, K // 2), dtype=np.uint8)
    scales = rng.integers(scale_lo, scale_hi + 1, (experts, N, K // 32), dtype=np.uint8)
    return codes, scales


def _decode_mxfp4(codes, scales, K):
    """Decoded weights [.., N, K] in float64 via the E2M1 table (numpy)."""
    table = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0,
                      -4.0, -6.0])
    lo, hi = codes & 15, codes >> 4
    el = np.stack([table[lo], table[hi]], axis=-1).reshape(*codes.shape[:-1], K)
    sc = np.repeat(2.0 ** (scales.astype(np.float64) - 127), 32, axis=-1)
    return el * sc


def test_conversion_is_exact_in_the_exact_scale_range(oracle_lib):
    # scales 2^-8 .. 2^6 keep every scaled E2M1 value an E4M3 number: at 2^-8
    # the smallest, 0.5 * 2^-8, is the smallest E4M3 subnormal 2^-9; at 2^6 the
    # largest, 6 * 2^6 = 384, is below 448
    rng = np.random.default_rng(1)
    codes, scales = _random_mxfp4(rng, 3, 48, 128)
    w8 = oracle_lib.mxfp4_to_fp8(codes, scales, [2, 0], 48, 128)
    dec = _decode_mxfp4(codes, scales, 128)
    got = torch.from_numpy(w8).view(torch.float8_e4m3fn).double().numpy()
    np.testing.assert_array_equal(got[0], dec[2])
    np.testing.assert_array_equal(got[1], dec[0])


def test_exact_range_is_tight(oracle_lib):
    # one step beyond either end some scaled element is not an E4M3 number
    half_at_118 = oracle_lib.e4m3_value(oracle_lib.mxfp4_to_fp8(
        np.full((1, 16, 16), 0x11, np.uint8), np.full((1, 16, 1), 118, np.uint8), [0], 16, 32)[0, 0, 0])
    assert half_at_118 != 0.5 * 2.0 ** -9       # 2^-10 rounds (to 0)
    six_at_134 = oracle_lib.e4m3_value(oracle_lib.mxfp4_to_fp8(
        np.full((1, 16, 16), 0x77, np.uint8), np.full((1, 16, 1), 134, np.uint8), [0], 16, 32)[0, 0, 0])
    assert six_at_134 == 448.0                  # 768 saturates


def test_conversion_rounds_and_saturates_outside_it(oracle_lib):
    rng = np.random.default_rng(2)
    codes, scales = _random_mxfp4(rng, 1, 16, 64, scale_lo=100, scale_hi=140)
    w8 = oracle_lib.mxfp4_to_fp8(codes, scales, [0], 16, 64)
    dec = _decode_mxfp4(codes, scales, 64)[0]
    small = np.abs(dec) < 464
    ref = torch.from_numpy(dec[small]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(w8[0][small], ref)
    assert (w8[0][~small] & 0x7F == 0x7E).all()


@pytest.mark.parametrize("seed", [3, 4])
def test_moe_gemm_matches_numpy(oracle_lib, seed):
    rng = np.random.default_rng(seed)
    experts, N, K = 5, 40, 256
    codes, scales = _random_mxfp4(rng, experts, N, K)
    rows = [3, 0, 1, 7]                      # an expert with no routed token
    ids = [4, 1, 1, 0]                       # the same expert listed twice
    off = np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)
    xv = rng.integers(-4, 5, (off[-1], K)).astype(np.float32)
    x = torch.from_numpy(xv).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    y = oracle_lib.moe_gemm(x, off, ids, codes, scales, N, K)
    dec = _decode_mxfp4(codes, scales, K)
    for i, e in enumerate(ids):
        ref = xv[off[i]:off[i + 1]].astype(np.float64) @ dec[e].T
        np.testing.assert_array_equal(y[off[i]:off[i + 1]], ref.astype(np.float32))
