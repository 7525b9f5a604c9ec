"""Pins of the oracle's storage formats against library casts and brute force."""

import numpy as np
import pytest
import torch

from oracle import (
    E2M1_VALUES,
    bf16_to_f64,
    e2m1_to_f64,
    e4m3_to_f64,
    e8m0_to_f64,
    f32_to_bf16,
    mxfp4_decode,
    mxfp4_encode,
)


def test_e2m1_table_matches_bit_fields():
    # E2M1: 1 sign bit, 2 exponent bits with bias 1, 1 mantissa bit; exponent
    # field 0 is subnormal (mantissa/2 * 2^0).  Derived from the fields, not the table.
    for code in range(16):
        s = -1.0 if code & 8 else 1.0
        e = (code >> 1) & 3
        mnt = code & 1
        mag = (mnt / 2.0) if e == 0 else (1.0 + mnt / 2.0) * 2.0 ** (e - 1)
        assert e2m1_to_f64(code) == s * mag
    assert list(E2M1_VALUES) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]


def test_e8m0_matches_torch():
    b = torch.arange(255, dtype=torch.uint8)
    ref = b.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    np.testing.assert_array_equal(e8m0_to_f64(np.arange(255)), ref)
    assert np.isnan(e8m0_to_f64(255))


def test_e4m3_matches_torch_all_codes():
    b = torch.arange(256, dtype=torch.uint8)
    ref = b.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = e4m3_to_f64(np.arange(256))
    nan = np.isnan(ref)
    assert nan.sum() == 2 and np.array_equal(nan, np.isnan(got))
    np.testing.assert_array_equal(got[~nan], ref[~nan])
    assert e4m3_to_f64(0x7E) == 448.0 and e4m3_to_f64(0x01) == 2.0 ** -9


def test_bf16_roundtrip_matches_torch():
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.standard_normal(100000) * 10.0 ** rng.integers(-30, 30, 100000),
                        [0.0, -0.0, 1.0, -2.5, 3.0e38, 1e-40]]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = f32_to_bf16(v)
    np.testing.assert_array_equal(got, ref)
    back = torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(bf16_to_f64(ref), back)


def _brute_e2m1(v):
    """Nearest E2M1 value by exhaustive search; ties to the even mantissa bit; saturate."""
    best, bestd = None, None
    for code in range(8):
        d = abs(abs(v) - E2M1_VALUES[code])
        if bestd is None or d < bestd or (d == bestd and code % 2 == 0):
            best, bestd = code, d
    if abs(v) > 6:
        best = 7
    return best | (8 if v < 0 else 0)


def _brute_block(vals):
    """MXFP4 of one block by search: the scale is the smallest power of two
    2^X (X >= -127) with max|v| / 2^X < 8, i.e. the OCP shared-exponent rule
    X = floor(log2 amax) - emax(E2M1) written as a search."""
    amax = max(abs(float(v)) for v in vals)
    if amax == 0:
        X = -127
    else:
        X = -127
        while amax / 2.0 ** X >= 8.0:
            X += 1
    X = min(X, 127)
    codes = [_brute_e2m1(float(v) / 2.0 ** X) for v in vals]
    return codes, X + 127


@pytest.mark.parametrize("seed", range(6))
def test_mxfp4_encode_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    nblk = 40
    v = rng.standard_normal((nblk, 32)) * np.exp2(rng.integers(-130, 120, nblk))[:, None]
    # plant exact midpoints and grid values at random scales
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, 6.0, 0.5])
    v[:10, :10] = (mids * np.exp2(rng.integers(-10, 10, 10))[:, None])[:, :10] * rng.choice([-1, 1], (10, 10))
    v[10, :] = 0.0
    v[11, :] = 0.0
    v[11, 3] = -1e-3
    v = v.astype(np.float32)
    packed, scales = mxfp4_encode(v)
    for b in range(nblk):
        codes, sb = _brute_block(v[b])
        assert scales[b] == sb, (b, scales[b], sb)
        got = [(packed[b, i // 2] >> (4 * (i % 2))) & 0xF for i in range(32)]
        assert got == codes, (b, got, codes)


def test_mxfp4_midpoint_rules():
    # A block whose maximum is 6 has X = 0, so the elements are rounded as given.
    vals = np.array([6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -0.1] + [0.0] * 22, np.float32)
    packed, scales = mxfp4_encode(vals)
    assert scales[0] == 127
    dec = mxfp4_decode(packed, scales)
    np.testing.assert_array_equal(dec[:10], [6.0, 0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, -0.0, -0.0])
    # sign is kept on negative values that round to zero
    assert (packed[4] & 0xF) == 0x8 and (packed[4] >> 4) == 0x8
    # saturation: amax 7.9 -> X = 0, 7.9 -> 6
    p2, s2 = mxfp4_encode(np.array([7.9] + [0.0] * 31, np.float32))
    assert s2[0] == 127 and (p2[0] & 0xF) == 7


def test_mxfp4_grid_roundtrip_every_scale():
    for sb in range(1, 254):
        X = sb - 127
        vals = np.array(list(E2M1_VALUES) + list(-E2M1_VALUES[1:]) + [0.0] * 17)[:32] * 2.0 ** X
        vals[0] = 6.0 * 2.0 ** X  # pins the scale
        packed, scales = mxfp4_encode(vals)
        assert scales[0] == sb
        np.testing.assert_array_equal(mxfp4_decode(packed, scales), vals)


def test_mxfp4_decode_all_code_scale_pairs():
    codes = np.arange(16, dtype=np.uint8)
    for sb in range(255):
        packed = np.tile((codes[0::2] | (codes[1::2] << 4)).astype(np.uint8), 2)
        dec = mxfp4_decode(packed[None, :], np.array([[sb]], np.uint8))[0]
        ref = np.array([e2m1_to_f64(c) for c in list(range(16)) * 2]) * 2.0 ** (sb - 127)
        np.testing.assert_array_equal(dec, ref)


def test_nibble_order_even_channel_low():
    vals = np.zeros(32, np.float32)
    vals[0] = 6.0
    vals[1] = 0.5
    packed, _ = mxfp4_encode(vals)
    assert packed[0] == (7 | (1 << 4))
