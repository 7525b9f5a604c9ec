"""Pins of the oracle's FP8 window format (MXFP8: E4M3 elements, one E8M0
scale per 32 channels; bf16 positional channels): the E4M3 table and
rounding against torch's float8_e4m3fn, brute-force nearest-value rounding
with ties to even, saturation, the scale rule's closed form, exact round
trips of representable values, the rounding error bound, and the window
planes."""

import numpy as np
import pytest
import torch

import oracle as O
from oracle.formats import _e4m3_round


def _torch_e4m3(x32):
    return torch.from_numpy(np.asarray(x32, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_table_matches_torch():
    codes = np.arange(127, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.E4M3_VALUES, ref)
    assert np.all(np.diff(O.E4M3_VALUES) > 0)
    assert O.E4M3_VALUES[126] == 448.0 and O.E4M3_VALUES[1] == 2.0 ** -9


def test_rounding_matches_torch_below_saturation():
    rng = np.random.default_rng(0)
    mags = np.concatenate([
        np.abs(rng.standard_normal(20000)) * 50,
        rng.uniform(0, 2.0 ** -6, 5000),                   # subnormal range
        (O.E4M3_VALUES[:-1] + O.E4M3_VALUES[1:]) / 2,     # every midpoint (ties)
        O.E4M3_VALUES,
    ]).astype(np.float32)
    mags = mags[mags < 448]
    np.testing.assert_array_equal(_e4m3_round(mags.astype(np.float64)), _torch_e4m3(mags).astype(np.int64))


def test_rounding_brute_force_and_saturation():
    rng = np.random.default_rng(1)
    mags = np.concatenate([rng.uniform(0, 600, 3000), (O.E4M3_VALUES[:-1] + O.E4M3_VALUES[1:]) / 2, [448, 449, 1e9]])
    got = _e4m3_round(mags)
    for mg, c in zip(mags, got):
        if mg >= 448:
            assert c == 126
            continue
        d = np.abs(O.E4M3_VALUES - mg)
        best = np.flatnonzero(d == d.min())
        want = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
        assert c == want, (mg, c, want)


def test_scale_rule_closed_form_and_sign():
    for k in (-130, -120, -3, 0, 5, 100):
        v = np.zeros((1, 32))
        v[0, 7] = 2.0 ** k
        v[0, 9] = -(2.0 ** (k - 20))                     # rounds to a signed zero
        c, s = O.mxfp8_encode(v)
        x = min(max(k - 8, -127), 127)
        assert s[0, 0] == x + 127
        if k - 8 >= -127:
            assert c[0, 7] == 0x78                         # 2^8 at scale 2^(k-8)
        assert c[0, 9] & 0x80
    c, s = O.mxfp8_encode(np.zeros((2, 64)))
    assert np.all(c == 0) and np.all(s == 0)
    # values between 448 and 512 times the scale saturate
    v = np.full((1, 32), 1.0)
    v[0, 0] = 1.9                                          # 1.9 * 2^8 = 486.4 > 448
    c, s = O.mxfp8_encode(v)
    assert c[0, 0] == 126


def test_representable_values_round_trip():
    rng = np.random.default_rng(2)
    codes = rng.integers(0, 127, (50, 64)) | (rng.integers(0, 2, (50, 64)) * 0x80)
    codes[:, 0] = 0x78                                     # make 256 * 2^X the block maximum in block 0
    codes[:, 32] = 0x7E                                    # and 448 in block 1
    xs = rng.integers(-100, 100, (50, 2))
    v = O.mxfp8_decode(codes.astype(np.uint8), (xs + 127).astype(np.uint8))
    c2, s2 = O.mxfp8_encode(v)
    np.testing.assert_array_equal(O.mxfp8_decode(c2, s2), v)


def test_error_bound_on_normal_data():
    rng = np.random.default_rng(3)
    v = rng.standard_normal((200, 512)) * np.exp(rng.uniform(-20, 20, (200, 1)))
    c, s = O.mxfp8_encode(v)
    d = O.mxfp8_decode(c, s)
    scale = np.repeat(O.e8m0_to_f64(s), 32, axis=1)
    sat = np.abs(v) / scale > 448
    # half a unit in the last place of E4M3 (3 mantissa bits), or of its subnormal step
    bound = np.maximum(np.abs(v) * 2.0 ** -4, scale * 2.0 ** -10)
    assert np.all(np.abs(d - v)[~sat] <= bound[~sat])
    np.testing.assert_array_equal(np.abs(d[sat]), (448 * scale)[sat])


def test_window_planes():
    rng = np.random.default_rng(4)
    x = torch.from_numpy(rng.standard_normal((40, 576)).astype(np.float32)).to(torch.bfloat16)
    xu = x.view(torch.int16).numpy().view(np.uint16)
    pl = O.swa_encode(xu)
    assert pl["codes"].shape == (40, 512) and pl["scales"].shape == (40, 16) and pl["rope"].shape == (40, 64)
    np.testing.assert_array_equal(pl["rope"], xu[:, 512:])
    rows = O.swa_decode(pl["codes"], pl["scales"], pl["rope"])
    np.testing.assert_array_equal(rows[:, 512:], O.bf16_to_f64(xu[:, 512:]))
    c, s = O.mxfp8_encode(O.bf16_to_f64(xu[:, :512]))
    np.testing.assert_array_equal(rows[:, :512], O.mxfp8_decode(c, s))
    # decoded rows of bf16 inputs are exact in bf16
    np.testing.assert_array_equal(O.bf16_to_f64(O.f32_to_bf16(rows.astype(np.float32))), rows)


def test_attention_takes_decoded_window_rows():
    """The window rows may be given as bf16 bits or as decoded float64 rows."""
    rng = np.random.default_rng(5)
    N, S = 64, 48
    nope, nscale = O.mxfp4_encode(rng.standard_normal((N, 512)).astype(np.float32))
    rope = torch.from_numpy(rng.standard_normal((N, 64)).astype(np.float32)).to(torch.bfloat16)
    rope = rope.view(torch.int16).numpy().view(np.uint16)
    x = torch.from_numpy(rng.standard_normal((S, 576)).astype(np.float32)).to(torch.bfloat16)
    xu = x.view(torch.int16).numpy().view(np.uint16)
    q = torch.from_numpy(rng.standard_normal((8, 576)).astype(np.float32) * 0.05).to(torch.bfloat16)
    qu = q.view(torch.int16).numpy().view(np.uint16)
    idx = np.arange(0, 30, 3)
    a = O.sparse_attention(qu, nope, nscale, rope, idx, xu, 10, 57, 16, 0.05, 1, N)
    b = O.sparse_attention(qu, nope, nscale, rope, idx, O.bf16_to_f64(xu), 10, 57, 16, 0.05, 1, N)
    np.testing.assert_array_equal(a[0], b[0])
    pl = O.swa_encode(xu)
    dec = O.swa_decode(pl["codes"], pl["scales"], pl["rope"])
    c = O.sparse_attention(qu, nope, nscale, rope, idx, dec, 10, 57, 16, 0.05, 1, N)
    assert not np.array_equal(c[0], a[0])                  # FP8 rows differ from bf16 rows
    assert np.abs(c[0] - a[0]).max() <= 0.1 * np.abs(a[0]).max()
