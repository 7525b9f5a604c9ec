"""Pins of the oracle's compressor: closed forms, invariants and a library routine."""

import numpy as np
import pytest
import torch

from oracle import bf16_to_f64, compress, f32_to_bf16, mxfp4_encode, pool_block


def _bf16(a):
    return f32_to_bf16(np.asarray(a, np.float32))


def _rand(rng, shape, s=1.0):
    return _bf16(rng.standard_normal(shape) * s)


D = 576


def test_m1_is_identity():
    rng = np.random.default_rng(0)
    x = _rand(rng, (8, D))
    z = _rand(rng, (8, D))
    out = compress(x, z, np.zeros(1, np.float32), None, m=1)
    np.testing.assert_array_equal(out["pooled"], bf16_to_f64(x))
    codes, scales = mxfp4_encode(bf16_to_f64(x)[:, :512].astype(np.float32))
    np.testing.assert_array_equal(out["nope"], codes)
    np.testing.assert_array_equal(out["nscale"], scales)
    np.testing.assert_array_equal(out["rope"], x[:, 512:])


def test_equal_gates_zero_bias_is_mean():
    rng = np.random.default_rng(1)
    x = _rand(rng, (64, D))
    z = _bf16(np.full((64, D), 0.75))
    out = compress(x, z, np.zeros(4, np.float32), None, m=4)
    ref = bf16_to_f64(x).reshape(16, 4, D).mean(axis=1)
    np.testing.assert_allclose(out["pooled"], ref, rtol=0, atol=1e-15)


def test_dominant_gate_copies_its_token():
    rng = np.random.default_rng(2)
    x = _rand(rng, (32, D))
    z = np.zeros((32, D), np.float32)
    slot = rng.integers(0, 4, 8)
    for j, s in enumerate(slot):
        z[4 * j + s] = 60.0
    out = compress(x, _bf16(z), np.zeros(4, np.float32), None, m=4)
    xf = bf16_to_f64(x)
    ref = np.stack([xf[4 * j + s] for j, s in enumerate(slot)])
    np.testing.assert_allclose(out["pooled"], ref, rtol=1e-20 + 1e-24, atol=1e-24 + 4 * np.exp(-60) * 5)


def test_constant_stream_is_constant():
    x = _bf16(np.full((128, D), -1.375))
    rng = np.random.default_rng(3)
    z = _rand(rng, (128, D), 3.0)
    out = compress(x, z, rng.standard_normal(128).astype(np.float32)[:128], None, m=128)
    np.testing.assert_allclose(out["pooled"], -1.375, rtol=1e-14)  # 128 rounded weights


def test_matches_torch_softmax_pooling():
    rng = np.random.default_rng(4)
    T, m = 256, 4
    x = _rand(rng, (T, D))
    z = _rand(rng, (T, D), 2.0)
    bias = rng.standard_normal(m).astype(np.float32)
    out = compress(x, z, bias, None, m=m)
    xt = torch.from_numpy(bf16_to_f64(x)).view(T // m, m, D)
    zt = torch.from_numpy(bf16_to_f64(z)).view(T // m, m, D)
    bt = torch.from_numpy(bias.astype(np.float64)).view(1, m, 1)
    ref = (torch.softmax(zt + bt, dim=1) * xt).sum(dim=1).numpy()
    np.testing.assert_allclose(out["pooled"], ref, rtol=1e-13, atol=1e-15)


def test_bias_shift_invariance_and_slot_binding():
    rng = np.random.default_rng(5)
    T, m = 64, 4
    x = _rand(rng, (T, D))
    z = _rand(rng, (T, D))
    bias = np.array([0.5, -1.0, 2.0, 0.25], np.float32)
    base = compress(x, z, bias, None, m=m)["pooled"]
    shifted = compress(x, z, bias + np.float32(3.0), None, m=m)["pooled"]
    np.testing.assert_allclose(shifted, base, rtol=1e-12, atol=1e-14)
    # Permute the tokens of every block and the bias slots alike: same result.
    perm = np.array([2, 0, 3, 1])
    xp = x.reshape(-1, m, D)[:, perm].reshape(T, D)
    zp = z.reshape(-1, m, D)[:, perm].reshape(T, D)
    permuted = compress(xp, zp, bias[perm], None, m=m)["pooled"]
    np.testing.assert_allclose(permuted, base, rtol=1e-12, atol=1e-14)
    # Moving the bias to the wrong slot changes the result.
    wrong = compress(xp, zp, bias, None, m=m)["pooled"]
    assert np.abs(wrong - base).max() > 1e-3


def test_single_gate_channel_broadcasts():
    rng = np.random.default_rng(6)
    x = _rand(rng, (32, D))
    z1 = _rand(rng, (32, 1))
    zfull = np.repeat(z1, D, axis=1)
    b = rng.standard_normal(4).astype(np.float32)
    np.testing.assert_array_equal(compress(x, z1, b, None, 4)["pooled"],
                                  compress(x, zfull, b, None, 4)["pooled"])


def test_pool_block_matches_compress():
    rng = np.random.default_rng(7)
    x = _rand(rng, (8, D))
    z = _rand(rng, (8, D))
    b = rng.standard_normal(4).astype(np.float32)
    out = compress(x, z, b, None, 4)["pooled"]
    for j in range(2):
        c = pool_block(bf16_to_f64(x[4 * j:4 * j + 4]), bf16_to_f64(z[4 * j:4 * j + 4]),
                       b.astype(np.float64))
        np.testing.assert_allclose(out[j], c, rtol=1e-14, atol=1e-16)


def test_indexer_key_projection_selection_matrix():
    rng = np.random.default_rng(8)
    x = _rand(rng, (16, D))
    z = _rand(rng, (16, D))
    d_idx = 64
    pick = rng.permutation(D)[:d_idx]
    W = np.zeros((D, d_idx), np.float32)
    W[pick, np.arange(d_idx)] = 1.0
    out = compress(x, z, np.zeros(4, np.float32), _bf16(W), 4)
    np.testing.assert_array_equal(out["kI"], out["pooled"][:, pick])
    codes, scales = mxfp4_encode(out["pooled"][:, pick].astype(np.float32))
    np.testing.assert_array_equal(out["ikey"], codes)
    np.testing.assert_array_equal(out["iscale"], scales)


def test_indexer_key_projection_matches_torch():
    rng = np.random.default_rng(9)
    x = _rand(rng, (64, D))
    z = _rand(rng, (64, D))
    W = _rand(rng, (D, 128), 1 / 24)
    out = compress(x, z, np.zeros(4, np.float32), W, 4)
    ref = torch.from_numpy(out["pooled"]).matmul(torch.from_numpy(bf16_to_f64(W))).numpy()
    np.testing.assert_allclose(out["kI"], ref, rtol=1e-12, atol=1e-14)


def test_rejects_ragged_block():
    with pytest.raises(ValueError):
        compress(np.zeros((6, D), np.uint16), np.zeros((6, D), np.uint16), np.zeros(4, np.float32), None, 4)


def test_decode_entries_places_every_channel():
    """decode_entries of an m = 1 compress gives back the raw rows exactly
    when every value is representable: channels 0..511 as the MXFP4 decode
    of grid values (one power-of-two scale per block of 32), channels
    512..575 as the bf16 rows themselves.  Every channel holds a value that
    identifies it, so a swapped, shifted or reversed channel range fails."""
    from oracle import decode_entries

    grid = np.array([0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    rows = []
    for r in range(6):
        v = np.empty(D)
        for blk in range(16):
            # block maximum 6 * 2^X fixes the block scale at 2^X; the other
            # 31 values are grid values times 2^X with a per-channel sign
            X = (blk + 3 * r) % 9 - 4
            vals = grid[(np.arange(32) + blk + r) % 7] * 2.0 ** X
            vals[(blk + r) % 32] = 6.0 * 2.0 ** X
            vals *= np.where((np.arange(32) + r) % 3 == 0, -1.0, 1.0)
            v[32 * blk:32 * blk + 32] = vals
        # positional channels: distinct bf16 values (128 + c) * 2^(r - 7)
        v[512:] = (128.0 + np.arange(64)) * 2.0 ** (r - 7)
        rows.append(v)
    x64 = np.array(rows)
    x = _bf16(x64)
    np.testing.assert_array_equal(bf16_to_f64(x), x64)           # exact in bf16
    z = _rand(np.random.default_rng(9), (6, D))
    out = compress(x, z, np.zeros(1, np.float32), None, m=1)
    dec = decode_entries(out["nope"], out["nscale"], out["rope"])
    assert dec.shape == (6, D)
    np.testing.assert_array_equal(dec, x64)
