"""Pins of the oracle's compressor fed from hidden states ([V4.1]
"アーキテクチャ", CED paragraph, eq. 1: C = H W^KV, Z = H W^Z): identity
projections reduce it to the stream compressor, torch matmul fixes the
projection, a zero gate projection gives the bias-weighted mean."""

import numpy as np
import torch

from oracle import bf16_to_f64, compress, compress_hidden, f32_to_bf16, mxfp4_encode

D = 576


def _bf16(a):
    return f32_to_bf16(np.asarray(a, np.float32))


def test_identity_projections_are_the_stream_compressor():
    """d_model = 576 with W^KV = W^Z = I: x = z = H exactly, so every plane
    equals the stream compressor's on (H, H)."""
    rng = np.random.default_rng(0)
    h = _bf16(rng.standard_normal((32, D)))
    eye = _bf16(np.eye(D))
    b = rng.standard_normal(4).astype(np.float32)
    w_ik = _bf16(rng.standard_normal((D, 64)) / 24)
    a = compress_hidden(h, eye, eye, b, w_ik, 4)
    r = compress(h, h, b, w_ik, 4)
    for k in ("nope", "nscale", "rope", "ikey", "iscale"):
        np.testing.assert_array_equal(a[k], r[k], err_msg=k)
    np.testing.assert_array_equal(a["pooled"], r["pooled"])


def test_m1_is_the_projection():
    """m = 1: each entry is the projected row itself, x = H W^KV (torch
    matmul in float64), quantised."""
    rng = np.random.default_rng(1)
    d_model = 96
    h = _bf16(rng.standard_normal((10, d_model)))
    wkv = _bf16(rng.standard_normal((d_model, D)) / np.sqrt(d_model))
    wz = _bf16(rng.standard_normal((d_model, 1)))
    out = compress_hidden(h, wkv, wz, np.zeros(1, np.float32), None, 1)
    x = (torch.from_numpy(bf16_to_f64(h)) @ torch.from_numpy(bf16_to_f64(wkv))).numpy()
    np.testing.assert_allclose(out["pooled"], x, rtol=1e-12, atol=1e-12)
    codes, scales = mxfp4_encode(x[:, :512].astype(np.float32))
    np.testing.assert_array_equal(out["nope"], codes)
    np.testing.assert_array_equal(out["nscale"], scales)
    np.testing.assert_array_equal(out["rope"], f32_to_bf16(x[:, 512:].astype(np.float32)))


def test_zero_gate_projection_is_the_bias_weighted_mean():
    """W^Z = 0: every gate logit is its slot's bias, so entry j is
    sum_i softmax(b)_i x_{jm+i} for every channel."""
    rng = np.random.default_rng(2)
    d_model, m = 64, 4
    h = _bf16(rng.standard_normal((8 * m, d_model)))
    wkv = _bf16(rng.standard_normal((d_model, D)) / 8)
    wz = np.zeros((d_model, D), np.uint16)
    b = np.array([0.5, -1.0, 2.0, 0.0], np.float32)
    out = compress_hidden(h, wkv, wz, b, None, m)
    x = bf16_to_f64(h) @ bf16_to_f64(wkv)
    sb = torch.softmax(torch.from_numpy(b.astype(np.float64)), 0).numpy()
    ref = (x.reshape(8, m, D) * sb[None, :, None]).sum(axis=1)
    np.testing.assert_allclose(out["pooled"], ref, rtol=1e-13, atol=1e-14)


def test_single_gate_channel_broadcasts():
    """G = 1 (one gate logit per token, as HCA uses): equal to G = D with
    that column repeated."""
    rng = np.random.default_rng(3)
    d_model, m = 48, 8
    h = _bf16(rng.standard_normal((4 * m, d_model)))
    wkv = _bf16(rng.standard_normal((d_model, D)) / 7)
    wz1 = _bf16(rng.standard_normal((d_model, 1)) / 7)
    b = rng.standard_normal(m).astype(np.float32)
    a = compress_hidden(h, wkv, wz1, b, None, m)
    r = compress_hidden(h, wkv, np.repeat(wz1, D, axis=1), b, None, m)
    np.testing.assert_array_equal(a["pooled"], r["pooled"])
    np.testing.assert_array_equal(a["nope"], r["nope"])
