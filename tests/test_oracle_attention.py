"""Pins of the oracle's attention: torch SDPA special cases, closed forms, algebra."""

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

from oracle import (
    attention,
    bf16_to_f64,
    compress,
    decode_entries,
    dense_attention,
    f32_to_bf16,
    sparse_attention,
)

D = 576
SCALE = np.float32(1.0 / 24.0)


def _bf16(a):
    return f32_to_bf16(np.asarray(a, np.float32))


def _cache(rng, T, m, scale=1.0):
    x = _bf16(rng.standard_normal((T, D)) * scale)
    z = _bf16(rng.standard_normal((T, D)))
    b = rng.standard_normal(m).astype(np.float32)
    return x, compress(x, z, b, None, m)


def test_m1_all_selected_no_window_is_causal_sdpa():
    """m = 1 with every visible entry selected and no window is textbook
    causal attention over the per-token FP4-dequantised KV."""
    rng = np.random.default_rng(0)
    T, H = 48, 4
    x, c = _cache(rng, T, 1)
    kv = decode_entries(c["nope"], c["nscale"], c["rope"])
    q = _bf16(rng.standard_normal((T, H, D)))
    qt = torch.from_numpy(bf16_to_f64(q)).permute(1, 0, 2)          # [H][T][D]
    kt = torch.from_numpy(kv)[None].expand(H, T, D)
    ref = F.scaled_dot_product_attention(qt, kt, kt, is_causal=True, scale=float(SCALE))
    for p in range(T):
        o, lse = sparse_attention(q[p], c["nope"], c["nscale"], c["rope"], np.arange(p + 1),
                                  x, 0, p, 0, SCALE, 1, T)
        np.testing.assert_allclose(o, ref[:, p].numpy(), rtol=1e-12, atol=1e-13)


def test_window_only_is_sliding_window_sdpa():
    rng = np.random.default_rng(1)
    T, H, n_win = 40, 2, 7
    x = _bf16(rng.standard_normal((T, D)))
    q = _bf16(rng.standard_normal((T, H, D)))
    empty = np.zeros((0, 256), np.uint8)
    i = np.arange(T)
    mask = (i[None, :] <= i[:, None]) & (i[None, :] > i[:, None] - n_win)
    xt = torch.from_numpy(bf16_to_f64(x))[None].expand(H, T, D)
    qt = torch.from_numpy(bf16_to_f64(q)).permute(1, 0, 2)
    ref = F.scaled_dot_product_attention(qt, xt, xt, attn_mask=torch.from_numpy(mask), scale=float(SCALE))
    for p in range(T):
        o, _ = sparse_attention(q[p], empty, np.zeros((0, 16), np.uint8), np.zeros((0, 64), np.uint16),
                                np.full(8, -1), x, 0, p, n_win, SCALE, 4, 0)
        np.testing.assert_allclose(o, ref[:, p].numpy(), rtol=1e-12, atol=1e-13)


def test_window_respects_buffer_start():
    rng = np.random.default_rng(2)
    x = _bf16(rng.standard_normal((100, D)))
    q = _bf16(rng.standard_normal((3, D)))
    p, n_win = 90, 20
    # A buffer holding rows 80..99 only: positions 71..79 are not available.
    o1, l1 = sparse_attention(q, np.zeros((0, 256), np.uint8), np.zeros((0, 16), np.uint8),
                              np.zeros((0, 64), np.uint16), [], x[80:], 80, p, n_win, SCALE, 4, 0)
    o2, l2 = attention(q, bf16_to_f64(x[80:91]), SCALE)
    np.testing.assert_allclose(o1, o2, rtol=1e-14)
    np.testing.assert_allclose(l1, l2, rtol=1e-14)


def test_all_selected_equals_dense():
    rng = np.random.default_rng(3)
    T, m = 512, 4
    x, c = _cache(rng, T, m)
    q = _bf16(rng.standard_normal((8, D)))
    p = T - 1
    N = T // m
    a = sparse_attention(q, c["nope"], c["nscale"], c["rope"], np.arange(N), x, 0, p, 16, SCALE, m, N)
    b = dense_attention(q, c["nope"], c["nscale"], c["rope"], x, 0, p, 16, SCALE, m, N)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_single_key_and_identical_keys():
    rng = np.random.default_rng(4)
    key = bf16_to_f64(_bf16(rng.standard_normal((1, D))))
    q = _bf16(rng.standard_normal((5, D)))
    o, lse = attention(q, key, SCALE)
    np.testing.assert_array_equal(o, np.repeat(key, 5, axis=0))
    o3, lse3 = attention(q, np.repeat(key, 3, axis=0), SCALE)
    np.testing.assert_allclose(o3, np.repeat(key, 5, axis=0), rtol=1e-15)
    np.testing.assert_allclose(lse3, lse + np.log(3.0), rtol=1e-14)


def test_lse_matches_scipy_and_output_is_convex():
    rng = np.random.default_rng(5)
    keys = rng.standard_normal((300, D))
    q = _bf16(rng.standard_normal((6, D)))
    o, lse = attention(q, keys, SCALE)
    logits = float(SCALE) * bf16_to_f64(q) @ keys.T
    np.testing.assert_allclose(lse, scipy.special.logsumexp(logits, axis=1), rtol=1e-14)
    assert np.all(o <= keys.max(axis=0) + 1e-12) and np.all(o >= keys.min(axis=0) - 1e-12)


def test_split_and_merge_identity():
    rng = np.random.default_rng(6)
    keys = rng.standard_normal((200, D))
    q = _bf16(rng.standard_normal((4, D)))
    o, lse = attention(q, keys, SCALE)
    o1, l1 = attention(q, keys[:77], SCALE)
    o2, l2 = attention(q, keys[77:], SCALE)
    lm = np.logaddexp(l1, l2)
    om = np.exp(l1 - lm)[:, None] * o1 + np.exp(l2 - lm)[:, None] * o2
    np.testing.assert_allclose(om, o, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lm, lse, rtol=1e-14)


def test_index_order_irrelevant_and_padding_skipped():
    rng = np.random.default_rng(7)
    T, m = 256, 4
    x, c = _cache(rng, T, m)
    q = _bf16(rng.standard_normal((4, D)))
    idx = np.array([5, 60, 3, 17, 40])
    a = sparse_attention(q, c["nope"], c["nscale"], c["rope"], idx, x, 0, T - 1, 8, SCALE, m, 64)
    b = sparse_attention(q, c["nope"], c["nscale"], c["rope"], np.concatenate([idx[::-1], [-1, -1]]),
                         x, 0, T - 1, 8, SCALE, m, 64)
    np.testing.assert_allclose(a[0], b[0], rtol=1e-13, atol=1e-15)


def test_causality_future_rows_do_not_matter():
    rng = np.random.default_rng(8)
    T, m = 256, 4
    x, c = _cache(rng, T, m)
    q = _bf16(rng.standard_normal((4, D)))
    p = 101                               # sees entries 0..24 and rows 94..101
    a = dense_attention(q, c["nope"], c["nscale"], c["rope"], x, 0, p, 8, SCALE, m, 64)
    x2 = x.copy()
    x2[p + 1:] = _bf16(rng.standard_normal((T - p - 1, D)) * 100)
    c2 = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in c.items()}
    c2["nope"][25:] = 0x77
    c2["nscale"][25:] = 140
    b = dense_attention(q, c2["nope"], c2["nscale"], c2["rope"], x2, 0, p, 8, SCALE, m, 64)
    np.testing.assert_array_equal(a[0], b[0])
    # an index beyond the visible range is skipped, not attended
    e = sparse_attention(q, c["nope"], c["nscale"], c["rope"], [3, 30], x, 0, p, 8, SCALE, m, 64)
    f = sparse_attention(q, c["nope"], c["nscale"], c["rope"], [3], x, 0, p, 8, SCALE, m, 64)
    np.testing.assert_array_equal(e[0], f[0])


def test_no_keys_gives_zero_and_minus_inf():
    q = _bf16(np.ones((2, D)))
    o, lse = sparse_attention(q, np.zeros((0, 256), np.uint8), np.zeros((0, 16), np.uint8),
                              np.zeros((0, 64), np.uint16), [-1], np.zeros((0, D), np.uint16), 0, 5, 0,
                              SCALE, 4, 0)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


@pytest.mark.parametrize("m", [4, 128])
def test_hca_equals_csa_with_every_block(m):
    rng = np.random.default_rng(9)
    T = 4 * m
    x, c = _cache(rng, T, m)
    q = _bf16(rng.standard_normal((3, D)))
    N = T // m
    for p in (m - 2, m - 1, 2 * m + 3, T - 1):
        a = dense_attention(q, c["nope"], c["nscale"], c["rope"], x, 0, p, 16, SCALE, m, N)
        b = sparse_attention(q, c["nope"], c["nscale"], c["rope"], np.arange(N), x, 0, p, 16, SCALE, m, N)
        np.testing.assert_array_equal(a[0], b[0])
