"""Pins of the oracle's fused rotary epilogue ([V4.1] "推論カーネル": a fused
RoPE-attention-RoPE-cast kernel; [V4] CSA paragraph: the positional channels
are kept in BF16).  The rotation is pinned by hand values, complex
multiplication and group laws; the rotated attention by torch SDPA over
operands rotated with complex numbers, by closed forms and by the
relative-position invariance the rotation exists for."""

import cmath
import math

import numpy as np
import torch
import torch.nn.functional as F

from oracle import (
    attention,
    bf16_to_f64,
    compress,
    decode_entries,
    f32_to_bf16,
    rope_rotate,
    sparse_attention,
)

D, DR = 576, 64
SCALE = np.float32(1.0 / 24.0)


def _bf16(a):
    return f32_to_bf16(np.asarray(a, np.float32))


def _complex_rot(x, pos, base):
    """Pairs (2i, 2i+1) as complex numbers times exp(i pos base^(-2i/d))."""
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    z = x[..., 0::2] + 1j * x[..., 1::2]
    f = np.array([cmath.exp(1j * p * base ** (-2.0 * i / d)) for p in np.ravel(pos) for i in range(d // 2)])
    z = z * f.reshape(np.shape(pos) + (d // 2,))
    out = np.empty(x.shape)
    out[..., 0::2], out[..., 1::2] = z.real, z.imag
    return out


def _to_bf16_f64(x):
    """Rounds float64 values to bf16 through float32 with torch's own cast."""
    t = torch.from_numpy(np.asarray(x, np.float64)).to(torch.float32).to(torch.bfloat16)
    return t.to(torch.float64).numpy()


def test_rotation_hand_values():
    # pair 0 turns by pos radians; pair 1 by pos * 10000^(-1/32) = pos * 10^(-1/8)
    x = np.zeros(DR)
    x[0] = 1.0
    r = rope_rotate(x, 1, 10000.0)
    assert abs(r[0] - math.cos(1.0)) < 1e-15 and abs(r[1] - math.sin(1.0)) < 1e-15
    assert np.all(r[2:] == 0.0)
    x = np.zeros(DR)
    x[3] = 2.0                      # second channel of pair 1
    r = rope_rotate(x, 5, 10000.0)
    t = 5 * 0.7498942093324559      # 10 ** (-0.125)
    assert abs(r[2] + 2.0 * math.sin(t)) < 1e-14 and abs(r[3] - 2.0 * math.cos(t)) < 1e-14
    assert np.count_nonzero(r) == 2
    # the last pair turns slowest: base^(-62/64)
    x = np.zeros(DR)
    x[62] = 1.0
    r = rope_rotate(x, 1000, 10000.0)
    t = 1000 * 10000.0 ** (-62 / 64)
    assert abs(r[62] - math.cos(t)) < 1e-14 and abs(r[63] - math.sin(t)) < 1e-14


def test_rotation_is_complex_multiplication():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((7, DR))
    pos = np.array([0, 1, 3, 127, 4095, 65535, 1048575])
    for base in (10000.0, 500000.0, 2.5):
        np.testing.assert_allclose(rope_rotate(x, pos, base), _complex_rot(x, pos, base), rtol=0, atol=1e-9)


def test_rotation_group_laws():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, DR))
    a, b = 1234, 98765
    np.testing.assert_array_equal(rope_rotate(x, 0, 10000.0), x)
    np.testing.assert_allclose(rope_rotate(rope_rotate(x, a, 10000.0), a, 10000.0, sign=-1.0), x, atol=1e-12)
    np.testing.assert_allclose(rope_rotate(rope_rotate(x, a, 10000.0), b, 10000.0), rope_rotate(x, a + b, 10000.0),
                               atol=1e-9)
    # each pair keeps its length
    r = rope_rotate(x, a, 10000.0)
    np.testing.assert_allclose(np.hypot(r[:, 0::2], r[:, 1::2]), np.hypot(x[:, 0::2], x[:, 1::2]), rtol=1e-13)


def test_dot_product_depends_on_relative_position_only():
    rng = np.random.default_rng(2)
    q, k = rng.standard_normal(DR), rng.standard_normal(DR)
    for (a, b, s) in [(10, 3, 1000), (700000, 699000, 12345), (5, 5, 77)]:
        d0 = rope_rotate(q, a, 10000.0) @ rope_rotate(k, b, 10000.0)
        d1 = rope_rotate(q, a + s, 10000.0) @ rope_rotate(k, b + s, 10000.0)
        assert abs(d0 - d1) <= 1e-9 * (np.abs(q) @ np.abs(k))
    # and it changes with the distance
    assert abs(rope_rotate(q, 10, 10000.0) @ rope_rotate(k, 3, 10000.0) - q @ k) > 1e-3


def test_rope_attention_is_sdpa_over_rotated_bf16_operands():
    """The fused epilogue equals: rotate q by p and every key by its position
    (complex multiplication), round both to bf16, SDPA with the rotated keys
    as values, rotate the output's positional channels back by -p."""
    rng = np.random.default_rng(3)
    H, n, base, p = 4, 23, 10000.0, 5000
    q_u16 = _bf16(rng.standard_normal((H, D)))
    keys = bf16_to_f64(_bf16(rng.standard_normal((n, D))))
    pos = np.sort(rng.choice(p + 1, n, replace=False))
    o, lse = attention(q_u16, keys, SCALE, rope=dict(base=base, p=p, pos=pos, d_rope=DR))

    q = bf16_to_f64(q_u16)
    qr, kr = q.copy(), keys.copy()
    qr[:, -DR:] = _to_bf16_f64(_complex_rot(q[:, -DR:], np.full(H, p), base))
    kr[:, -DR:] = _to_bf16_f64(_complex_rot(keys[:, -DR:], pos, base))
    ref = F.scaled_dot_product_attention(torch.from_numpy(qr)[None], torch.from_numpy(kr)[None],
                                         torch.from_numpy(kr)[None], scale=float(SCALE))[0].numpy()
    ref[:, -DR:] = _complex_rot(ref[:, -DR:], np.full(H, -p), base)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)
    lref = np.log(np.exp(float(SCALE) * (qr @ kr.T)).sum(axis=1))
    np.testing.assert_allclose(lse, lref, rtol=1e-12)


def test_rope_attention_single_key_closed_form():
    """One key: the softmax weight is 1, so the output is the key with its
    positional channels turned by pos - p (up to the bf16 rounding of the
    rotated key)."""
    rng = np.random.default_rng(4)
    key = bf16_to_f64(_bf16(rng.standard_normal((1, D))))
    q_u16 = _bf16(rng.standard_normal((2, D)))
    for P, p in [(3, 3), (3, 40), (1023, 4095)]:
        o, _ = attention(q_u16, key, SCALE, rope=dict(base=10000.0, p=p, pos=[P], d_rope=DR))
        np.testing.assert_array_equal(o[:, :-DR], np.broadcast_to(key[:, :-DR], (2, D - DR)))
        want = _complex_rot(key[0, -DR:], np.array(P - p), 10000.0)
        np.testing.assert_allclose(o[0, -DR:], want, rtol=0, atol=2.0 ** -8 * np.abs(key[0, -DR:]).max())
        if P == p:   # same position: the rotation and its inverse cancel up to the bf16 rounding
            np.testing.assert_allclose(o[1, -DR:], key[0, -DR:], rtol=0, atol=2.0 ** -8 * np.abs(key).max())


def test_rope_attention_zero_positional_channels_is_plain_attention():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((3, D))
    q[:, -DR:] = 0.0
    keys = bf16_to_f64(_bf16(rng.standard_normal((9, D))))
    keys[:, -DR:] = 0.0
    q_u16 = _bf16(q)
    o0, l0 = attention(q_u16, keys, SCALE)
    o1, l1 = attention(q_u16, keys, SCALE, rope=dict(base=10000.0, p=100, pos=np.arange(9) * 11, d_rope=DR))
    np.testing.assert_array_equal(o0, o1)
    np.testing.assert_array_equal(l0, l1)


def test_rope_attention_shift_invariance():
    """Shifting the query and every key by the same distance changes nothing
    but the bf16 rounding of the rotated operands."""
    rng = np.random.default_rng(6)
    H, n = 4, 31
    q_u16 = _bf16(rng.standard_normal((H, D)))
    keys = bf16_to_f64(_bf16(rng.standard_normal((n, D))))
    pos = np.sort(rng.choice(3000, n, replace=False))
    o0, l0 = attention(q_u16, keys, SCALE, rope=dict(base=10000.0, p=3000, pos=pos, d_rope=DR))
    for s in (1, 517, 200000):
        o1, l1 = attention(q_u16, keys, SCALE, rope=dict(base=10000.0, p=3000 + s, pos=pos + s, d_rope=DR))
        den = np.abs(o0).max(axis=1, keepdims=True)
        assert (np.abs(o1 - o0) / den).max() < 2e-2
        assert np.abs(l1 - l0).max() < 2e-2


def test_sparse_attention_positions_of_entries_and_window_rows():
    """Entry j sits at its last raw token (j+1)m - 1; a window row at its own
    position; the query at p."""
    rng = np.random.default_rng(7)
    T, m, H, p, n_win = 64, 4, 2, 37, 5
    x = _bf16(rng.standard_normal((T, D)))
    z = _bf16(rng.standard_normal((T, D)))
    c = compress(x, z, rng.standard_normal(m).astype(np.float32), None, m)
    q = _bf16(rng.standard_normal((H, D)))
    idx = np.array([0, 3, 8, -1])
    o, lse = sparse_attention(q, c["nope"], c["nscale"], c["rope"], idx, x, 0, p, n_win, SCALE, m, T // m,
                              rope_base=10000.0)
    ent = decode_entries(c["nope"][[0, 3, 8]], c["nscale"][[0, 3, 8]], c["rope"][[0, 3, 8]])
    win = bf16_to_f64(x[33:38])
    pos = np.array([3, 15, 35, 33, 34, 35, 36, 37])
    o2, l2 = attention(q, np.concatenate([ent, win]), SCALE, rope=dict(base=10000.0, p=p, pos=pos, d_rope=DR))
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, l2)
    # the window buffer may start later: rows keep their raw positions
    o3, _ = sparse_attention(q, c["nope"], c["nscale"], c["rope"], idx, x[35:], 35, p, n_win, SCALE, m, T // m,
                             rope_base=10000.0)
    o4, _ = attention(q, np.concatenate([ent, bf16_to_f64(x[35:38])]), SCALE,
                      rope=dict(base=10000.0, p=p, pos=np.array([3, 15, 35, 35, 36, 37]), d_rope=DR))
    np.testing.assert_array_equal(o3, o4)
