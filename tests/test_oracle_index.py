"""Pins of the oracle's indexer and top-k: closed forms, brute force, a library routine."""

import numpy as np
import pytest
import torch

from oracle import (
    e4m3_to_f64,
    index_scores,
    index_topk,
    mxfp4_decode,
    mxfp4_encode,
    topk_select,
    visible_count,
)


def _keys(rng, N, d):
    k = rng.standard_normal((N, d)).astype(np.float32)
    return mxfp4_encode(k)


def _qI(rng, H, d):
    v = torch.from_numpy(rng.standard_normal((H, d)).astype(np.float32) * 0.3)
    return v.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_visible_count_block_causal():
    # entry j is visible at p when its last raw token (j+1)m-1 is at or before p
    assert visible_count(0, 4, 100) == 0
    assert visible_count(2, 4, 100) == 0
    assert visible_count(3, 4, 100) == 1
    assert visible_count(4, 4, 100) == 1
    assert visible_count(7, 4, 100) == 2
    assert visible_count(4095, 4, 1024) == 1024
    assert visible_count(4095, 4, 10) == 10
    assert visible_count(127, 128, 8) == 1
    assert visible_count(-1, 1, 8) == 0


def test_one_hot_closed_form():
    d, H, N = 64, 4, 8
    kv = np.zeros((N, d), np.float32)
    kv[:, 5] = np.arange(N) - 3.0          # -3 .. 4, exact in MXFP4 at scale 1 for |v|<=4? use grid values
    kv[:, 5] = np.array([-3, -2, -1, 0, 1, 2, 3, 4], np.float32)
    ik, isc = mxfp4_encode(kv)
    q = np.zeros((H, d), np.float32)
    q[2, 5] = 1.0
    qI = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    w = np.array([7.0, -3.0, 0.5, 2.0], np.float32)
    s = index_scores(ik, isc, qI, w, np.arange(N))
    np.testing.assert_array_equal(s, 0.5 * np.maximum(kv[:, 5], 0))


def test_negative_dots_score_zero():
    rng = np.random.default_rng(0)
    d, H, N = 128, 8, 16
    kv = np.abs(rng.standard_normal((N, d))).astype(np.float32)
    ik, isc = mxfp4_encode(kv)
    qI = torch.from_numpy(-np.abs(rng.standard_normal((H, d))).astype(np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()
    s = index_scores(ik, isc, qI, rng.standard_normal(H).astype(np.float32), np.arange(N))
    np.testing.assert_array_equal(s, np.zeros(N))


def test_scores_match_torch_einsum():
    rng = np.random.default_rng(1)
    d, H, N = 128, 32, 300
    ik, isc = _keys(rng, N, d)
    qI = _qI(rng, H, d)
    w = rng.standard_normal(H).astype(np.float32)
    s = index_scores(ik, isc, qI, w, np.arange(N))
    k = torch.from_numpy(mxfp4_decode(ik, isc))
    q = torch.from_numpy(qI).view(torch.float8_e4m3fn).to(torch.float64)
    ref = torch.einsum("hd,nd->nh", q, k).clamp_min(0).mul(torch.from_numpy(w.astype(np.float64))).sum(1)
    np.testing.assert_allclose(s, ref.numpy(), rtol=1e-12, atol=1e-12)


def _brute_topk(scores, js, k):
    """Rank by counting: element i is kept when fewer than k elements beat it
    (a larger score, or an equal score at a lower entry index)."""
    keep = []
    for i in range(len(js)):
        beats = sum(1 for t in range(len(js))
                    if scores[t] > scores[i] or (scores[t] == scores[i] and js[t] < js[i]))
        if beats < k:
            keep.append(int(js[i]))
    return sorted(keep)


@pytest.mark.parametrize("seed", range(5))
def test_topk_matches_rank_counting(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 120))
    js = rng.permutation(500)[:n]
    scores = np.round(rng.standard_normal(n), 1)   # many exact ties
    for k in (1, 3, 17, n, n + 5):
        idx, sc = topk_select(scores, js, k)
        ref = _brute_topk(scores, js, k)
        assert list(idx[: len(ref)]) == ref
        assert np.all(idx[len(ref):] == -1)
        pos = {int(j): i for i, j in enumerate(js)}
        np.testing.assert_array_equal(sc[: len(ref)], [scores[pos[j]] for j in ref])


def test_ties_go_to_lower_index():
    scores = np.array([1.0, 2.0, 2.0, 2.0, 0.5])
    idx, _ = topk_select(scores, np.arange(5), 2)
    assert list(idx) == [1, 2]


def test_scale_of_weights_keeps_selection():
    rng = np.random.default_rng(2)
    d, H, N = 64, 4, 200
    ik, isc = _keys(rng, N, d)
    qI = _qI(rng, H, d)
    w = rng.standard_normal(H).astype(np.float32)
    a = index_topk(ik, isc, qI, w, 10_000, 4, N, 16)
    b = index_topk(ik, isc, qI, w * np.float32(8.0), 10_000, 4, N, 16)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_allclose(b[1], 8.0 * a[1], rtol=1e-15)


def test_causality_invisible_keys_ignored():
    rng = np.random.default_rng(3)
    d, H, N, m = 64, 4, 64, 4
    ik, isc = _keys(rng, N, d)
    qI = _qI(rng, H, d)
    w = rng.standard_normal(H).astype(np.float32)
    p = 4 * 20 + 1                      # sees entries 0..19
    a = index_topk(ik, isc, qI, w, p, m, N, 8)
    ik2, isc2 = ik.copy(), isc.copy()
    ik2[20:] = rng.integers(0, 256, ik2[20:].shape)
    isc2[20:] = 140
    b = index_topk(ik2, isc2, qI, w, p, m, N, 8)
    np.testing.assert_array_equal(a[0], b[0])
    assert a[0].max() < 20
    # fewer visible entries than k: all of them, then -1 padding
    c = index_topk(ik, isc, qI, w, 4 * 3 - 1, m, N, 8)
    assert list(c[0]) == [0, 1, 2] + [-1] * 5
    e = index_topk(ik, isc, qI, w, 2, m, N, 8)
    assert list(e[0]) == [-1] * 8


def test_reindex_nesting():
    """A second layer that used the first layer's query would re-find the
    first layer's own top-k_B inside the candidates ([V4.1] Fig. 4)."""
    rng = np.random.default_rng(4)
    d, H, N = 128, 8, 500
    ik, isc = _keys(rng, N, d)
    qI = _qI(rng, H, d)
    w = rng.standard_normal(H).astype(np.float32)
    idx_a, _, _, _ = index_topk(ik, isc, qI, w, 10 ** 6, 4, N, 64)
    idx_b, _, _, _ = index_topk(ik, isc, qI, w, 10 ** 6, 4, N, 16, cand=idx_a)
    ref, _, _, _ = index_topk(ik, isc, qI, w, 10 ** 6, 4, N, 16)
    np.testing.assert_array_equal(idx_b, ref)
    # keeping every candidate returns the candidate set
    qI2 = _qI(rng, H, d)
    all_b, _, _, _ = index_topk(ik, isc, qI2, w, 10 ** 6, 4, N, 64, cand=idx_a)
    np.testing.assert_array_equal(all_b, np.sort(idx_a))


def test_e4m3_queries_decode_exactly():
    rng = np.random.default_rng(5)
    q = _qI(rng, 4, 64)
    np.testing.assert_array_equal(
        e4m3_to_f64(q), torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float64).numpy())
