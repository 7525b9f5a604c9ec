"""Pins of the oracle's hierarchical candidate pool ([V4.1], "Hierarchical
Sparse Indexer" bullet and Fig. 5): a hand-worked example, the two special
cases that reduce to known results (block = 1 is the entry top-k; enough
blocks keep every visible entry), brute-force block ranking on small
inputs, and the nesting facts that make the pool useful (the Full layer's
own top-k lies inside it, so a Reindex layer asking with the same query
re-finds it)."""

import numpy as np
import pytest
import torch

from oracle import block_pool, hier_pair, index_topk, mxfp4_encode, topk_select


def _rounded_scores(rng, n, step):
    return np.round(rng.standard_normal(n) / step) * step


def test_hand_worked_example():
    # 10 visible entries in blocks of 4: [0..3], [4..7], [8, 9] (partial).
    s = np.array([0.1, 5.0, -1.0, 0.0, 2.0, 2.0, 2.0, 2.0, 5.0, -7.0])
    # block maxima 5, 2, 5: the two best are blocks 0 and 2
    pool, kept = block_pool(s, 10, 4, 2)
    assert list(kept) == [0, 2]
    assert list(pool) == [0, 1, 2, 3, 8, 9, -1, -1]
    # one block: the tie at 5 goes to the lower block
    pool, kept = block_pool(s, 10, 4, 1)
    assert list(kept) == [0]
    assert list(pool) == [0, 1, 2, 3]
    # an entry beyond V takes no part: with V = 9 block 2 holds entry 8 only
    pool, kept = block_pool(s, 9, 4, 3)
    assert list(kept) == [0, 1, 2]
    assert list(pool) == [0, 1, 2, 3, 4, 5, 6, 7, 8, -1, -1, -1]
    # block maxima of the first 8 entries only: 5 and 2
    pool, kept = block_pool(s, 8, 4, 1)
    assert list(pool) == [0, 1, 2, 3]
    # a negative block maximum still ranks by value
    s2 = np.array([-3.0, -4.0, -1.0, -2.0])
    pool, kept = block_pool(s2, 4, 2, 1)
    assert list(pool) == [2, 3]


@pytest.mark.parametrize("seed", range(4))
def test_block_one_is_entry_topk(seed):
    rng = np.random.default_rng(seed)
    V = 300 + seed * 17
    s = _rounded_scores(rng, V, 0.25)
    for n in (1, 7, 64, 299):
        pool, kept = block_pool(s, V, 1, n)
        ref, _ = topk_select(s, np.arange(V), n)
        np.testing.assert_array_equal(pool, ref)
        np.testing.assert_array_equal(kept, ref)


@pytest.mark.parametrize("block", [2, 3, 8])
def test_enough_blocks_keep_every_visible_entry(block):
    rng = np.random.default_rng(block)
    V = 101
    s = rng.standard_normal(V)
    nb = -(-V // block)
    for n in (nb, nb + 5):
        pool, kept = block_pool(s, V, block, n)
        np.testing.assert_array_equal(pool[:V], np.arange(V))
        assert np.all(pool[V:] == -1)
        np.testing.assert_array_equal(kept[:nb], np.arange(nb))
    pool, kept = block_pool(s, 0, block, 4)
    assert np.all(pool == -1) and np.all(kept == -1)


@pytest.mark.parametrize("seed,V,block,n", [(0, 50, 4, 5), (1, 37, 8, 2), (2, 64, 8, 8), (3, 200, 3, 30),
                                            (4, 9, 8, 1), (5, 120, 5, 40)])
def test_kept_blocks_outrank_dropped_brute_force(seed, V, block, n):
    rng = np.random.default_rng(seed)
    s = _rounded_scores(rng, V, 0.5)          # many exact ties
    pool, kept = block_pool(s, V, block, n)
    # block maxima by a plain loop over entries
    nb = (V + block - 1) // block
    bm = [max(s[j] for j in range(b * block, min(V, (b + 1) * block))) for b in range(nb)]
    ks = [int(b) for b in kept if b >= 0]
    assert len(ks) == min(n, nb)
    assert ks == sorted(ks)
    dropped = [b for b in range(nb) if b not in ks]
    for b in ks:
        for d in dropped:
            assert bm[b] > bm[d] or (bm[b] == bm[d] and b < d)
    # the pool is exactly the visible entries of the kept blocks, ascending
    members = [j for j in range(V) if j // block in ks]
    assert [int(j) for j in pool if j >= 0] == members
    assert np.all(pool[len(members):] == -1)


@pytest.mark.parametrize("seed", range(6))
def test_own_topk_lies_in_pool(seed):
    """Each of the k best entries lies in a block whose maximum ranks among
    the k best blocks, so with k <= n_blocks the pool holds the whole top-k
    (also under exact ties, both rules preferring the lower index)."""
    rng = np.random.default_rng(100 + seed)
    V = 1000 + 37 * seed
    s = _rounded_scores(rng, V, 0.1 if seed % 2 else 1.0)
    for block in (2, 8):
        for k, n in ((16, 16), (64, 100), (5, 5)):
            idx, _ = topk_select(s, np.arange(V), k)
            pool, _ = block_pool(s, V, block, n)
            assert set(idx[idx >= 0].tolist()) <= set(pool[pool >= 0].tolist())


def _small_cache(rng, N, d):
    kv = rng.standard_normal((N, d)).astype(np.float32)
    ik, isc = mxfp4_encode(kv)
    main = rng.standard_normal((N, 512)).astype(np.float32)
    nope, nscale = mxfp4_encode(main)
    rope = torch.from_numpy(rng.standard_normal((N, 64)).astype(np.float32)).to(torch.bfloat16)
    return dict(ikey=ik, iscale=isc, nope=nope, nscale=nscale,
                rope=rope.view(torch.int16).numpy().view(np.uint16))


def _layer(rng, H_I, d, H, n_rows):
    qI = torch.from_numpy(rng.standard_normal((H_I, d)).astype(np.float32) * 0.3).to(torch.float8_e4m3fn)
    q = torch.from_numpy(rng.standard_normal((H, 576)).astype(np.float32) * 0.05).to(torch.bfloat16)
    swa = torch.from_numpy(rng.standard_normal((n_rows, 576)).astype(np.float32)).to(torch.bfloat16)
    return dict(qI=qI.view(torch.uint8).numpy(), w=rng.standard_normal(H_I).astype(np.float32),
                q=q.view(torch.int16).numpy().view(np.uint16), swa=swa.view(torch.int16).numpy().view(np.uint16),
                swa_pos0=0)


def test_reindex_over_pool_refinds_own_topk():
    """A Reindex layer that asked with the Full layer's own indexer query
    would re-find the Full layer's top-k inside the pool, and its attention
    would equal the Full layer's."""
    rng = np.random.default_rng(7)
    N, d, m = 700, 64, 4
    cache = _small_cache(rng, N, d)
    a = _layer(rng, 4, d, 16, 64)
    p = 4 * 650 + 1                         # 650 entries visible
    r = hier_pair(cache, a, a, p, m, N, 16, 0.05, 32, 32, 8, 32)
    np.testing.assert_array_equal(r["idx_b"], r["idx_a"])
    np.testing.assert_array_equal(r["o_b"], r["o_a"])
    # the pool holds only visible entries
    assert r["pool"].max() < 650
    # a different query rescoring the pool selects from the pool only
    b = _layer(rng, 4, d, 16, 64)
    r2 = hier_pair(cache, a, b, p, m, N, 16, 0.05, 32, 16, 8, 32)
    assert set(r2["idx_b"][r2["idx_b"] >= 0].tolist()) <= set(r2["pool"][r2["pool"] >= 0].tolist())
    ref, _, _, _ = index_topk(cache["ikey"], cache["iscale"], b["qI"], b["w"], p, m, N, 16, cand=r2["pool"])
    np.testing.assert_array_equal(r2["idx_b"], ref)
