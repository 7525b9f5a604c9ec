"""Pins of the oracle's CSA2 layer stack ([V4.1], CSA2 paragraph and Fig. 4:
Full, Reindex and Reuse layers; Fig. 5: the hierarchical pool).  Each pin
checks where a layer takes its cache, candidates and selection from, against
the single-layer functions pinned elsewhere, on cases built so that the
wrong source gives a different answer."""

import numpy as np
import pytest
import torch

from oracle import (
    CAND_AUTO,
    CAND_POOL,
    CAND_SCAN,
    CAND_SELECTION,
    FULL,
    REINDEX,
    REUSE,
    block_pool,
    csa2_pair,
    csa2_stack,
    index_topk,
    mxfp4_encode,
    sparse_attention,
)
from oracle.formats import e4m3_to_f64, mxfp4_decode

M, NWIN, SCALE = 4, 16, 0.05


def _cache(rng, N, d=64, n_entries=None):
    ik, isc = mxfp4_encode(rng.standard_normal((N, d)).astype(np.float32))
    nope, nscale = mxfp4_encode(rng.standard_normal((N, 512)).astype(np.float32))
    rope = torch.from_numpy(rng.standard_normal((N, 64)).astype(np.float32)).to(torch.bfloat16)
    return dict(ikey=ik, iscale=isc, nope=nope, nscale=nscale, rope=rope.view(torch.int16).numpy().view(np.uint16),
                n_entries=N if n_entries is None else n_entries)


def _q(rng, H_I=4, d=64, H=16, rows=64):
    qI = torch.from_numpy(rng.standard_normal((H_I, d)).astype(np.float32) * 0.3).to(torch.float8_e4m3fn)
    q = torch.from_numpy(rng.standard_normal((H, 576)).astype(np.float32) * 0.05).to(torch.bfloat16)
    swa = torch.from_numpy(rng.standard_normal((rows, 576)).astype(np.float32)).to(torch.bfloat16)
    return dict(qI=qI.view(torch.uint8).numpy(), w=rng.standard_normal(H_I).astype(np.float32),
                q=q.view(torch.int16).numpy().view(np.uint16), swa=swa.view(torch.int16).numpy().view(np.uint16),
                swa_pos0=0, scale=SCALE)


P = 4 * 600 + 3        # 601 entries visible


def _attend(c, L, idx):
    return sparse_attention(L["q"], c["nope"], c["nscale"], c["rope"], idx, L["swa"], L["swa_pos0"], P, NWIN,
                            SCALE, M, c["n_entries"])


def test_single_full_layer_is_index_topk_then_attention():
    rng = np.random.default_rng(1)
    c = _cache(rng, 700)
    a = _q(rng)
    r = csa2_stack([dict(mode=FULL, cache=c, k=40, **a)], P, M, NWIN)[0]
    idx, _, _, _ = index_topk(c["ikey"], c["iscale"], a["qI"], a["w"], P, M, 700, 40)
    np.testing.assert_array_equal(r["idx"], idx)
    o, lse = _attend(c, a, idx)
    np.testing.assert_array_equal(r["o"], o)
    np.testing.assert_array_equal(r["lse"], lse)
    assert "pool" not in r


def test_reuse_takes_the_latest_selection():
    """Full (k=64) -> Reindex (k=16, its own query) -> Reuse: the Reuse layer
    attends to the Reindex selection, not to the Full layer's."""
    rng = np.random.default_rng(2)
    c = _cache(rng, 700)
    a, b, u = _q(rng), _q(rng), _q(rng)
    rs = csa2_stack([dict(mode=FULL, cache=c, k=64, **a),
                     dict(mode=REINDEX, k=16, cand=CAND_SELECTION, **b),
                     dict(mode=REUSE, **u)], P, M, NWIN)
    np.testing.assert_array_equal(rs[2]["idx"], rs[1]["idx"])
    o, _ = _attend(c, u, rs[1]["idx"])
    np.testing.assert_array_equal(rs[2]["o"], o)
    o_wrong, _ = _attend(c, u, rs[0]["idx"])
    assert not np.allclose(rs[2]["o"], o_wrong)
    # the Reindex selection nests in the Full layer's
    assert set(rs[1]["idx"].tolist()) <= set(rs[0]["idx"].tolist())
    # a Reuse layer asking with the index-producing layer's own query gives its output
    rr = csa2_stack([dict(mode=FULL, cache=c, k=64, **a), dict(mode=REUSE, **a)], P, M, NWIN)
    np.testing.assert_array_equal(rr[1]["o"], rr[0]["o"])


def test_candidate_sources():
    rng = np.random.default_rng(3)
    c = _cache(rng, 700)
    a, b = _q(rng), _q(rng)
    full = dict(mode=FULL, cache=c, k=32, pool_block=8, pool_blocks=12, **a)
    scan = csa2_stack([full, dict(mode=REINDEX, k=24, cand=CAND_SCAN, **b)], P, M, NWIN)
    ref, _, _, _ = index_topk(c["ikey"], c["iscale"], b["qI"], b["w"], P, M, 700, 24)
    np.testing.assert_array_equal(scan[1]["idx"], ref)
    pool = csa2_stack([full, dict(mode=REINDEX, k=24, cand=CAND_POOL, **b)], P, M, NWIN)
    auto = csa2_stack([full, dict(mode=REINDEX, k=24, cand=CAND_AUTO, **b)], P, M, NWIN)
    np.testing.assert_array_equal(pool[1]["idx"], auto[1]["idx"])
    pl = pool[0]["pool"]
    _, _, js, s = index_topk(c["ikey"], c["iscale"], a["qI"], a["w"], P, M, 700, 32)
    np.testing.assert_array_equal(pl, block_pool(s, len(js), 8, 12)[0])
    assert set(pool[1]["idx"].tolist()) <= set(pl[pl >= 0].tolist())
    ref, _, _, _ = index_topk(c["ikey"], c["iscale"], b["qI"], b["w"], P, M, 700, 24, cand=pl)
    np.testing.assert_array_equal(pool[1]["idx"], ref)
    sel = csa2_stack([full, dict(mode=REINDEX, k=24, cand=CAND_SELECTION, **b)], P, M, NWIN)
    ref, _, _, _ = index_topk(c["ikey"], c["iscale"], b["qI"], b["w"], P, M, 700, 24, cand=sel[0]["idx"])
    np.testing.assert_array_equal(sel[1]["idx"], ref)
    # without a pool, AUTO rescores the selection
    nopool = dict(mode=FULL, cache=c, k=32, **a)
    a2 = csa2_stack([nopool, dict(mode=REINDEX, k=24, **b)], P, M, NWIN)
    np.testing.assert_array_equal(a2[1]["idx"], sel[1]["idx"])
    # a full scan with the Full layer's own query re-finds its selection
    again = csa2_stack([nopool, dict(mode=REINDEX, k=32, cand=CAND_SCAN, **a)], P, M, NWIN)
    np.testing.assert_array_equal(again[1]["idx"], again[0]["idx"])


def test_second_full_layer_switches_cache_and_drops_pool():
    rng = np.random.default_rng(4)
    c1, c2 = _cache(rng, 700), _cache(rng, 700, n_entries=650)
    a, b, d = _q(rng), _q(rng), _q(rng)
    rs = csa2_stack([dict(mode=FULL, cache=c1, k=32, pool_block=8, pool_blocks=10, **a),
                     dict(mode=FULL, cache=c2, k=48, **b),
                     dict(mode=REINDEX, k=20, cand=CAND_AUTO, **d),
                     dict(mode=REUSE, **d)], P, M, NWIN)
    # AUTO after a Full layer without a pool rescores that layer's selection on its cache
    ref, _, _, _ = index_topk(c2["ikey"], c2["iscale"], d["qI"], d["w"], P, M, 650, 20, cand=rs[1]["idx"])
    np.testing.assert_array_equal(rs[2]["idx"], ref)
    o, _ = _attend(c2, d, rs[2]["idx"])
    np.testing.assert_array_equal(rs[3]["o"], o)
    o_wrong, _ = _attend(c1, d, rs[2]["idx"])
    assert not np.allclose(rs[3]["o"], o_wrong)
    with pytest.raises(ValueError):
        csa2_stack([dict(mode=FULL, cache=c1, k=32, pool_block=8, pool_blocks=10, **a),
                    dict(mode=FULL, cache=c2, k=48, **b),
                    dict(mode=REINDEX, k=20, cand=CAND_POOL, **d)], P, M, NWIN)


def test_invalid_stacks():
    rng = np.random.default_rng(5)
    a = _q(rng)
    with pytest.raises(ValueError):
        csa2_stack([dict(mode=REUSE, **a)], P, M, NWIN)
    with pytest.raises(ValueError):
        csa2_stack([dict(mode=REINDEX, k=8, **a)], P, M, NWIN)
    with pytest.raises(ValueError):
        csa2_stack([dict(mode=FULL, cache=_cache(rng, 100), k=8, **a), dict(mode=REINDEX, k=8, cand=CAND_POOL, **a)],
                   P, M, NWIN)


def test_csa2_pair_against_the_definition():
    """Full then Reindex ([V4.1] Fig. 4) for one query: layer B's selection is
    the k_b best of layer A's selection under B's own indexer query, scored
    here entry by entry from the indexer's definition (sum over heads of
    w_h * ReLU(q_h . k_j) on the decoded keys); the same query at the same k
    reproduces layer A; k_b at or above A's count keeps all of A."""
    rng = np.random.default_rng(6)
    c = _cache(rng, 700)
    a, b = _q(rng), _q(rng)
    r = csa2_pair(c, a, b, P, M, 700, NWIN, SCALE, 64, 16)
    sel_a = r["idx_a"][r["idx_a"] >= 0]
    sel_b = r["idx_b"][r["idx_b"] >= 0]
    assert len(sel_a) == 64 and len(sel_b) == 16
    assert set(sel_b.tolist()) <= set(sel_a.tolist())
    keys = mxfp4_decode(c["ikey"], c["iscale"])
    qI = e4m3_to_f64(b["qI"])
    wb = b["w"].astype(np.float64)
    score = {}
    for j in sel_a.tolist():
        score[j] = sum(wb[h] * max(0.0, float(np.dot(qI[h], keys[j]))) for h in range(len(wb)))
    best = sorted(score, key=lambda j: (-score[j], j))[:16]
    assert sorted(best) == sorted(sel_b.tolist())
    # layer B attends with its own query and window over the shared cache
    o, lse = sparse_attention(b["q"], c["nope"], c["nscale"], c["rope"], r["idx_b"], b["swa"], b["swa_pos0"], P,
                              NWIN, SCALE, M, 700)
    np.testing.assert_array_equal(r["o_b"], o)
    np.testing.assert_array_equal(r["lse_b"], lse)
    same = csa2_pair(c, a, a, P, M, 700, NWIN, SCALE, 64, 64)
    np.testing.assert_array_equal(same["idx_b"], same["idx_a"])
    np.testing.assert_array_equal(same["o_b"], same["o_a"])
    wide = csa2_pair(c, a, b, P, M, 700, NWIN, SCALE, 64, 100)
    assert set(wide["idx_b"][wide["idx_b"] >= 0].tolist()) == set(sel_a.tolist())
