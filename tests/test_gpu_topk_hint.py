"""The top-k of decode rows from the indexer's histogram hint.

csa_index_topk and csa_compress_index_topk select decode rows (one to three
queries per sequence, at most 32,768 entries) from per-row counts of the
scores by the top 11 bits of their keys, written by the indexer launch: a
compaction launch keeps the keys in the threshold bin and above, a final
launch settles the selection.  The counts are checked against the scores,
so a workspace holding anything gives the same selection; a zero workspace
takes the hint path, a garbage one the fallback, and both leave the counts
zero.  Every case is compared with the oracle's selection rule.
"""

import numpy as np
import pytest
import torch

import compressed_sparse_attention_compressor_amd as csa
import oracle as O
from gpu_check import check_topk
from synth.workloads import Workload, params, queries, raw_rows, synthetic_cache

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _cache(w, N_cap, n_entries, kinds=None):
    planes = synthetic_cache(w, N_cap=N_cap)
    if kinds is not None:
        # only `kinds` distinct key rows: the scores take few values (crowded ties)
        sel = np.arange(N_cap) % kinds
        planes["ikey"] = planes["ikey"][:, sel].contiguous()
        planes["iscale"] = planes["iscale"][:, sel].contiguous()
    p = {k: v.to(DEV) for k, v in planes.items()}
    p["n_entries"] = torch.tensor(n_entries, dtype=torch.int32, device=DEV)
    return planes, csa.Cache(w.B, N_cap, w.m, w.d_idx, planes=p)


def _hint_region(w, Q, N_cap, ws):
    sbytes = w.B * Q * N_cap * 4
    off = (sbytes + 255) // 256 * 256
    return ws[off:off + w.B * Q * 2048 * 4].view(torch.int32)


HINT_CASES = [
    # (name, workload, N_cap, entries per sequence, positions [B][Q], k, distinct key rows or None)
    ("b8-32k", Workload("h1", 60, B=8, T=131072, m=4, d_idx=128, H_I=32, k=512, H=64, n_win=0), 32768,
     [32768, 32768, 30000, 32768, 1, 32768, 700, 32768], None, 512, None),
    ("q3-ragged", Workload("h2", 61, B=2, T=40000, m=4, d_idx=128, H_I=32, k=300, H=64, n_win=0, Q=3), 10000,
     [10000, 6001], [[39999, 17003, 2], [39999, 100, 24003]], 300, None),
    ("d64-k-over-visible", Workload("h3", 62, B=3, T=8192, m=4, d_idx=64, H_I=16, k=256, H=64, n_win=0), 2048,
     [2048, 200, 256], None, 256, None),
    ("crowded-ties", Workload("h4", 63, B=2, T=65536, m=4, d_idx=128, H_I=32, k=512, H=64, n_win=0), 16384,
     [16384, 9999], None, 512, 5),
    ("all-equal", Workload("h5", 64, B=1, T=16384, m=4, d_idx=128, H_I=32, k=100, H=64, n_win=0, Q=2), 4096,
     [4096], [[16383, 9000]], 100, 1),
]


@pytest.mark.parametrize("name,w,N_cap,n_ent,pos,k,kinds", HINT_CASES, ids=[c[0] for c in HINT_CASES])
def test_index_topk_hint_and_fallback(name, w, N_cap, n_ent, pos, k, kinds):
    planes, cache = _cache(w, N_cap, n_ent, kinds)
    qs = queries(w, device=DEV)
    Q = w.Q
    if pos is None:
        pos = np.full((w.B, Q), w.T - 1, np.int32)
    pos = np.asarray(pos, np.int32)
    qp = torch.from_numpy(pos).to(DEV)
    need = csa.workspace_bytes(csa.WS_INDEX_TOPK, w.B, Q, k, N_cap, 0)
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    garbage = torch.randint(0, 256, (need,), dtype=torch.uint8, device=DEV)
    results = []
    for label, buf in (("zero", ws), ("garbage", garbage), ("after garbage", garbage)):
        idx, sc = csa.index_topk(cache, qs["qI"], qs["w"], qp, k, want_scores=True, ws=buf)
        torch.cuda.synchronize()
        assert torch.count_nonzero(_hint_region(w, Q, N_cap, buf)) == 0, f"{label}: hint not left zero"
        results.append((label, idx.cpu().numpy(), sc.cpu().numpy()))
    for label, g, gs in results[1:]:
        np.testing.assert_array_equal(g, results[0][1], err_msg=label)
        np.testing.assert_array_equal(gs.view(np.int32), results[0][2].view(np.int32), err_msg=label)
    g = results[0][1]
    ik, isc = planes["ikey"].numpy(), planes["iscale"].numpy()
    for b in range(w.B):
        for t in range(Q):
            oi, _, js, s = O.index_topk(ik[b], isc[b], qs["qI"][b, t].cpu().numpy(), qs["w"][b, t].cpu().numpy(),
                                        int(pos[b, t]), w.m, n_ent[b], k)
            check_topk(g[b, t], oi, js, s, what=f"{name} b={b} t={t}")


def test_compress_index_topk_matches_separate_calls():
    """The decode front half (fused append + indexer with the hint, hinted
    top-k) against compress + index_scores + two-stage top-k: identical
    cache bytes, selections and selected scores."""
    w = Workload("hc", 65, B=4, T=32768, m=4, d_idx=128, H_I=32, k=512, H=64, n_win=0)
    N = w.N
    planes = synthetic_cache(w)
    n_ent = [N, N, N - 1, N]
    c1 = csa.Cache(w.B, N, w.m, w.d_idx, planes=dict({k: v.to(DEV) for k, v in planes.items()},
                   n_entries=torch.tensor(n_ent, dtype=torch.int32, device=DEV)))
    c2 = csa.Cache(w.B, N, w.m, w.d_idx, planes=dict({k: v.clone().to(DEV) for k, v in planes.items()},
                   n_entries=torch.tensor(n_ent, dtype=torch.int32, device=DEV)))
    tok0 = (N - 1) * w.m
    x, z = raw_rows(w, tok0, N * w.m, device=DEV)
    bias, wik = params(w, device=DEV)
    qs = queries(w, device=DEV)
    pos = torch.full((w.B, 1), N * w.m - 1, dtype=torch.int32, device=DEV)
    pos[3, 0] = N * w.m - 2                       # the new entry is not visible to this query
    sc = csa.compress_index_scores(c1, x, z, bias, wik, tok0, qs["qI"], qs["w"], pos)
    i1, s1 = csa.topk(c1, sc, pos, w.k, want_scores=True)
    for rep in range(2):                          # the second call reuses the workspace the first left
        ws = torch.zeros(csa.workspace_bytes(csa.WS_INDEX_TOPK, w.B, 1, w.k, N, 0), dtype=torch.uint8,
                         device=DEV) if rep == 0 else ws
        i2, s2 = csa.compress_index_topk(c2, x, z, bias, wik, tok0, qs["qI"], qs["w"], pos, w.k, want_scores=True,
                                         ws=ws)
        torch.cuda.synchronize()
        for plane in ("nope", "nscale", "rope", "ikey", "iscale"):
            a, b2 = getattr(c1, plane), getattr(c2, plane)
            assert torch.equal(a.view(torch.uint8), b2.view(torch.uint8)), plane
        assert torch.equal(i1, i2)
        assert torch.equal(s1.view(torch.int32), s2.view(torch.int32))
        assert torch.count_nonzero(_hint_region(w, 1, N, ws)) == 0
