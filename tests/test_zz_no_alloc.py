"""csa_index_topk_noalloc (the allocation-free variant of csa_index_topk,
whose workspace is the library's fixed per-GPU scratch) against
csa_index_topk with a workspace of its own, through the C ABI: identical
selections and selected scores, bit for bit, on two calls in a row, the
second with a smaller input."""

import ctypes

import numpy as np
import pytest
import torch

import compressed_sparse_attention_compressor_amd as csa
from compressed_sparse_attention_compressor_amd._lib import lib
from synth.workloads import Workload, queries, synthetic_cache

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _case(w, N_cap, n_ent):
    planes = synthetic_cache(w, N_cap=N_cap)
    p = {k: v.to(DEV) for k, v in planes.items()}
    p["n_entries"] = torch.tensor(n_ent, dtype=torch.int32, device=DEV)
    cache = csa.Cache(w.B, N_cap, w.m, w.d_idx, planes=p)
    return cache, queries(w, device=DEV)


def _noalloc(cache, qs, k):
    B, Q, H_I = qs["qI"].shape[:3]
    idx = torch.full((B, Q, k), -7, dtype=torch.int32, device=DEV)
    sc = torch.full((B, Q, k), -7.0, dtype=torch.float32, device=DEV)
    cs = cache.struct()
    st = lib().csa_index_topk_noalloc(ctypes.byref(cs), qs["qI"].data_ptr(), qs["w"].data_ptr(), H_I,
                                      qs["q_pos"].data_ptr(), Q, None, 0, k, idx.data_ptr(), sc.data_ptr(),
                                      torch.cuda.current_stream().cuda_stream)
    assert st == 0, lib().csa_status_str(st)
    return idx, sc


@pytest.mark.parametrize("first,second", [
    # the batched 128K decode shape, then a smaller ragged one
    ((Workload("na1", 70, B=32, T=131072, m=4, d_idx=128, H_I=32, k=512, H=64, n_win=0, prescaled=True), 32768,
      None), (Workload("na2", 71, B=3, T=8000, m=4, d_idx=64, H_I=16, k=100, H=64, n_win=0, Q=2), 2000,
              [2000, 123, 1999])),
])
def test_noalloc_matches_index_topk(first, second):
    for w, N_cap, n_ent in (first, second):
        n_ent = n_ent or [N_cap] * w.B
        cache, qs = _case(w, N_cap, n_ent)
        ref_i, ref_s = csa.index_topk(cache, qs["qI"], qs["w"], qs["q_pos"], w.k, want_scores=True)
        got_i, got_s = _noalloc(cache, qs, w.k)
        torch.cuda.synchronize()
        assert torch.equal(got_i, ref_i), w.name
        assert torch.equal(got_s.view(torch.int32), ref_s.view(torch.int32)), w.name
        # the selections are real ones (ascending, -1 padded) for every row
        g = got_i.cpu().numpy().reshape(-1, w.k)
        for row in g:
            v = row[row >= 0]
            assert np.all(np.diff(v) > 0) and np.all(row[len(v):] == -1)
