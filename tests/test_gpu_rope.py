"""The fused rotary epilogue of the attention kernels against the oracle.

[V4.1] "推論カーネル": a fused RoPE-attention-RoPE-cast kernel; the rotation
and the positions follow the oracle's reading (query at p, compressed entry
j at (j+1)m - 1, window rows at their own positions, output turned back by
-p).  Cases cover sparse and dense attention, bf16 and FP8 window rows,
16, 64 and 128 heads, one split and several, fp32 and bf16 outputs, and
positions near 2^20 where the angles run to ~10^6 radians.
"""

import numpy as np
import pytest
import torch

import compressed_sparse_attention_compressor_amd as csa
import oracle as O
from gpu_check import row_rel_err
from synth import TensorId, normal_bf16
from synth.workloads import Workload, as_u16
from test_gpu_parity import DEV, TOL, _attn_inputs, _check_attn, _gpu_cache, _np

pytestmark = pytest.mark.gpu

CASES = [
    # (name, workload, N_cap, n_entries, positions, S, swa_pos0, dense, fp8 window, base)
    ("sparse-h64-splits", Workload("r1", 50, B=2, T=4000, m=4, d_idx=0, H_I=0, k=96, H=64, n_win=128, Q=2), 1000,
     [1000, 777], [[3999, 1500], [3103, 3999]], None, None, False, False, 10000.0),
    # positions near 2^20: entries far behind the query, the window buffer at the query
    ("sparse-h16-far", Workload("r2", 51, B=1, T=1048576, m=4, d_idx=0, H_I=0, k=64, H=16, n_win=128, Q=2), 500,
     [500], [[1048575, 1048500]], 300, [1048276], False, False, 1000000.0),
    ("dense-hca", Workload("r3", 52, B=2, T=8192, m=128, d_idx=0, H_I=0, k=0, H=64, n_win=128, Q=1), 64, [64, 50],
     [[8191], [7000]], None, None, True, False, 10000.0),
    ("sparse-w8", Workload("r4", 53, B=2, T=2000, m=4, d_idx=0, H_I=0, k=60, H=64, n_win=128, Q=2), 500,
     [500, 400], [[1999, 700], [1603, 1999]], 300, [1750, 1700], False, True, 10000.0),
    ("dense-w8-h32", Workload("r5", 54, B=1, T=8192, m=128, d_idx=0, H_I=0, k=0, H=32, n_win=64, Q=2), 64, [64],
     [[8191, 8000]], 256, [7936], True, True, 50000.0),
    ("sparse-h128", Workload("r6", 55, B=1, T=2000, m=4, d_idx=0, H_I=0, k=100, H=128, n_win=64, Q=2), 500, [500],
     [[1999, 700]], None, None, False, False, 10000.0),
]


def _selection(w, pos, n_entries, seed):
    rng = np.random.default_rng(seed)
    B, Q = pos.shape
    idx = np.full((B, Q, w.k), -1, np.int32)
    for b in range(B):
        for t in range(Q):
            V = O.visible_count(int(pos[b, t]), w.m, n_entries[b])
            n = min(w.k - 1, V)
            idx[b, t, :n] = np.sort(rng.choice(V, n, replace=False))
    return idx


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("name,w,N_cap,n_entries,pos,S,swa_pos0,dense,w8,base", CASES, ids=[c[0] for c in CASES])
def test_rope_attention_parity(name, w, N_cap, n_entries, pos, S, swa_pos0, dense, w8, base, dtype):
    pos = np.array(pos, np.int32)
    planes, qs, swa, s0 = _attn_inputs(w, N_cap, n_entries, pos, S, swa_pos0)
    B, Q = pos.shape
    cache = _gpu_cache(planes, B, N_cap, w.m, 0, n_entries)
    idx = None if dense else _selection(w, pos, n_entries, w.cfg)
    q, qp, s0d = qs["q"].to(DEV), torch.from_numpy(pos).to(DEV), torch.from_numpy(s0).to(DEV)
    kw = dict(out_dtype=dtype, rope_base=base)
    if w8:
        pl = csa.swa_encode(swa.to(DEV))
        if dense:
            out, lse = csa.hca_dense_attn_w8(cache, q, qp, pl, s0d, w.n_win, w.softmax_scale, **kw)
        else:
            out, lse = csa.sparse_attn_w8(cache, q, qp, torch.from_numpy(idx).to(DEV), pl, s0d, w.n_win,
                                          w.softmax_scale, **kw)
        rows = [O.swa_decode(*(_np(t)[b] for t in pl)) for b in range(B)]
    else:
        if dense:
            out, lse = csa.hca_dense_attn(cache, q, qp, swa.to(DEV), s0d, w.n_win, w.softmax_scale, **kw)
        else:
            out, lse = csa.sparse_attn(cache, q, qp, torch.from_numpy(idx).to(DEV), swa.to(DEV), s0d, w.n_win,
                                       w.softmax_scale, **kw)
        rows = [as_u16(swa[b]) for b in range(B)]
    torch.cuda.synchronize()
    nope, nsc, rope = planes["nope"].numpy(), planes["nscale"].numpy(), as_u16(planes["rope"])
    o = np.zeros((B, Q, w.H, 576))
    l = np.zeros((B, Q, w.H))
    for b in range(B):
        for t in range(Q):
            sel = np.arange(O.visible_count(int(pos[b, t]), w.m, n_entries[b])) if dense else idx[b, t]
            o[b, t], l[b, t] = O.sparse_attention(as_u16(qs["q"][b, t]), nope[b], nsc[b], rope[b], sel, rows[b],
                                                  int(s0[b]), int(pos[b, t]), w.n_win, w.softmax_scale, w.m,
                                                  n_entries[b], rope_base=base)
    _check_attn(out, lse, o, l, dtype, name)
    # the rotation matters: the unrotated result is far from the rotated one
    # in the positional channels
    plain = O.sparse_attention(as_u16(qs["q"][0, 0]), nope[0], nsc[0], rope[0],
                               np.arange(O.visible_count(int(pos[0, 0]), w.m, n_entries[0])) if dense else idx[0, 0],
                               rows[0], int(s0[0]), int(pos[0, 0]), w.n_win, w.softmax_scale, w.m, n_entries[0])[0]
    assert row_rel_err(o[0, 0][:, 512:], plain[:, 512:]).max() > 0.05, name


def test_rope_base_zero_is_the_plain_path():
    """rope_base = 0 reproduces the unrotated kernel bit for bit."""
    name, w, N_cap, n_entries, pos, S, swa_pos0 = CASES[0][:7]
    pos = np.array(pos, np.int32)
    planes, qs, swa, s0 = _attn_inputs(w, N_cap, n_entries, pos, S, swa_pos0)
    cache = _gpu_cache(planes, w.B, N_cap, w.m, 0, n_entries)
    idx = torch.from_numpy(_selection(w, pos, n_entries, 3)).to(DEV)
    args = (cache, qs["q"].to(DEV), torch.from_numpy(pos).to(DEV), idx, swa.to(DEV), torch.from_numpy(s0).to(DEV),
            w.n_win, w.softmax_scale)
    a, la = csa.sparse_attn(*args, out_dtype=torch.float32)
    b, lb = csa.sparse_attn(*args, out_dtype=torch.float32, rope_base=0.0)
    c, lc = csa.sparse_attn(*args, out_dtype=torch.float32, rope_base=10000.0)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(la, lb)
    assert not torch.equal(a, c)


def test_rope_layer_stack_matches_single_call():
    """A Full layer of the CSA2 stack with a rotary base equals
    csa_sparse_attn with the same base over the stack's selection."""
    w = Workload("r7", 56, B=2, T=4096, m=4, d_idx=64, H_I=4, k=64, H=64, n_win=128, Q=1)
    from synth.workloads import queries, synthetic_cache
    N_cap = 1024
    planes = synthetic_cache(w, N_cap=N_cap)
    n_entries = [1024, 900]
    cache = _gpu_cache(planes, w.B, N_cap, w.m, w.d_idx, n_entries)
    qs = queries(w)
    pos = torch.tensor([[4095], [3800]], dtype=torch.int32, device=DEV)
    swa = torch.stack([normal_bf16(w.seed, TensorId.SWA, (1, 4096, 576), first_seq=b)[0] for b in range(w.B)]).to(DEV)
    s0 = torch.zeros(w.B, dtype=torch.int32, device=DEV)
    L = dict(mode=csa.CSA2_FULL, cache=cache, qI=qs["qI"].to(DEV), w=qs["w"].to(DEV), k=w.k, q=qs["q"].to(DEV),
             swa=swa, swa_pos0=s0, n_win=w.n_win, scale=w.softmax_scale, out_dtype=torch.float32, rope_base=10000.0)
    r = csa.layer_stack([L], pos)[0]
    o, lo = csa.sparse_attn(cache, qs["q"].to(DEV), pos, r["idx"], swa, s0, w.n_win, w.softmax_scale,
                            out_dtype=torch.float32, rope_base=10000.0)
    torch.cuda.synchronize()
    assert torch.equal(r["out"], o) and torch.equal(r["lse"], lo)
