"""HIP path vs the oracle at the full sizes of the measured workloads.

The launch configurations are the ones the benchmark times.  Inputs come
from the seeded generators (synthetic cache planes for the stages after the
compressor, so that the oracle does not have to rebuild multi-GB caches);
where the oracle cannot afford every output, sampled outputs are compared
one by one.
"""

import numpy as np
import pytest
import torch

import compressed_sparse_attention_compressor_amd as csa
import oracle as O
from gpu_check import check_topk, compare_bf16_rounding, compare_mxfp4, compress_bounds, row_rel_err
from synth.workloads import (
    BATCHED_DECODE,
    CSA2_DECODE,
    CSA2_HIER_DECODE,
    HCA_DECODE,
    PREFILL,
    as_u16,
    params,
    queries,
    raw_rows,
    second_layer_window,
    synthetic_cache,
)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _cache_from(planes, w, n_entries):
    p = {k: v for k, v in planes.items()}
    p["n_entries"] = torch.tensor(n_entries, dtype=torch.int32, device=DEV)
    if "ikey" not in p:
        p["ikey"] = p["iscale"] = None
    return csa.Cache(w.B, planes["nope"].shape[1], w.m, w.d_idx, planes=p)


def _np(t):
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def _oracle_rows(planes_cpu, b, qs, t, idx_row, swa_u16, swa_pos0, p, w, n_entries, dense=False):
    qb = as_u16(qs["q"][b, t])
    if dense:
        return O.dense_attention(qb, planes_cpu["nope"][b], planes_cpu["nscale"][b], planes_cpu["rope"][b], swa_u16,
                                 swa_pos0, p, w.n_win, w.softmax_scale, w.m, n_entries)
    return O.sparse_attention(qb, planes_cpu["nope"][b], planes_cpu["nscale"][b], planes_cpu["rope"][b], idx_row,
                              swa_u16, swa_pos0, p, w.n_win, w.softmax_scale, w.m, n_entries)


def _cpu_planes(planes):
    out = {}
    for k, v in planes.items():
        out[k] = _np(v)
    return out


def test_batched_decode_128k_fullsize():
    """32 sequences x 32,768 entries: indexer + top-512 for every sequence,
    attention (bf16 output) for every sequence and head."""
    w = BATCHED_DECODE
    planes = synthetic_cache(w, device=DEV)
    pc = _cpu_planes(planes)
    cache = _cache_from(planes, w, [w.N] * w.B)
    qs = queries(w, device=DEV)
    scores = csa.index_scores(cache, qs["qI"], qs["w"], qs["q_pos"])
    idx, sc = csa.topk(cache, scores, qs["q_pos"], w.k, want_scores=True)
    x_win, _ = raw_rows(w, w.T - w.n_win, w.T, device=DEV)
    s0 = torch.full((w.B,), w.T - w.n_win, dtype=torch.int32, device=DEV)
    torch.cuda.synchronize()
    g_idx = _np(idx)
    o_idx = np.zeros_like(g_idx)
    qI, wt = _np(qs["qI"]), _np(qs["w"])
    # the combined entry point (scores in its workspace, then both selections)
    f_idx, f_sc = csa.index_topk(cache, qs["qI"], qs["w"], qs["q_pos"], w.k, want_scores=True)
    f_idx, f_sc = _np(f_idx), _np(f_sc)
    swaps = 0
    for b in range(w.B):
        oi, _, js, s = O.index_topk(pc["ikey"][b], pc["iscale"][b], qI[b, 0], wt[b, 0], w.T - 1, w.m, w.N, w.k)
        swaps += check_topk(g_idx[b, 0], oi, js, s, what=f"b={b}")
        swaps += check_topk(f_idx[b, 0], oi, js, s, what=f"index_topk b={b}")
        ref = dict(zip(js.tolist(), s.tolist()))
        r = np.array([ref[j] for j in f_idx[b, 0]])
        assert np.abs(f_sc[b, 0] - r).max() <= 1e-5 * (np.abs(s).max() + 1e-30)
        o_idx[b, 0] = oi
    assert swaps <= 4
    # attention stage-wise on the oracle's selection, as the benchmark launches it (bf16 out)
    out, lse = csa.sparse_attn(cache, qs["q"], qs["q_pos"], torch.from_numpy(o_idx).to(DEV), x_win, s0, w.n_win,
                               w.softmax_scale, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    g = O.bf16_to_f64(_np(out))
    xw = _np(x_win)
    worst = 0.0
    for b in range(w.B):
        o, l = _oracle_rows(pc, b, {"q": qs["q"].cpu()}, 0, o_idx[b, 0], xw[b], w.T - w.n_win, w.T - 1, w, w.N)
        worst = max(worst, float(row_rel_err(g[b, 0], o).max()))
        assert np.abs(_np(lse)[b, 0] - l).max() <= 1e-4 * max(1.0, np.abs(l).max())
    assert worst <= 2e-2, worst


def test_batched_decode_fused_append_fullsize():
    """The benchmark's fused decode append at full size (32 sequences x
    32,768 entries, the newest 4-token block compressed and every entry
    scored): cache bytes and all 1,048,576 scores identical to
    csa_compress followed by csa_index_scores."""
    w = BATCHED_DECODE
    planes = synthetic_cache(w, device=DEV)
    c1 = _cache_from(planes, w, [w.N] * w.B)
    c2 = _cache_from({k: v.clone() for k, v in planes.items()}, w, [w.N] * w.B)
    x, z = raw_rows(w, w.T - w.m, w.T, device=DEV)
    bias, wik = params(w, device=DEV)
    qs = queries(w, device=DEV)
    csa.compress(c1, x, z, bias, wik, tok_begin=w.T - w.m)
    s1 = csa.index_scores(c1, qs["qI"], qs["w"], qs["q_pos"])
    s2 = csa.compress_index_scores(c2, x, z, bias, wik, w.T - w.m, qs["qI"], qs["w"], qs["q_pos"])
    torch.cuda.synchronize()
    for plane in ("nope", "nscale", "rope", "ikey", "iscale"):
        a, b = getattr(c1, plane), getattr(c2, plane)
        assert torch.equal(a.view(torch.uint8) if a.dtype != torch.uint8 else a,
                           b.view(torch.uint8) if b.dtype != torch.uint8 else b), plane
    assert torch.equal(s1.view(torch.int32), s2.view(torch.int32))


def test_batched_decode_compress_fullsize_sampled():
    """The decode-step compressor launch (newest block of 32 sequences) and a
    4,096-token chunk of every sequence, compared entry by entry."""
    w = BATCHED_DECODE
    bias, wik = params(w, device=DEV)
    cache = csa.Cache(w.B, w.N, w.m, w.d_idx, device=DEV)
    t0 = w.T - 4096
    x, z = raw_rows(w, t0, w.T, device=DEV)
    csa.compress(cache, x, z, bias, wik, tok_begin=t0)
    torch.cuda.synchronize()
    ref = {k: _np(getattr(cache, k)).copy() for k in ("nope", "nscale", "rope", "ikey", "iscale")}
    # the decode launch: one block per sequence, entry N-1, must reproduce the same bytes
    csa.compress(cache, x[:, -w.m:].contiguous(), z[:, -w.m:].contiguous(), bias, wik, tok_begin=w.T - w.m)
    torch.cuda.synchronize()
    for k in ref:
        np.testing.assert_array_equal(_np(getattr(cache, k))[:, -1], ref[k][:, -1])
    xc, zc = _np(x), _np(z)
    W = as_u16(wik)
    e0 = t0 // w.m
    exempt = total = 0
    for b in range(0, w.B, 4):
        o = O.compress(xc[b], zc[b], bias.cpu().numpy(), W, w.m)
        pb = (8 + 2 * w.m) * 2.0 ** -22 * o["pooled_abs"]
        kb = 2.0 ** -14 * o["kI_abs"] + (8 + 2 * w.m) * 2.0 ** -22 * (o["pooled_abs"] @ np.abs(O.bf16_to_f64(W)))
        sl = slice(e0, w.N)
        exempt += compare_mxfp4(ref["nope"][b, sl], ref["nscale"][b, sl], o["nope"], o["nscale"],
                                o["pooled"][:, :512], pb[:, :512], f"nope b={b}")
        exempt += compare_bf16_rounding(ref["rope"][b, sl], o["pooled"][:, 512:], pb[:, 512:], "rope")
        exempt += compare_mxfp4(ref["ikey"][b, sl], ref["iscale"][b, sl], o["ikey"], o["iscale"], o["kI"], kb,
                                f"ikey b={b}")
        total += o["pooled"].size + o["kI"].size
    assert exempt <= 1e-4 * total + 4


def test_hca_decode_1m_fullsize():
    """8 sequences x 8,192 entries of m = 128, dense attention for every head."""
    w = HCA_DECODE
    planes = synthetic_cache(w, device=DEV)
    pc = _cpu_planes(planes)
    cache = _cache_from(planes, w, [w.N] * w.B)
    qs = queries(w, device=DEV)
    x_win, _ = raw_rows(w, w.T - w.n_win, w.T, device=DEV)
    s0 = torch.full((w.B,), w.T - w.n_win, dtype=torch.int32, device=DEV)
    out, lse = csa.hca_dense_attn(cache, qs["q"], qs["q_pos"], x_win, s0, w.n_win, w.softmax_scale,
                                  out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    g = O.bf16_to_f64(_np(out))
    xw = _np(x_win)
    qcpu = {"q": qs["q"].cpu()}
    for b in range(w.B):
        o, l = _oracle_rows(pc, b, qcpu, 0, None, xw[b], w.T - w.n_win, w.T - 1, w, w.N, dense=True)
        assert row_rel_err(g[b, 0], o).max() <= 2e-2
        assert np.abs(_np(lse)[b, 0] - l).max() <= 1e-4 * max(1.0, np.abs(l).max())


def test_csa2_two_layer_1m_fullsize():
    """4 sequences x 262,144 entries: layer A top-2048 over every entry,
    layer B rescoring A's selection to top-512 with its own queries, both
    attentions (the second over A's cache with its own window rows)."""
    w = CSA2_DECODE
    planes = synthetic_cache(w, device=DEV)
    pc = _cpu_planes(planes)
    cache = _cache_from(planes, w, [w.N] * w.B)
    qa = queries(w, device=DEV)
    qb = queries(w, device=DEV, second=True)
    ia, _ = csa.index_topk(cache, qa["qI"], qa["w"], qa["q_pos"], w.k)
    torch.cuda.synchronize()
    g_a = _np(ia)
    o_a = np.zeros_like(g_a)
    for b in range(w.B):
        oi, _, js, s = O.index_topk(pc["ikey"][b], pc["iscale"][b], _np(qa["qI"])[b, 0], _np(qa["w"])[b, 0],
                                    w.T - 1, w.m, w.N, w.k)
        check_topk(g_a[b, 0], oi, js, s, what=f"layer A b={b}")
        o_a[b, 0] = oi
    cand = torch.from_numpy(o_a).to(DEV)
    ib, _ = csa.index_topk(cache, qb["qI"], qb["w"], qb["q_pos"], w.k_b, cand=cand)
    torch.cuda.synchronize()
    g_b = _np(ib)
    o_b = np.zeros_like(g_b)
    for b in range(w.B):
        oi, _, js, s = O.index_topk(pc["ikey"][b], pc["iscale"][b], _np(qb["qI"])[b, 0], _np(qb["w"])[b, 0],
                                    w.T - 1, w.m, w.N, w.k_b, cand=o_a[b, 0])
        check_topk(g_b[b, 0], oi, js, s, what=f"layer B b={b}")
        o_b[b, 0] = oi
    x_win, _ = raw_rows(w, w.T - w.n_win, w.T, device=DEV)
    xb_win = second_layer_window(w, w.T - w.n_win, w.T, device=DEV)
    s0 = torch.full((w.B,), w.T - w.n_win, dtype=torch.int32, device=DEV)
    outs = []
    for qs, sel, win in ((qa, o_a, x_win), (qb, o_b, xb_win)):
        out, _ = csa.sparse_attn(cache, qs["q"], qs["q_pos"], torch.from_numpy(sel).to(DEV), win, s0, w.n_win,
                                 w.softmax_scale, out_dtype=torch.bfloat16)
        outs.append(out)
    torch.cuda.synchronize()
    for (qs, sel, win), out in zip(((qa, o_a, x_win), (qb, o_b, xb_win)), outs):
        g = O.bf16_to_f64(_np(out))
        wc = _np(win)
        for b in range(w.B):
            o, _ = _oracle_rows(pc, b, {"q": qs["q"].cpu()}, 0, sel[b, 0], wc[b], w.T - w.n_win, w.T - 1, w, w.N)
            assert row_rel_err(g[b, 0], o).max() <= 2e-2


def test_csa2_hier_pool_1m_fullsize():
    """4 sequences x 262,144 entries with the hierarchical pool: the Full
    layer's scores, its own top-512, the pool of the 2,048 best blocks of 8
    entries, the Reindex layer's top-512 over the 16,384 pool entries, and
    both attentions (the second over the shared cache with its own window)."""
    w = CSA2_HIER_DECODE
    planes = synthetic_cache(w, device=DEV)
    pc = _cpu_planes(planes)
    cache = _cache_from(planes, w, [w.N] * w.B)
    qa = queries(w, device=DEV)
    qb = queries(w, device=DEV, second=True)
    scores = csa.index_scores(cache, qa["qI"], qa["w"], qa["q_pos"])
    ia, _ = csa.topk(cache, scores, qa["q_pos"], w.k)
    pool = csa.index_pool(cache, scores, qa["q_pos"], w.pool_block, w.pool_blocks)
    ib, _ = csa.index_topk(cache, qb["qI"], qb["w"], qb["q_pos"], w.k_b, cand=pool)
    torch.cuda.synchronize()
    g_s, g_a, g_p, g_b = _np(scores), _np(ia), _np(pool), _np(ib)
    C = w.pool_block * w.pool_blocks
    assert g_p.shape == (w.B, 1, C)
    for b in range(w.B):
        oi, _, js, s = O.index_topk(pc["ikey"][b], pc["iscale"][b], _np(qa["qI"])[b, 0], _np(qa["w"])[b, 0],
                                    w.T - 1, w.m, w.N, w.k)
        check_topk(g_a[b, 0], oi, js, s, what=f"own top-k b={b}")
        ref, _ = O.block_pool(g_s[b, 0].astype(np.float64), w.N, w.pool_block, w.pool_blocks)
        np.testing.assert_array_equal(g_p[b, 0], ref, err_msg=f"pool b={b}")
        assert np.all(g_p[b, 0] >= 0)                 # every sequence fills the pool
        assert set(g_a[b, 0].tolist()) <= set(g_p[b, 0].tolist())
        ob, _, jb, sb = O.index_topk(pc["ikey"][b], pc["iscale"][b], _np(qb["qI"])[b, 0], _np(qb["w"])[b, 0],
                                     w.T - 1, w.m, w.N, w.k_b, cand=g_p[b, 0])
        check_topk(g_b[b, 0], ob, jb, sb, what=f"reindex b={b}")
    x_win, _ = raw_rows(w, w.T - w.n_win, w.T, device=DEV)
    xb_win = second_layer_window(w, w.T - w.n_win, w.T, device=DEV)
    s0 = torch.full((w.B,), w.T - w.n_win, dtype=torch.int32, device=DEV)
    runs = ((qa, g_a, x_win), (qb, g_b, xb_win))
    outs = [csa.sparse_attn(cache, qs["q"], qs["q_pos"], torch.from_numpy(sel).to(DEV), win, s0, w.n_win,
                            w.softmax_scale, out_dtype=torch.bfloat16)[0] for qs, sel, win in runs]
    torch.cuda.synchronize()
    for (qs, sel, win), out in zip(runs, outs):
        g = O.bf16_to_f64(_np(out))
        wc = _np(win)
        for b in range(w.B):
            o, _ = _oracle_rows(pc, b, {"q": qs["q"].cpu()}, 0, sel[b, 0], wc[b], w.T - w.n_win, w.T - 1, w, w.N)
            assert row_rel_err(g[b, 0], o).max() <= 2e-2


def test_prefill_64k_fullsize_sampled():
    """The whole 65,536-query prefill chunk (indexer with causal visibility,
    top-1024 per query, attention with the window), compared on sampled
    queries across the positions."""
    w = PREFILL
    planes = synthetic_cache(w, device=DEV)
    pc = _cpu_planes(planes)
    cache = _cache_from(planes, w, [w.N])
    qs = queries(w, device=DEV)
    idx, _ = csa.index_topk(cache, qs["qI"], qs["w"], qs["q_pos"], w.k)
    x, _ = raw_rows(w, 0, w.T, device=DEV)
    s0 = torch.zeros(1, dtype=torch.int32, device=DEV)
    out, lse = csa.sparse_attn(cache, qs["q"], qs["q_pos"], idx, x, s0, w.n_win, w.softmax_scale,
                               out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    sample = np.unique(np.concatenate([[0, 1, 2, 3, 4, 5, 7, 4095, 4096, 65535],
                                       rng.integers(0, w.T, 22)]))
    g_idx = _np(idx[0, torch.from_numpy(sample).to(DEV)])
    g_out = O.bf16_to_f64(_np(out[0, torch.from_numpy(sample).to(DEV)]))
    qI = _np(qs["qI"][0, torch.from_numpy(sample).to(DEV)])
    wt = _np(qs["w"][0, torch.from_numpy(sample).to(DEV)])
    qq = qs["q"][0, torch.from_numpy(sample).to(DEV)].cpu()
    xc = _np(x[0])
    for n, t in enumerate(sample):
        p = int(t)
        oi, _, js, s = O.index_topk(pc["ikey"][0], pc["iscale"][0], qI[n], wt[n], p, w.m, w.N, w.k)
        check_topk(g_idx[n], oi, js, s, what=f"query {p}")
        # the attention stage on the same cache bytes and the GPU's selection
        o, _ = O.sparse_attention(as_u16(qq[n]), pc["nope"][0], pc["nscale"][0], pc["rope"][0], g_idx[n], xc, 0, p,
                                  w.n_win, w.softmax_scale, w.m, w.N)
        assert row_rel_err(g_out[n], o).max() <= 2e-2, p


def _prefill_sample(T, m, rng, n_random):
    """Query positions of the prefill end-to-end check: the first tokens
    (nothing or little visible), positions around entry boundaries and around
    the compressor's 4,096-token chunk edges, the last token, and random ones."""
    edges = [0, 1, 2, 3, 4, 5, 6, 7, 8, 11, 12, 15, 16, 127, 128, 129, 130, 131]
    for t in (4096, 8192, 32768, 61440):
        edges += [t - m - 1, t - m, t - 2, t - 1, t, t + 1, t + m - 1, t + m]
    edges += [T - m - 1, T - m, T - 2, T - 1]
    pos = np.unique(np.concatenate([np.array(edges), rng.integers(0, T, n_random)]))
    return pos[(pos >= 0) & (pos < T)]


def test_prefill_64k_end_to_end():
    """The 65,536-token prefill chunk end to end ([V4] Fig. 3: compressor ->
    indexer -> top-k -> attention with the window): the GPU compresses the
    whole stream and every one of the 16,384 entries and indexer keys is
    compared with the oracle's compressor; then, on sampled queries, the
    GPU's selection against the oracle's indexer on the GPU's keys, the
    GPU's attention against the oracle on the GPU's cache and selection
    (stage-wise), and against the oracle pipeline run from the raw inputs
    alone (end to end)."""
    w = PREFILL
    bias, wik = params(w)
    x, z = raw_rows(w, 0, w.T)
    cache = csa.Cache(w.B, w.N, w.m, w.d_idx, device=DEV)
    cache.n_entries.fill_(w.N)
    xd = x.to(DEV)
    csa.compress(cache, xd, z.to(DEV), bias.to(DEV), wik.to(DEV))
    qs = queries(w, device=DEV)
    idx, _ = csa.index_topk(cache, qs["qI"], qs["w"], qs["q_pos"], w.k)
    s0 = torch.zeros(1, dtype=torch.int32, device=DEV)
    out, lse = csa.sparse_attn(cache, qs["q"], qs["q_pos"], idx, xd, s0, w.n_win, w.softmax_scale,
                               out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    # the compressor: all 16,384 entries and keys
    o = O.compress(as_u16(x[0]), as_u16(z[0]), bias.numpy(), as_u16(wik), w.m)
    pb, kb = compress_bounds(o, w.m, as_u16(wik))
    gn, gs, gr = _np(cache.nope[0]), _np(cache.nscale[0]), _np(cache.rope[0])
    gk, gks = _np(cache.ikey[0]), _np(cache.iscale[0])
    ex = compare_mxfp4(gn, gs, o["nope"], o["nscale"], o["pooled"][:, :512], pb[:, :512], "prefill nope")
    ex_k = compare_mxfp4(gk, gks, o["ikey"], o["iscale"], o["kI"], kb, "prefill ikey")
    rz = compare_bf16_rounding(gr, o["pooled"][:, 512:], pb[:, 512:], "prefill rope")
    print(f"prefill compressor: {ex} + {ex_k} exempted codes, {rz} rope roundings over {w.N} entries")
    assert ex + ex_k <= 1e-4 * w.N * (512 + w.d_idx)
    # sampled queries
    sample = _prefill_sample(w.T, w.m, np.random.default_rng(7), 260)
    assert len(sample) >= 256
    sel = torch.from_numpy(sample).to(DEV)
    g_idx = _np(idx[0, sel])
    g_out = O.bf16_to_f64(_np(out[0, sel]))
    g_lse = _np(lse[0, sel]).astype(np.float64)
    qI, wt = _np(qs["qI"][0, sel]), _np(qs["w"][0, sel])
    qq = qs["q"][0, sel].cpu()
    xc = as_u16(x[0])
    swaps = 0
    for n, t in enumerate(sample):
        p = int(t)
        qb = as_u16(qq[n])
        si, _, sj, ss = O.index_topk(gk, gks, qI[n], wt[n], p, w.m, w.N, w.k)
        check_topk(g_idx[n], si, sj, ss, what=f"stage-wise top-k, query {p}")
        so, sl = O.sparse_attention(qb, gn, gs, gr, g_idx[n], xc, 0, p, w.n_win, w.softmax_scale, w.m, w.N)
        assert row_rel_err(g_out[n], so).max() <= 2e-2, f"stage-wise attention, query {p}"
        assert np.abs(g_lse[n] - sl).max() <= 1e-4 * max(1.0, np.abs(sl).max()), f"stage-wise lse, query {p}"
        oi, _, oj, os_ = O.index_topk(o["ikey"], o["iscale"], qI[n], wt[n], p, w.m, w.N, w.k)
        swaps += check_topk(g_idx[n], oi, oj, os_, what=f"end-to-end top-k, query {p}")
        eo, _ = O.sparse_attention(qb, o["nope"], o["nscale"], o["rope"], oi, xc, 0, p, w.n_win, w.softmax_scale,
                                   w.m, w.N)
        assert row_rel_err(g_out[n], eo).max() <= 2e-2, f"end-to-end attention, query {p}"
    print(f"prefill: {len(sample)} queries compared stage-wise and end to end, {swaps} near-tie swaps")
