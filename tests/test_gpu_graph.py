"""The benchmark times the path from HIP graphs.  A graph of one decode step
(the fused append + indexer, the two-stage top-k, the hierarchical pool,
split attention and its merge with a bf16 window, the FP8 window encode and
the attention reading it, dense attention whose merge spreads its splits
over four lanes) and of a radix top-k over long rows is replayed
several times, with eager runs of the same calls on the same workspaces and
unrelated GPU work between the replays.  Every replay must give the eager
results bit for bit: no stale workspace state carried between launches, no
memset nodes, nothing that depends on the capture stream."""

import pytest
import torch

import compressed_sparse_attention_compressor_amd as csa
from synth import TensorId, normal_f32
from synth.workloads import Workload, params, queries, raw_rows, synthetic_cache

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _bits(t):
    if t.dtype in (torch.bfloat16, torch.int16):
        return t.view(torch.int16)
    if t.dtype == torch.uint8:
        return t
    return t.view(torch.int32)


def test_graph_replays_match_eager():
    w = Workload("gr", 26, B=4, T=32768, m=4, d_idx=128, H_I=32, k=64, H=64, n_win=32)
    N = w.N
    planes = {k: v.to(DEV) for k, v in synthetic_cache(w).items()}
    # sequence 2 has not published the appended entry, sequence 3 sees few entries
    planes["n_entries"] = torch.tensor([N, N, N - 3, 5000], dtype=torch.int32, device=DEV)
    cache = csa.Cache(w.B, N, w.m, w.d_idx, planes=planes)
    x, z = raw_rows(w, w.T - w.m, w.T)
    x, z = x.to(DEV), z.to(DEV)
    bias, wik = params(w)
    bias, wik = bias.to(DEV), wik.to(DEV)
    qs = {k: v.to(DEV) for k, v in queries(w).items()}
    win, _ = raw_rows(w, w.T - w.n_win, w.T)
    win = win.to(DEV)
    s0 = torch.full((w.B,), w.T - w.n_win, dtype=torch.int32, device=DEV)

    # two rows of 1,048,576 scores (m = 1: entry j visible when j <= position):
    # few rows this long take the multi-workgroup radix selection
    LN, LK = 1 << 20, 2048
    long_sc = normal_f32(77, TensorId.W, (2, LN)).to(DEV).view(2, 1, LN)
    long_cache = csa.Cache(2, LN, 1, 0, planes=dict(
        nope=torch.zeros(2, 1, 256, dtype=torch.uint8, device=DEV),
        nscale=torch.zeros(2, 1, 16, dtype=torch.uint8, device=DEV),
        rope=torch.zeros(2, 1, 64, dtype=torch.bfloat16, device=DEV), ikey=None, iscale=None,
        n_entries=torch.full((2,), LN, dtype=torch.int32, device=DEV)))
    long_pos = torch.tensor([[LN - 1], [400000]], dtype=torch.int32, device=DEV)

    PB, PN = 8, 64
    sizes = dict(topk=csa.workspace_bytes(csa.WS_TOPK, w.B, 1, w.k, N),
                 attn=csa.workspace_bytes(csa.WS_SPARSE_ATTN, w.B, 1, w.H, w.k, w.n_win),
                 pool=csa.workspace_bytes(csa.WS_INDEX_POOL, w.B, 1, PN, N, PB),
                 radix=csa.workspace_bytes(csa.WS_TOPK, 2, 1, LK, LN),
                 dense=csa.workspace_bytes(csa.WS_DENSE_ATTN, w.B, 1, w.H, N, w.n_win))
    # the paths under test: two-stage and radix top-k, split attention
    assert sizes["topk"] > 0 and sizes["attn"] > 0 and sizes["radix"] > 0
    ws = {k: torch.empty(max(v, 16), dtype=torch.uint8, device=DEV) for k, v in sizes.items()}

    def outputs():
        u8 = dict(dtype=torch.uint8, device=DEV)
        return dict(scores=torch.empty(w.B, 1, N, dtype=torch.float32, device=DEV),
                    idx=torch.empty(w.B, 1, w.k, dtype=torch.int32, device=DEV),
                    pool=torch.empty(w.B, 1, PN * PB, dtype=torch.int32, device=DEV),
                    out=torch.empty(w.B, 1, w.H, 576, dtype=torch.bfloat16, device=DEV),
                    lse=torch.empty(w.B, 1, w.H, dtype=torch.float32, device=DEV),
                    codes=torch.empty(w.B, w.n_win, 512, **u8),
                    scales=torch.empty(w.B, w.n_win, 16, **u8),
                    rope=torch.empty(w.B, w.n_win, 64, dtype=torch.bfloat16, device=DEV),
                    out8=torch.empty(w.B, 1, w.H, 576, dtype=torch.float32, device=DEV),
                    lse8=torch.empty(w.B, 1, w.H, dtype=torch.float32, device=DEV),
                    lidx=torch.empty(2, 1, LK, dtype=torch.int32, device=DEV),
                    dout=torch.empty(w.B, 1, w.H, 576, dtype=torch.float32, device=DEV),
                    dlse=torch.empty(w.B, 1, w.H, dtype=torch.float32, device=DEV))

    def step(o):
        o["scores"].fill_(0.0)   # slots the indexer leaves unwritten start from a fixed value
        csa.compress_index_scores(cache, x, z, bias, wik, w.T - w.m, qs["qI"], qs["w"], qs["q_pos"],
                                  scores=o["scores"])
        csa.topk(cache, o["scores"], qs["q_pos"], w.k, out=o["idx"], ws=ws["topk"])
        csa.index_pool(cache, o["scores"], qs["q_pos"], PB, PN, out=o["pool"], ws=ws["pool"])
        csa.sparse_attn(cache, qs["q"], qs["q_pos"], o["idx"], win, s0, w.n_win, w.softmax_scale,
                        out_dtype=torch.bfloat16, ws=ws["attn"], out=o["out"], lse=o["lse"])
        sw8 = csa.swa_encode(win, codes=o["codes"], scales=o["scales"], rope=o["rope"])
        csa.sparse_attn_w8(cache, qs["q"], qs["q_pos"], o["idx"], sw8, s0, w.n_win, w.softmax_scale,
                           out_dtype=torch.float32, ws=ws["attn"], out=o["out8"], lse=o["lse8"])
        csa.topk(long_cache, long_sc, long_pos, LK, out=o["lidx"], ws=ws["radix"])
        # dense attention over every entry: 52 splits per row, merged four
        # lanes per output group in two rounds of loads per lane
        csa.hca_dense_attn(cache, qs["q"], qs["q_pos"], win, s0, w.n_win, w.softmax_scale,
                           out_dtype=torch.float32, ws=ws["dense"], out=o["dout"], lse=o["dlse"])

    ref = outputs()
    step(ref)
    torch.cuda.synchronize()
    assert bool((ref["idx"] >= 0).all()) and bool((ref["lidx"][0] >= 0).all())
    assert torch.isfinite(ref["lse"]).all() and torch.isfinite(ref["lse8"]).all()
    assert torch.isfinite(ref["dlse"]).all()

    g_out = outputs()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up on a side stream, as graph capture expects
        step(g_out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(g_out)
    torch.cuda.synchronize()

    eager = outputs()
    for rep in range(3):
        for v in g_out.values():
            v.zero_()
        graph.replay()
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(_bits(g_out[k]), _bits(ref[k])), f"replay {rep}: {k}"
        # eager work between the replays: the same calls into other outputs
        # (the shared workspaces are rewritten), then an unrelated kernel
        step(eager)
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(_bits(eager[k]), _bits(ref[k])), f"eager {rep}: {k}"
        torch.randn(1 << 20, device=DEV).sum().item()
