"""torch-facing wrappers of the C ABI: argument marshalling only.

Every step of the path runs in the HIP kernels of libcsa.so; these
functions pass device pointers, sizes and the current HIP stream.
"""

from __future__ import annotations

import ctypes

import torch

from ._lib import CacheT, Csa2LayerT, check, lib

D, D_NOPE, D_ROPE = 576, 512, 64
WS_INDEX_TOPK, WS_SPARSE_ATTN, WS_DENSE_ATTN, WS_TOPK, WS_INDEX_POOL = 0, 1, 2, 3, 4
OUT_F32, OUT_BF16 = 0, 1


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t, dtype, name):
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")


class Cache:
    """Planes of one compressed cache (caller-owned device memory).

    nope uint8 [B][N_cap][256], nscale uint8 [B][N_cap][16], rope bf16
    [B][N_cap][64], ikey uint8 [B][N_cap][d_idx/2], iscale uint8
    [B][N_cap][d_idx/32] (absent when d_idx = 0), n_entries int32 [B].
    """

    def __init__(self, B, N_cap, m, d_idx, device="cuda", planes=None):
        self.B, self.N_cap, self.m, self.d_idx = int(B), int(N_cap), int(m), int(d_idx)
        if planes is None:
            u8 = dict(dtype=torch.uint8, device=device)
            planes = dict(
                nope=torch.zeros(B, N_cap, D_NOPE // 2, **u8),
                nscale=torch.zeros(B, N_cap, D_NOPE // 32, **u8),
                rope=torch.zeros(B, N_cap, D_ROPE, dtype=torch.bfloat16, device=device),
                ikey=torch.zeros(B, N_cap, d_idx // 2, **u8) if d_idx else None,
                iscale=torch.zeros(B, N_cap, d_idx // 32, **u8) if d_idx else None,
                n_entries=torch.zeros(B, dtype=torch.int32, device=device),
            )
        for k, v in planes.items():
            setattr(self, k, v)

    def struct(self) -> CacheT:
        return CacheT(
            self.nope.data_ptr(), self.nscale.data_ptr(), self.rope.data_ptr(),
            self.ikey.data_ptr() if self.ikey is not None else None,
            self.iscale.data_ptr() if self.iscale is not None else None,
            self.n_entries.data_ptr(), self.B, self.N_cap, D_NOPE, D_ROPE, self.d_idx, self.m)


def workspace_bytes(op, B, Q, H, n_or_k, C=0) -> int:
    return int(lib().csa_workspace_bytes(op, B, Q, H, n_or_k, C))


def _workspace(nbytes, ws, device, zero=False):
    if nbytes == 0:
        return None, 0
    if ws is None:
        ws = (torch.zeros if zero else torch.empty)(nbytes, dtype=torch.uint8, device=device)
    return ws, ws.numel() * ws.element_size()


def compress(cache: Cache, x, z, pos_bias, w_ik=None, tok_begin=0):
    """Writes entries tok_begin/m .. (tok_begin+T)/m - 1 from x [B][T][576] and z [B][T][G]."""
    _need(x, torch.bfloat16, "x")
    _need(z, torch.bfloat16, "z")
    _need(pos_bias, torch.float32, "pos_bias")
    B, T = x.shape[0], x.shape[1]
    G = z.shape[2]
    if x.stride(2) != 1 or x.stride(1) != D or z.stride(2) != 1 or z.stride(1) != G:
        raise ValueError("x and z rows must be contiguous")
    if w_ik is not None:
        _need(w_ik, torch.bfloat16, "w_ik")
    cs = cache.struct()
    check(lib().csa_compress(_ptr(x), x.stride(0), _ptr(z), z.stride(0), G, _ptr(pos_bias), _ptr(w_ik),
                             int(tok_begin), int(T), ctypes.byref(cs), _stream()), "csa_compress")


def compress_hidden(cache: Cache, h, w_kv, w_z, pos_bias, w_ik=None, tok_begin=0, ws=None):
    """Compressor fed from hidden states: h bf16 [B][T][d_model], w_kv bf16
    [d_model][576], w_z bf16 [d_model][G] (G = 576 or 1), pos_bias fp32 [m];
    x = h w_kv and z = h w_z are pooled on the GPU without being written out.
    Writes entries tok_begin/m .. (tok_begin+T)/m - 1 (csa_compress_hidden)."""
    for t, n in ((h, "h"), (w_kv, "w_kv"), (w_z, "w_z")):
        _need(t, torch.bfloat16, n)
    if h.stride(2) != 1 or h.stride(1) != h.shape[2]:
        raise ValueError("h rows must be contiguous")
    B, T, d_model = h.shape
    G = w_z.shape[1]
    need = lib().csa_compress_hidden_ws_bytes(B, T, cache.m, int(w_ik is not None))
    ws, wsb = _workspace(need, ws, h.device)
    cs = cache.struct()
    check(lib().csa_compress_hidden(_ptr(h), h.stride(0), d_model, _ptr(w_kv), _ptr(w_z), G, _ptr(pos_bias),
                                    _ptr(w_ik), int(tok_begin), T, ctypes.byref(cs), _ptr(ws), wsb, _stream()),
          "csa_compress_hidden")
    return ws


def compress_index_scores(cache: Cache, x, z, pos_bias, w_ik, tok_begin, q_idx, w_idx, q_pos, scores=None):
    """compress() then a full-scan index_scores() (one launch for a one-entry decode append)."""
    _need(x, torch.bfloat16, "x")
    _need(z, torch.bfloat16, "z")
    _need(pos_bias, torch.float32, "pos_bias")
    _need(q_idx, torch.uint8, "q_idx")
    _need(w_idx, torch.float32, "w_idx")
    _need(q_pos, torch.int32, "q_pos")
    B, T = x.shape[0], x.shape[1]
    G = z.shape[2]
    if x.stride(2) != 1 or x.stride(1) != D or z.stride(2) != 1 or z.stride(1) != G:
        raise ValueError("x and z rows must be contiguous")
    if w_ik is not None:
        _need(w_ik, torch.bfloat16, "w_ik")
    Q, H_I = q_idx.shape[1], q_idx.shape[2]
    if scores is None:
        scores = torch.empty(B, Q, cache.N_cap, dtype=torch.float32, device=q_idx.device)
    cs = cache.struct()
    check(lib().csa_compress_index_scores(_ptr(x), x.stride(0), _ptr(z), z.stride(0), G, _ptr(pos_bias), _ptr(w_ik),
                                          int(tok_begin), int(T), ctypes.byref(cs), _ptr(q_idx), _ptr(w_idx), H_I,
                                          _ptr(q_pos), Q, _ptr(scores), scores.numel() * 4, _stream()),
          "csa_compress_index_scores")
    return scores


def index_topk(cache: Cache, q_idx, w_idx, q_pos, k, cand=None, want_scores=False, ws=None, out=None):
    """Returns (idx int32 [B][Q][k], scores fp32 [B][Q][k] or None)."""
    _need(q_idx, torch.uint8, "q_idx")
    _need(w_idx, torch.float32, "w_idx")
    _need(q_pos, torch.int32, "q_pos")
    B, Q, H_I = q_idx.shape[0], q_idx.shape[1], q_idx.shape[2]
    C = 0
    if cand is not None:
        _need(cand, torch.int32, "cand")
        C = cand.shape[2]
    dev = q_idx.device
    idx = out if out is not None else torch.empty(B, Q, k, dtype=torch.int32, device=dev)
    sc = torch.empty(B, Q, k, dtype=torch.float32, device=dev) if want_scores else None
    need = workspace_bytes(WS_INDEX_TOPK, B, Q, k, cache.N_cap, C)
    # a zeroed workspace lets the first call start from the indexer's hint
    ws, wsb = _workspace(need, ws, dev, zero=True)
    cs = cache.struct()
    check(lib().csa_index_topk(ctypes.byref(cs), _ptr(q_idx), _ptr(w_idx), H_I, _ptr(q_pos), Q, _ptr(cand), C, int(k),
                               _ptr(idx), _ptr(sc), _ptr(ws), wsb, _stream()), "csa_index_topk")
    return idx, sc


def compress_index_topk(cache: Cache, x, z, pos_bias, w_ik, tok_begin, q_idx, w_idx, q_pos, k, want_scores=False,
                        ws=None, out=None):
    """compress() then a full-scan index_topk(): the decode step's front half
    (append + indexer in one launch for a one-entry decode append, then the
    hinted top-k).  Returns (idx, scores or None)."""
    _need(x, torch.bfloat16, "x")
    _need(z, torch.bfloat16, "z")
    _need(pos_bias, torch.float32, "pos_bias")
    _need(q_idx, torch.uint8, "q_idx")
    _need(w_idx, torch.float32, "w_idx")
    _need(q_pos, torch.int32, "q_pos")
    B, T = x.shape[0], x.shape[1]
    G = z.shape[2]
    if x.stride(2) != 1 or x.stride(1) != D or z.stride(2) != 1 or z.stride(1) != G:
        raise ValueError("x and z rows must be contiguous")
    if w_ik is not None:
        _need(w_ik, torch.bfloat16, "w_ik")
    Q, H_I = q_idx.shape[1], q_idx.shape[2]
    dev = q_idx.device
    idx = out if out is not None else torch.empty(B, Q, k, dtype=torch.int32, device=dev)
    sc = torch.empty(B, Q, k, dtype=torch.float32, device=dev) if want_scores else None
    need = workspace_bytes(WS_INDEX_TOPK, B, Q, k, cache.N_cap, 0)
    ws, wsb = _workspace(need, ws, dev, zero=True)
    cs = cache.struct()
    check(lib().csa_compress_index_topk(_ptr(x), x.stride(0), _ptr(z), z.stride(0), G, _ptr(pos_bias), _ptr(w_ik),
                                        int(tok_begin), int(T), ctypes.byref(cs), _ptr(q_idx), _ptr(w_idx), H_I,
                                        _ptr(q_pos), Q, int(k), _ptr(idx), _ptr(sc), _ptr(ws), wsb, _stream()),
          "csa_compress_index_topk")
    return idx, sc


def index_scores(cache: Cache, q_idx, w_idx, q_pos, cand=None, scores=None):
    """Indexer stage alone: fp32 scores [B][Q][Ns] (Ns = N_cap, or C with candidates)."""
    _need(q_idx, torch.uint8, "q_idx")
    _need(w_idx, torch.float32, "w_idx")
    _need(q_pos, torch.int32, "q_pos")
    B, Q, H_I = q_idx.shape[0], q_idx.shape[1], q_idx.shape[2]
    C = cand.shape[2] if cand is not None else 0
    Ns = C if cand is not None else cache.N_cap
    if scores is None:
        scores = torch.empty(B, Q, Ns, dtype=torch.float32, device=q_idx.device)
    cs = cache.struct()
    check(lib().csa_index_scores(ctypes.byref(cs), _ptr(q_idx), _ptr(w_idx), H_I, _ptr(q_pos), Q, _ptr(cand), C,
                                 _ptr(scores), scores.numel() * 4, _stream()), "csa_index_scores")
    return scores


def topk(cache: Cache, scores, q_pos, k, cand=None, want_scores=False, out=None, ws=None):
    """Top-k stage alone, from the scores of index_scores()."""
    B, Q = q_pos.shape
    C = cand.shape[2] if cand is not None else 0
    dev = q_pos.device
    idx = out if out is not None else torch.empty(B, Q, k, dtype=torch.int32, device=dev)
    sc = torch.empty(B, Q, k, dtype=torch.float32, device=dev) if want_scores else None
    need = 0 if cand is not None else workspace_bytes(WS_TOPK, B, Q, k, cache.N_cap)
    ws, wsb = _workspace(need, ws, dev)
    cs = cache.struct()
    check(lib().csa_topk(ctypes.byref(cs), _ptr(scores), _ptr(q_pos), Q, _ptr(cand), C, int(k), _ptr(idx), _ptr(sc),
                         _ptr(ws), wsb, _stream()), "csa_topk")
    return idx, sc


def index_pool(cache: Cache, scores, q_pos, block, n_blocks, out=None, ws=None):
    """Hierarchical indexer candidate pool [B][Q][n_blocks*block] from full-scan scores."""
    B, Q = q_pos.shape
    dev = q_pos.device
    C = int(n_blocks) * int(block)
    pool = out if out is not None else torch.empty(B, Q, C, dtype=torch.int32, device=dev)
    need = workspace_bytes(WS_INDEX_POOL, B, Q, int(n_blocks), cache.N_cap, int(block))
    ws, wsb = _workspace(max(need, 16), ws, dev)
    cs = cache.struct()
    check(lib().csa_index_pool(ctypes.byref(cs), _ptr(scores), _ptr(q_pos), Q, int(block), int(n_blocks), _ptr(pool),
                               _ptr(ws), wsb, _stream()), "csa_index_pool")
    return pool


CSA2_FULL, CSA2_REINDEX, CSA2_REUSE = 0, 1, 2
CAND_AUTO, CAND_SCAN, CAND_SELECTION, CAND_POOL = 0, 1, 2, 3


def layer_stack(layers, q_pos, ws=None):
    """A stack of CSA2 layers (Full / Reindex / Reuse) in one call.

    ``layers``: dicts with ``mode`` and, as the mode needs them, ``cache``
    (Full), ``qI``, ``w``, ``k``, ``cand`` (Reindex), ``pool_block`` /
    ``pool_blocks`` (Full), and for every layer ``q``, ``swa``, ``swa_pos0``,
    ``n_win``, ``scale`` and optionally ``out_dtype``, ``out``, ``lse``,
    ``idx_out``, ``pool_out``, ``rope_base`` (0 = positional channels as
    stored; see sparse_attn).  Returns one dict per layer with ``out``,
    ``lse``, and ``idx`` / ``pool`` where the layer writes them.
    """
    B, Q = q_pos.shape
    dev = q_pos.device
    n = len(layers)
    arr = (Csa2LayerT * n)()
    keep, res = [], []
    for i, L in enumerate(layers):
        mode = int(L["mode"])
        q = L["q"]
        _need(q, torch.bfloat16, "q")
        H = q.shape[2]
        od = L.get("out_dtype", torch.bfloat16)
        r = {"out": L.get("out") if L.get("out") is not None else _attn_out(B, Q, H, od, dev, None)}
        r["lse"] = L.get("lse") if L.get("lse") is not None else torch.empty(B, Q, H, dtype=torch.float32, device=dev)
        e = arr[i]
        e.mode = mode
        e.cand = int(L.get("cand", CAND_AUTO))
        if mode == CSA2_FULL:
            cs = L["cache"].struct()
            keep.append(cs)
            e.cache = ctypes.pointer(cs)
        if mode != CSA2_REUSE:
            k = int(L["k"])
            r["idx"] = L.get("idx_out") if L.get("idx_out") is not None else torch.empty(
                B, Q, k, dtype=torch.int32, device=dev)
            e.q_idx, e.w_idx, e.H_I, e.k = _ptr(L["qI"]), _ptr(L["w"]), L["qI"].shape[2], k
            e.idx_out = _ptr(r["idx"])
        if mode == CSA2_FULL and int(L.get("pool_blocks", 0)) > 0:
            C = int(L["pool_blocks"]) * int(L["pool_block"])
            r["pool"] = L.get("pool_out") if L.get("pool_out") is not None else torch.empty(
                B, Q, C, dtype=torch.int32, device=dev)
            e.pool_block, e.pool_blocks = int(L["pool_block"]), int(L["pool_blocks"])
            e.pool_out = _ptr(r["pool"])
        swa = L.get("swa")
        e.q, e.H, e.n_win = _ptr(q), H, int(L["n_win"])
        e.swa, e.swa_pos0, e.S = _ptr(swa), _ptr(L.get("swa_pos0")), swa.shape[1] if swa is not None else 0
        e.softmax_scale = float(L["scale"])
        e.rope_base = float(L.get("rope_base", 0.0))
        e.out_dtype = OUT_BF16 if od == torch.bfloat16 else OUT_F32
        e.out, e.lse = _ptr(r["out"]), _ptr(r["lse"])
        res.append(r)
    L_ = lib()
    need = L_.csa2_stack_workspace_bytes(arr, n, Q)
    ws, wsb = _workspace(max(need, 16), ws, dev)
    check(L_.csa2_layer_stack(arr, n, _ptr(q_pos), Q, _ptr(ws), wsb, _stream()), "csa2_layer_stack")
    return res


def _attn_out(B, Q, H, out_dtype, dev, out):
    if out is not None:
        return out
    return torch.empty(B, Q, H, D, dtype=out_dtype, device=dev)


def sparse_attn(cache: Cache, q, q_pos, idx, swa, swa_pos0, n_win, scale, out_dtype=torch.bfloat16, ws=None,
                out=None, lse=None, rope_base=0.0):
    """Returns (out [B][Q][H][576], lse fp32 [B][Q][H]).  rope_base > 0
    applies the fused rotary epilogue (csa_sparse_attn in include/csa.h)."""
    _need(q, torch.bfloat16, "q")
    B, Q, H = q.shape[0], q.shape[1], q.shape[2]
    k = idx.shape[2] if idx is not None else 0
    S = swa.shape[1] if swa is not None else 0
    dev = q.device
    out = _attn_out(B, Q, H, out_dtype, dev, out)
    lse = lse if lse is not None else torch.empty(B, Q, H, dtype=torch.float32, device=dev)
    need = workspace_bytes(WS_SPARSE_ATTN, B, Q, H, k, n_win)
    ws, wsb = _workspace(need, ws, dev)
    cs = cache.struct()
    check(lib().csa_sparse_attn(ctypes.byref(cs), _ptr(q), H, _ptr(q_pos), Q, _ptr(idx), k, _ptr(swa), _ptr(swa_pos0),
                                S, int(n_win), float(scale), float(rope_base),
                                OUT_BF16 if out_dtype == torch.bfloat16 else OUT_F32, _ptr(out), _ptr(lse), _ptr(ws),
                                wsb, _stream()), "csa_sparse_attn")
    return out, lse


def hca_dense_attn(cache: Cache, q, q_pos, swa, swa_pos0, n_win, scale, out_dtype=torch.bfloat16, ws=None,
                   out=None, lse=None, rope_base=0.0):
    _need(q, torch.bfloat16, "q")
    B, Q, H = q.shape[0], q.shape[1], q.shape[2]
    S = swa.shape[1] if swa is not None else 0
    dev = q.device
    out = _attn_out(B, Q, H, out_dtype, dev, out)
    lse = lse if lse is not None else torch.empty(B, Q, H, dtype=torch.float32, device=dev)
    need = workspace_bytes(WS_DENSE_ATTN, B, Q, H, cache.N_cap, n_win)
    ws, wsb = _workspace(need, ws, dev)
    cs = cache.struct()
    check(lib().hca_dense_attn(ctypes.byref(cs), _ptr(q), H, _ptr(q_pos), Q, _ptr(swa), _ptr(swa_pos0), S,
                               int(n_win), float(scale), float(rope_base),
                               OUT_BF16 if out_dtype == torch.bfloat16 else OUT_F32, _ptr(out), _ptr(lse), _ptr(ws),
                               wsb, _stream()), "hca_dense_attn")
    return out, lse


def swa_encode(x, codes=None, scales=None, rope=None):
    """bf16 window rows x [B][S][576] -> FP8 window planes (codes uint8
    [B][S][512], scales uint8 [B][S][16], rope bf16 [B][S][64])."""
    _need(x, torch.bfloat16, "x")
    B, S = x.shape[0], x.shape[1]
    if x.stride(2) != 1 or x.stride(1) != D:
        raise ValueError("x rows must be contiguous")
    dev = x.device
    codes = codes if codes is not None else torch.empty(B, S, D_NOPE, dtype=torch.uint8, device=dev)
    scales = scales if scales is not None else torch.empty(B, S, D_NOPE // 32, dtype=torch.uint8, device=dev)
    rope = rope if rope is not None else torch.empty(B, S, D_ROPE, dtype=torch.bfloat16, device=dev)
    check(lib().csa_swa_encode(_ptr(x), x.stride(0), B, S, _ptr(codes), _ptr(scales), _ptr(rope), _stream()),
          "csa_swa_encode")
    return codes, scales, rope


def sparse_attn_w8(cache: Cache, q, q_pos, idx, swa8, swa_pos0, n_win, scale, out_dtype=torch.bfloat16, ws=None,
                   out=None, lse=None, rope_base=0.0):
    """sparse_attn with the window rows as the FP8 planes (codes, scales, rope) of swa_encode."""
    _need(q, torch.bfloat16, "q")
    B, Q, H = q.shape[0], q.shape[1], q.shape[2]
    k = idx.shape[2] if idx is not None else 0
    codes, scales, rope = swa8
    S = codes.shape[1]
    dev = q.device
    out = _attn_out(B, Q, H, out_dtype, dev, out)
    lse = lse if lse is not None else torch.empty(B, Q, H, dtype=torch.float32, device=dev)
    need = workspace_bytes(WS_SPARSE_ATTN, B, Q, H, k, n_win)
    ws, wsb = _workspace(need, ws, dev)
    cs = cache.struct()
    check(lib().csa_sparse_attn_w8(ctypes.byref(cs), _ptr(q), H, _ptr(q_pos), Q, _ptr(idx), k, _ptr(codes),
                                   _ptr(scales), _ptr(rope), _ptr(swa_pos0), S, int(n_win), float(scale),
                                   float(rope_base), OUT_BF16 if out_dtype == torch.bfloat16 else OUT_F32, _ptr(out), _ptr(lse),
                                   _ptr(ws), wsb, _stream()), "csa_sparse_attn_w8")
    return out, lse


def hca_dense_attn_w8(cache: Cache, q, q_pos, swa8, swa_pos0, n_win, scale, out_dtype=torch.bfloat16, ws=None,
                      out=None, lse=None, rope_base=0.0):
    """hca_dense_attn with the window rows as FP8 planes."""
    _need(q, torch.bfloat16, "q")
    B, Q, H = q.shape[0], q.shape[1], q.shape[2]
    codes, scales, rope = swa8
    S = codes.shape[1]
    dev = q.device
    out = _attn_out(B, Q, H, out_dtype, dev, out)
    lse = lse if lse is not None else torch.empty(B, Q, H, dtype=torch.float32, device=dev)
    need = workspace_bytes(WS_DENSE_ATTN, B, Q, H, cache.N_cap, n_win)
    ws, wsb = _workspace(need, ws, dev)
    cs = cache.struct()
    check(lib().hca_dense_attn_w8(ctypes.byref(cs), _ptr(q), H, _ptr(q_pos), Q, _ptr(codes), _ptr(scales), _ptr(rope),
                                  _ptr(swa_pos0), S, int(n_win), float(scale), float(rope_base),
                                  OUT_BF16 if out_dtype == torch.bfloat16 else OUT_F32, _ptr(out), _ptr(lse),
                                  _ptr(ws), wsb, _stream()), "hca_dense_attn_w8")
    return out, lse


FLAG_IDX_RANGE = 1
FLAG_IDX_ORDER = 2
FLAG_WINDOW = 4
FLAG_CAND = 8
FLAG_ENTRIES = 16


def read_device_flags() -> int:
    """Reads and clears the current GPU's fault word (CSA_FLAG_* bits) on the
    current stream; waits for that stream."""
    v = ctypes.c_uint32(0)
    check(lib().csa_read_device_flags(_stream(), ctypes.byref(v)), "csa_read_device_flags")
    return int(v.value)
