"""The compressed sparse attention path, one sequence and one query at a time.

Notation: D = d_nope + d_rope channels per KV row (512 + 64 in every
workload); m tokens fold into one compressed entry; entry j covers raw
positions [j*m, (j+1)*m); a query at raw position p (0-based) sees entry j
when (j+1)*m - 1 <= p and j is below the sequence's entry count.

Readings of the pages taken here (each is listed with its reason in the
design notes of the repository):

* Pooling [V4, "ハイブリッド注意：CSAとHCA", CSA paragraph and Fig. 3]:
  softmax-gated pooling with a learned positional bias.  The gate logit z is
  a per-token, per-channel stream of the same shape as the KV rows (the
  parallel projections C and Z of [V4.1], CED paragraph, eq. 1); a single
  gate channel (G = 1) is broadcast.  The bias b_i (one value per slot i of
  the m-token block) is added to the logit, and the softmax runs over the m
  tokens of the block independently per channel.  Blocks do not overlap
  ([V4.1], CSA2 paragraph: CSA2 drops the overlap of compressed entries).
* Indexer key [V4.1], CSA2 paragraph: the indexer key is a projection of
  the main KV entry; it is taken from the pooled entry before quantisation,
  kI = W_IK^T c, and stored in MXFP4 like the main entry.
* Indexer score [V4], CSA paragraph: FP4 keys, ReLU-scored multi-head dot
  product; one key per entry shared by all indexer heads, per-head weights
  w_h of any sign: s_j = sum_h w_h * max(0, qI_h . kI_j).
* Top-k: the min(k, |visible|) entries of largest score, exact ties to the
  lower entry index, returned in ascending entry order and padded with -1.
* Attention [V4], Fig. 3 and Fig. 4: one softmax over the union of the
  selected (or, for HCA, all visible) compressed entries and the sliding
  window of raw rows at positions max(0, p - n_win + 1) .. p; the key and
  the value are the same full D-channel decoded entry.  Without a rotary
  base the positional channels are data.
* Fused RoPE epilogue ([V4.1], "推論カーネル" bullet: a fused
  RoPE-attention-RoPE-cast kernel; [V4], CSA paragraph: the positional
  channels are stored in BF16), taken when a rotary base is given: the
  last d_rope channels of the query, of every key and of every window row
  are rotated as adjacent pairs (2i, 2i+1) by the angle pos * base^(-2i /
  d_rope), the rotation of the original rotary embedding; the query's
  position is p, a compressed entry's is its last raw token (j+1)*m - 1,
  a window row's is its own raw position.  The rotated operands are
  rounded to bf16, the precision the channels are stored in, and the same
  rotated key is the value.  After the softmax-weighted sum, the output's
  positional channels are rotated back by -p; the cast to the output type
  follows.
"""

from __future__ import annotations

import numpy as np

from .formats import (
    bf16_to_f64,
    e4m3_to_f64,
    f32_to_bf16,
    mxfp4_decode,
    mxfp4_encode,
    mxfp8_decode,
    mxfp8_encode,
)


def visible_count(p: int, m: int, n_entries: int) -> int:
    """Number of compressed entries visible to a query at raw position p."""
    if p < 0:
        return 0
    return int(max(0, min(int(n_entries), (int(p) + 1) // int(m))))


def pool_block(x_rows: np.ndarray, z_rows: np.ndarray, bias: np.ndarray) -> np.ndarray:
    """Softmax-gated pooling of one m-token block.

    x_rows: float64 [m][D]; z_rows: float64 [m][G] with G = D or 1;
    bias: float64 [m].  Returns c[d] = sum_i softmax_i(z[i, d] + bias[i]) * x[i, d].
    """
    a = z_rows + bias[:, None]
    a = np.broadcast_to(a, x_rows.shape)
    e = np.exp(a - a.max(axis=0, keepdims=True))
    w = e / e.sum(axis=0, keepdims=True)
    return (w * x_rows).sum(axis=0)


def compress(x_u16, z_u16, bias_f32, w_ik_u16, m: int, d_nope: int = 512) -> dict:
    """Compressor of one sequence: raw rows -> compressed cache planes.

    x_u16 bf16 bits [T][D]; z_u16 bf16 bits [T][G]; bias_f32 [m];
    w_ik_u16 bf16 bits [D][d_idx] or None (no indexer keys, as in HCA).
    T must be a multiple of m.  The quantisation decisions are taken on the
    float32 rounding of the float64 pooled value, the precision in which the
    GPU kernel holds it (the pages fix no precision for this step).

    Returns a dict with the cache planes (``nope`` uint8 [N][d_nope/2],
    ``nscale`` uint8 [N][d_nope/32], ``rope`` uint16 [N][D-d_nope],
    ``ikey`` uint8 [N][d_idx/2], ``iscale`` uint8 [N][d_idx/32]) and the
    float64 intermediates ``pooled`` [N][D], ``pooled_abs`` (sum of the
    absolute weighted terms, a bound on the size of the rounding error of any
    evaluation order), ``kI`` [N][d_idx] and ``kI_abs``.
    """
    return _compress_rows(bf16_to_f64(x_u16), bf16_to_f64(z_u16), bias_f32, w_ik_u16, m, d_nope)


def compress_hidden(h_u16, w_kv_u16, w_z_u16, bias_f32, w_ik_u16, m: int, d_nope: int = 512) -> dict:
    """Compressor fed from hidden states ([V4.1] "アーキテクチャ", CED
    paragraph, eq. 1: a decoder layer's KV entries C^l, Z^l are projected
    from the encoder's last hidden state H^{L/2} by W^KV_l, W^Z_l).

    h_u16 bf16 bits [T][d_model]; w_kv_u16 bf16 bits [d_model][D]; w_z_u16
    bf16 bits [d_model][G] (G = D or 1).  The raw rows are x = H W^KV and the
    gate logits z = H W^Z, exact products summed in float64 and used at that
    precision (they are never rounded to a stream format: the projection
    feeds the pooling directly); everything after is ``compress``.  Returns
    ``compress``'s dict.
    """
    h = bf16_to_f64(h_u16)
    return _compress_rows(h @ bf16_to_f64(w_kv_u16), h @ bf16_to_f64(w_z_u16), bias_f32, w_ik_u16, m, d_nope)


def _compress_rows(x, z, bias_f32, w_ik_u16, m: int, d_nope: int) -> dict:
    """The compressor on float64 raw rows x [T][D] and gate logits z [T][G]."""
    bias = np.asarray(bias_f32, dtype=np.float32).astype(np.float64)
    T, D = x.shape
    if T % m:
        raise ValueError("T must be a multiple of m")
    if bias.shape != (m,):
        raise ValueError("one bias value per block slot")
    N = T // m
    G = z.shape[1]
    xb = x.reshape(N, m, D)
    zb = z.reshape(N, m, G)
    a = np.broadcast_to(zb + bias[None, :, None], (N, m, D))
    e = np.exp(a - a.max(axis=1, keepdims=True))
    w = e / e.sum(axis=1, keepdims=True)
    pooled = (w * xb).sum(axis=1)
    pooled_abs = (w * np.abs(xb)).sum(axis=1)

    c32 = pooled.astype(np.float32)
    nope, nscale = mxfp4_encode(c32[:, :d_nope])
    rope = f32_to_bf16(c32[:, d_nope:])
    out = dict(pooled=pooled, pooled_abs=pooled_abs, nope=nope, nscale=nscale, rope=rope,
               ikey=None, iscale=None, kI=None, kI_abs=None)
    if w_ik_u16 is not None:
        W = bf16_to_f64(w_ik_u16)
        kI = pooled @ W
        out["kI"] = kI
        out["kI_abs"] = np.abs(pooled) @ np.abs(W)
        out["ikey"], out["iscale"] = mxfp4_encode(kI.astype(np.float32))
    return out


def decode_entries(nope, nscale, rope) -> np.ndarray:
    """Cache planes of some entries -> float64 [n][d_nope + d_rope]."""
    return np.concatenate([mxfp4_decode(nope, nscale), bf16_to_f64(rope)], axis=-1)


def index_scores(ikey, iscale, qI_u8, w_f32, js) -> np.ndarray:
    """Lightning-indexer scores of entries ``js`` for one query.

    ikey uint8 [N][d_idx/2], iscale uint8 [N][d_idx/32] (MXFP4 keys);
    qI_u8 E4M3 codes [H_I][d_idx]; w_f32 [H_I].
    s_j = sum_h w_h * max(0, qI_h . kI_j), all in float64 from exact decodes.
    """
    js = np.asarray(js, dtype=np.int64)
    k = mxfp4_decode(np.asarray(ikey)[js], np.asarray(iscale)[js])
    q = e4m3_to_f64(qI_u8)
    w = np.asarray(w_f32, dtype=np.float32).astype(np.float64)
    dots = k @ q.T
    return (np.maximum(dots, 0.0) * w[None, :]).sum(axis=1)


def topk_select(scores, js, k: int) -> tuple[np.ndarray, np.ndarray]:
    """Top-k of (score, entry) pairs: largest scores, ties to the lower entry.

    Returns (idx int32 [k] ascending and padded with -1, score of each
    selected entry in the same order, NaN in the padding).
    """
    scores = np.asarray(scores, dtype=np.float64)
    js = np.asarray(js, dtype=np.int64)
    order = np.lexsort((js, -scores))
    take = order[: min(int(k), len(js))]
    sel = np.sort(js[take])
    pos = {int(j): i for i, j in enumerate(js)}
    idx = np.full(int(k), -1, dtype=np.int32)
    sc = np.full(int(k), np.nan, dtype=np.float64)
    idx[: len(sel)] = sel
    sc[: len(sel)] = [scores[pos[int(j)]] for j in sel]
    return idx, sc


def index_topk(ikey, iscale, qI_u8, w_f32, p: int, m: int, n_entries: int, k: int, cand=None):
    """Indexer plus top-k for one query at raw position p.

    Without ``cand`` every visible entry is scored.  With ``cand`` (the
    entries an earlier layer selected, -1 meaning none; [V4.1] Fig. 4,
    Reindex mode) only the visible candidates are rescored; repeated
    candidates count once.  Returns (idx [k], selected scores [k], all
    scored entries, their scores).
    """
    V = visible_count(p, m, n_entries)
    if cand is None:
        js = np.arange(V, dtype=np.int64)
    else:
        c = np.asarray(cand, dtype=np.int64)
        js = np.unique(c[(c >= 0) & (c < V)])
    s = index_scores(ikey, iscale, qI_u8, w_f32, js) if len(js) else np.zeros(0)
    idx, sc = topk_select(s, js, k)
    return idx, sc, js, s


def block_pool(scores, V: int, block: int, n_blocks: int) -> tuple[np.ndarray, np.ndarray]:
    """Candidate pool of the hierarchical sparse indexer for one query
    ([V4.1], "Hierarchical Sparse Indexer" bullet and Fig. 5).

    ``scores`` float [>= V]: the Full layer's indexer scores of the visible
    entries 0..V-1.  Entries fall into blocks of ``block`` consecutive
    entries (block b holds entries b*block .. b*block + block - 1; the last
    visible block may be partly visible).  A block's score is the largest
    score among its visible entries.  The ``n_blocks`` blocks of largest
    score are kept, exact ties going to the lower block (the top-k rule), and
    the pool lists every visible entry of the kept blocks in ascending order,
    padded with -1 to n_blocks * block slots.

    Returns (pool int32 [n_blocks*block], kept blocks int32 [n_blocks],
    ascending and padded with -1).
    """
    scores = np.asarray(scores, dtype=np.float64)
    V, block, n_blocks = int(V), int(block), int(n_blocks)
    nb = -(-V // block)
    starts = np.arange(nb, dtype=np.int64) * block
    bmax = np.maximum.reduceat(scores[:V], starts) if nb else np.zeros(0)
    kept, _ = topk_select(bmax, np.arange(nb), n_blocks)
    ents = [np.arange(b * block, min((b + 1) * block, V)) for b in kept if b >= 0]
    sel = np.concatenate(ents) if ents else np.zeros(0, dtype=np.int64)
    pool = np.full(n_blocks * block, -1, dtype=np.int32)
    pool[: len(sel)] = sel
    return pool, kept


def rope_rotate(x, pos, base, sign: float = 1.0) -> np.ndarray:
    """Rotary rotation of the positional channels, float64.

    x float64 [..., d] (d even, the positional channels only); pos an integer
    or an array broadcasting against x's leading dimensions.  Channel pair
    (2i, 2i+1) is turned by sign * pos * base^(-2i/d) radians:
    (a, b) -> (a cos t - b sin t, a sin t + b cos t).
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    theta = float(base) ** (-2.0 * np.arange(d // 2, dtype=np.float64) / d)
    t = sign * np.asarray(pos, dtype=np.float64)[..., None] * theta
    c, s = np.cos(t), np.sin(t)
    a, b = x[..., 0::2], x[..., 1::2]
    out = np.empty(np.broadcast_shapes(x.shape, c.shape[:-1] + (d,)))
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = a * s + b * c
    return out


def _rotated_bf16(rows, pos, base, d_rope: int) -> np.ndarray:
    """rows float64 [n][D]: the last d_rope channels rotated by pos and
    rounded to bf16 (through their float32 value); the others unchanged."""
    out = np.array(rows, dtype=np.float64, copy=True)
    rot = rope_rotate(out[:, -d_rope:], pos, base)
    out[:, -d_rope:] = bf16_to_f64(f32_to_bf16(rot.astype(np.float32)))
    return out


def attention(q_u16, keys: np.ndarray, scale, rope=None) -> tuple[np.ndarray, np.ndarray]:
    """Softmax attention of H query heads over n keys, the value equal to the key.

    q_u16 bf16 bits [H][D]; keys float64 [n][D]; scale is the float32
    softmax scale.  ``rope`` (optional) = dict(base, p, pos [n], d_rope):
    the fused rotary epilogue (query rotated by p, key j by pos[j], output
    rotated back by -p).  Returns (o float64 [H][D], lse float64 [H]); with
    no key at all o = 0 and lse = -inf.
    """
    q = bf16_to_f64(q_u16)
    H, D = q.shape
    if keys.shape[0] == 0:
        return np.zeros((H, D)), np.full(H, -np.inf)
    if rope is not None:
        dr = int(rope.get("d_rope", 64))
        q = _rotated_bf16(q, int(rope["p"]), rope["base"], dr)
        keys = _rotated_bf16(keys, np.asarray(rope["pos"], dtype=np.int64), rope["base"], dr)
    s = float(np.float32(scale))
    logits = s * (q @ keys.T)
    mx = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - mx)
    den = e.sum(axis=1, keepdims=True)
    o = (e / den) @ keys
    lse = (mx + np.log(den))[:, 0]
    if rope is not None:
        o[:, -dr:] = rope_rotate(o[:, -dr:], int(rope["p"]), rope["base"], sign=-1.0)
    return o, lse


def _window_rows(swa, swa_pos0: int, p: int, n_win: int) -> np.ndarray:
    """Raw rows of the sliding window of a query at p that the buffer holds;
    ``swa`` holds bf16 bit patterns (uint16) or decoded float64 rows."""
    swa = np.asarray(swa)
    if n_win <= 0 or p < 0:
        return np.zeros((0, swa.shape[-1]))
    lo = max(0, p - n_win + 1, int(swa_pos0))
    hi = min(p, int(swa_pos0) + swa.shape[0] - 1)
    if hi < lo:
        return np.zeros((0, swa.shape[-1]))
    rows = swa[lo - swa_pos0: hi - swa_pos0 + 1]
    return rows.astype(np.float64) if rows.dtype == np.float64 else bf16_to_f64(rows)


def swa_encode(x_u16, d_nope: int = 512) -> dict:
    """bf16 window rows [S][D] -> FP8 window planes ([V4.1] "FP4 主 KV キャッシュ":
    the sliding-window KV stays FP8): ``codes`` uint8 [S][d_nope] (MXFP8 of the
    content channels), ``scales`` uint8 [S][d_nope/32], ``rope`` uint16
    [S][D - d_nope] (the positional channels' bf16 bits, unchanged)."""
    x = np.asarray(x_u16)
    codes, scales = mxfp8_encode(bf16_to_f64(x[:, :d_nope]))
    return dict(codes=codes, scales=scales, rope=x[:, d_nope:].copy())


def swa_decode(codes, scales, rope) -> np.ndarray:
    """FP8 window planes -> float64 rows [S][D]."""
    return np.concatenate([mxfp8_decode(codes, scales), bf16_to_f64(rope)], axis=-1)


def sparse_attention(q_u16, nope, nscale, rope, idx, swa_u16, swa_pos0, p, n_win, scale,
                     m: int, n_entries: int, rope_base=None):
    """Attention over the selected compressed entries plus the sliding window.

    ``idx`` lists entry indices; -1 and entries not visible at p are
    skipped; a repeated index is attended once per occurrence.  With
    ``rope_base`` the fused rotary epilogue applies (entry j at position
    (j+1)*m - 1, window rows at their own positions).  Returns
    (o [H][D], lse [H]).
    """
    V = visible_count(p, m, n_entries)
    idx = np.asarray(idx, dtype=np.int64)
    sel = idx[(idx >= 0) & (idx < V)]
    ent = decode_entries(np.asarray(nope)[sel], np.asarray(nscale)[sel], np.asarray(rope)[sel])
    win = _window_rows(swa_u16, swa_pos0, p, n_win)
    rp = None
    if rope_base is not None:
        lo = max(0, p - n_win + 1, int(swa_pos0)) if (n_win > 0 and p >= 0) else 0
        pos = np.concatenate([(sel + 1) * m - 1, lo + np.arange(win.shape[0], dtype=np.int64)])
        rp = dict(base=rope_base, p=p, pos=pos, d_rope=np.asarray(rope).shape[-1])
    return attention(q_u16, np.concatenate([ent, win], axis=0), scale, rope=rp)


def dense_attention(q_u16, nope, nscale, rope, swa_u16, swa_pos0, p, n_win, scale, m, n_entries,
                    rope_base=None):
    """HCA [V4], Fig. 4: every visible compressed entry plus the same window."""
    V = visible_count(p, m, n_entries)
    return sparse_attention(q_u16, nope, nscale, rope, np.arange(V), swa_u16, swa_pos0, p,
                            n_win, scale, m, n_entries, rope_base=rope_base)


def csa2_pair(cache: dict, layer_a: dict, layer_b: dict, p: int, m: int, n_entries: int,
              n_win: int, scale, k_a: int, k_b: int):
    """Two CSA2 layers for one query, [V4.1] Fig. 4: a Full layer then a Reindex layer.

    Layer A scores every visible entry with its own indexer query and keeps
    k_a; layer B reuses A's main and indexer-key caches, rescores only A's
    selection with its own indexer query and weights, keeps k_b, and attends
    with its own query and its own window rows over A's main cache.
    ``layer_*`` hold ``qI``, ``w``, ``q``, ``swa`` and ``swa_pos0``.
    """
    idx_a, sc_a, _, _ = index_topk(cache["ikey"], cache["iscale"], layer_a["qI"], layer_a["w"],
                                   p, m, n_entries, k_a)
    o_a, lse_a = sparse_attention(layer_a["q"], cache["nope"], cache["nscale"], cache["rope"], idx_a,
                                  layer_a["swa"], layer_a["swa_pos0"], p, n_win, scale, m, n_entries)
    idx_b, sc_b, _, _ = index_topk(cache["ikey"], cache["iscale"], layer_b["qI"], layer_b["w"],
                                   p, m, n_entries, k_b, cand=idx_a)
    o_b, lse_b = sparse_attention(layer_b["q"], cache["nope"], cache["nscale"], cache["rope"], idx_b,
                                  layer_b["swa"], layer_b["swa_pos0"], p, n_win, scale, m, n_entries)
    return dict(idx_a=idx_a, score_a=sc_a, o_a=o_a, lse_a=lse_a,
                idx_b=idx_b, score_b=sc_b, o_b=o_b, lse_b=lse_b)


def hier_pair(cache: dict, layer_a: dict, layer_b: dict, p: int, m: int, n_entries: int,
              n_win: int, scale, k_a: int, k_b: int, block: int, n_blocks: int):
    """A Full layer that also builds the hierarchical candidate pool, then a
    Reindex layer over that pool ([V4.1], "Hierarchical Sparse Indexer"
    bullet and Fig. 5).

    Layer A scores every visible entry, keeps its own top-k_a over all of
    them and attends to it, and builds the pool of ``block_pool`` from the
    same scores; layer B rescores only the pool with its own indexer query
    and weights, keeps k_b and attends over A's main cache with its own
    query and window.  ``layer_*`` as in ``csa2_pair``.
    """
    idx_a, sc_a, js, s = index_topk(cache["ikey"], cache["iscale"], layer_a["qI"], layer_a["w"],
                                    p, m, n_entries, k_a)
    pool, kept = block_pool(s, len(js), block, n_blocks)
    o_a, lse_a = sparse_attention(layer_a["q"], cache["nope"], cache["nscale"], cache["rope"], idx_a,
                                  layer_a["swa"], layer_a["swa_pos0"], p, n_win, scale, m, n_entries)
    idx_b, sc_b, _, _ = index_topk(cache["ikey"], cache["iscale"], layer_b["qI"], layer_b["w"],
                                   p, m, n_entries, k_b, cand=pool)
    o_b, lse_b = sparse_attention(layer_b["q"], cache["nope"], cache["nscale"], cache["rope"], idx_b,
                                  layer_b["swa"], layer_b["swa_pos0"], p, n_win, scale, m, n_entries)
    return dict(idx_a=idx_a, score_a=sc_a, pool=pool, kept=kept, o_a=o_a, lse_a=lse_a,
                idx_b=idx_b, score_b=sc_b, o_b=o_b, lse_b=lse_b)


# Candidate sources of a Reindex layer (see ``csa2_stack``).
CAND_AUTO, CAND_SCAN, CAND_SELECTION, CAND_POOL = 0, 1, 2, 3
FULL, REINDEX, REUSE = 0, 1, 2


def csa2_stack(layers: list, p: int, m: int, n_win: int) -> list:
    """A stack of CSA2 layers for one query, each statically Full, Reindex or
    Reuse ([V4.1], CSA2 paragraph and Fig. 4; hierarchical pool: the
    "Hierarchical Sparse Indexer" bullet and Fig. 5).

    * Full: scores every visible entry of its own cache (``cache`` holds the
      planes and ``n_entries``) with its own indexer query, keeps its top-k,
      optionally builds the block pool (``pool_block`` / ``pool_blocks``),
      and attends to its selection.
    * Reindex: reuses the cache of the most recent Full layer, scores
      candidates with its own indexer query and keeps its own top-k.  The
      candidates (``cand``): CAND_SCAN every visible entry; CAND_SELECTION
      the selection of the most recent index-producing layer (Full or
      Reindex); CAND_POOL the pool of the most recent Full layer; CAND_AUTO
      the pool when that Full layer built one, else the selection.
    * Reuse: reuses the most recent Full layer's cache and the selection of
      the most recent index-producing layer; no indexer work.

    Every layer attends with its own query ``q`` and window (``swa``,
    ``swa_pos0``) and ``scale``.  Returns one dict per layer with ``idx``
    (the selection it attended to), ``pool`` (Full layers with a pool) and
    ``o`` / ``lse``.
    """
    out = []
    full = None        # most recent Full layer's cache
    pool = None        # ... and its pool (None when it built none)
    sel = None         # most recent index-producing layer's selection
    for L in layers:
        mode = L["mode"]
        r = {}
        if mode == FULL:
            full = L["cache"]
            idx, _, js, s = index_topk(full["ikey"], full["iscale"], L["qI"], L["w"], p, m, full["n_entries"],
                                       L["k"])
            pool = None
            if L.get("pool_blocks", 0) > 0:
                pool, _ = block_pool(s, len(js), L["pool_block"], L["pool_blocks"])
                r["pool"] = pool
            sel = idx
        elif mode == REINDEX:
            if full is None:
                raise ValueError("a Reindex layer needs an earlier Full layer")
            src = L.get("cand", CAND_AUTO)
            if src == CAND_AUTO:
                src = CAND_POOL if pool is not None else CAND_SELECTION
            if src == CAND_POOL and pool is None:
                raise ValueError("no pool to rescore")
            cand = None if src == CAND_SCAN else (pool if src == CAND_POOL else sel)
            idx, _, _, _ = index_topk(full["ikey"], full["iscale"], L["qI"], L["w"], p, m, full["n_entries"],
                                      L["k"], cand=cand)
            sel = idx
        elif mode == REUSE:
            if full is None or sel is None:
                raise ValueError("a Reuse layer needs an earlier index-producing layer")
            idx = sel
        else:
            raise ValueError(f"unknown mode {mode}")
        r["idx"] = idx
        r["o"], r["lse"] = sparse_attention(L["q"], full["nope"], full["nscale"], full["rope"], idx, L["swa"],
                                            L["swa_pos0"], p, n_win, L["scale"], m, full["n_entries"])
        out.append(r)
    return out
