"""Comparison rules between the HIP path and the oracle (test infrastructure).

* FP4 codes and scales: bit-exact, except where the GPU's fp32 pre-image
  may legitimately land on the other side of a rounding decision: the
  oracle's float64 pre-image lies within `bound` (an error bound of the fp32
  evaluation, derived from the magnitudes of the summed terms) of an E2M1
  rounding boundary, of a power of two that changes the block scale, or of
  zero (sign).  Each exemption is counted.
* Top-k: the same number of selected entries, ascending and unique; entries
  in only one of the two selections must have oracle scores within 1e-4
  relative of the oracle's k-th score.
* Attention: row-normalised max error max_c |g - r| / max_c |r| per
  (sequence, query, head) row, 1e-3 for fp32 outputs and 2e-2 for bf16.
"""

from __future__ import annotations

import numpy as np

from oracle import bf16_to_f64, e4m3_to_f64, mxfp4_decode

_BOUNDS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])


def _nibbles(packed):
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out


def compare_mxfp4(g_packed, g_scales, o_packed, o_scales, pre, bound, what=""):
    """Returns the number of exempted (mismatching but explained) elements."""
    g_c = _nibbles(g_packed).reshape(-1, 32)
    o_c = _nibbles(o_packed).reshape(-1, 32)
    gs = np.asarray(g_scales).reshape(-1)
    os_ = np.asarray(o_scales).reshape(-1)
    pre = np.asarray(pre, np.float64).reshape(-1, 32)
    bnd = np.asarray(bound, np.float64).reshape(-1, 32)
    exempt = 0
    amax = np.abs(pre).max(axis=1)
    bmax = bnd.max(axis=1)
    p2 = np.exp2(np.round(np.log2(np.where(amax > 0, amax, 1.0))))
    near_p2 = np.abs(amax - p2) <= bmax + 1e-300
    bad_scale = (gs != os_) & ~near_p2
    assert not bad_scale.any(), f"{what}: {bad_scale.sum()} block scales differ away from a power of two"
    skip = gs != os_
    exempt += int(skip.sum()) * 32
    X = os_.astype(np.float64) - 127.0
    scaled = np.abs(pre) / np.exp2(X)[:, None]
    dist = np.min(np.abs(scaled[..., None] - _BOUNDS), axis=-1) * np.exp2(X)[:, None]
    diff = (g_c != o_c) & ~skip[:, None]
    mag_diff = ((g_c & 7) != (o_c & 7)) & diff
    sign_diff = ((g_c & 8) != (o_c & 8)) & diff
    bad = (mag_diff & (dist > bnd)) | (sign_diff & (np.abs(pre) > bnd))
    assert not bad.any(), (f"{what}: {bad.sum()} codes differ away from a rounding boundary "
                           f"(first at {np.argwhere(bad)[0]})")
    exempt += int(diff.sum())
    return exempt


def compare_bf16_rounding(g_u16, pre, bound, what=""):
    """bf16 of an fp32 value: the GPU choice may be at most `bound` worse than the nearest."""
    g = bf16_to_f64(g_u16)
    pre = np.asarray(pre, np.float64)
    v32 = pre.astype(np.float32)
    u = v32.view(np.uint32).astype(np.uint64)
    o = ((u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)).astype(np.uint16)
    od = bf16_to_f64(o)
    ok = np.abs(g - pre) <= np.abs(od - pre) + np.asarray(bound) + 1e-300
    assert ok.all(), f"{what}: {(~ok).sum()} bf16 values off"
    return int((g != od).sum())


def check_topk(g_idx, o_idx, js, scores, rel=1e-4, what=""):
    """g_idx, o_idx: int [k] rows; js/scores: every scored entry and its oracle score."""
    g = np.asarray(g_idx)
    o = np.asarray(o_idx)
    gv, ov = g[g >= 0], o[o >= 0]
    assert len(gv) == len(ov), f"{what}: {len(gv)} selected vs {len(ov)}"
    assert np.all(g[len(gv):] == -1), f"{what}: -1 padding not at the end"
    assert np.all(np.diff(gv) > 0), f"{what}: selection not strictly ascending"
    d = set(gv.tolist()) ^ set(ov.tolist())
    if not d:
        return 0
    sc = dict(zip(np.asarray(js).tolist(), np.asarray(scores).tolist()))
    sk = min(sc[j] for j in ov.tolist())
    for j in d:
        assert j in sc, f"{what}: entry {j} was not a scored entry"
        assert abs(sc[j] - sk) <= rel * abs(sk) + 1e-30, f"{what}: entry {j} score {sc[j]} vs k-th {sk}"
    return len(d) // 2


def index_score_tol(qI_u8, w_f32, ikey_rows, iscale_rows, ref=None):
    """Per-entry bound on |GPU score - oracle score| for the indexer.

    Four parts:
    * fp32 evaluation of the head sum: any order of summing the H_I weighted
      heads (and of summing fp32 partials) errs by at most (d_idx + H_I) *
      2^-24 relative to the sum of the absolute terms,
      sum_h |w_h| * sum_c |q_hc * k_jc|; 1e-5 covers d_idx + H_I <= 160;
    * the block-scaled matrix instruction's own sum of one head's (up to)
      128 products: measured on gfx950 to hold each such dot product only to
      a fraction of its largest product (at most 3.3e-4 of it over query
      codes spanning 2^-6..448 and key scale bytes 100..154; nearly exact
      when the products span few binades); bounded here by 2^-9 x that
      largest product: 2^-9 * sum_h |w_h| * max_c |q_hc * k_jc|;
    * rounding in the subnormal range (keys with tiny block scales): at most
      2^-149 per operation, (d_idx + H_I) * 2^-149 * sum_h |w_h|;
    * subnormal E4M3 query codes in a block of 32 channels that also holds a
      magnitude above 56: the kernels multiply every other block by 2^3 (and
      give it the scale 2^-3), which makes its subnormal codes normal, but
      such a block keeps scale 1, and the instruction keeps products of
      subnormal E4M3 codes with E2M1 codes only to a multiple of 2^-9 before
      the block scale (measured on gfx950), a loss of up to 2^-10 x its key
      block's scale per product, through ReLU (1-Lipschitz) and the head
      weight: sum_h |w_h| * sum_{c in such blocks} [q_hc subnormal] 2^-10 *
      S_j(c).  Zero for every query whose blocks all stay at or below 56.
    """
    q = np.asarray(qI_u8, dtype=np.uint8)
    H, d = q.shape
    wa = np.abs(np.asarray(w_f32, dtype=np.float32).astype(np.float64))
    k = np.abs(mxfp4_decode(np.asarray(ikey_rows), np.asarray(iscale_rows)))    # [V][d]
    qa = np.abs(e4m3_to_f64(q))                                                 # [H][d]
    mag = (k @ qa.T) @ wa                                                       # [V]
    big = np.empty(k.shape[0])
    for j0 in range(0, k.shape[0], 512):                                        # max_c |q_hc k_jc|, chunked
        big[j0:j0 + 512] = (k[j0:j0 + 512, None, :] * qa[None, :, :]).max(axis=2) @ wa
    nb = d // 32
    sub = ((q & 0x78) == 0) & ((q & 0x07) != 0)                                 # [H][d]
    keeps1 = ((q & 0x7F).reshape(H, nb, 32) > 0x66).any(axis=2)                # [H][nb]
    n_hb = sub.reshape(H, nb, 32).sum(axis=2) * keeps1                          # [H][nb]
    per_blk = (n_hb * wa[:, None]).sum(axis=0)                                  # [nb]
    S = np.exp2(np.asarray(iscale_rows, dtype=np.float64)[:, :nb] - 127.0)     # [V][nb]
    return (1e-5 * mag + 2.0 ** -9 * big + (d + H) * 2.0 ** -149 * wa.sum()
            + 2.0 ** -10 * (S @ per_blk))


def compress_bounds(out, m, W=None):
    """Error bounds of the GPU's fp32 pooling (and key projection) for each
    pooled value: (8 + 2m) * 2^-22 * sum of the absolute weighted terms, and
    for indexer keys 2^-14 * |kI| (bf16 W_IK products in fp32) plus the
    pooled-value bound carried through |W|."""
    pool_b = (8 + 2 * m) * 2.0 ** -22 * out["pooled_abs"]
    kb = None
    if W is not None:
        Wa = np.abs(bf16_to_f64(W))
        kb = 2.0 ** -14 * out["kI_abs"] + (8 + 2 * m) * 2.0 ** -22 * (out["pooled_abs"] @ Wa)
    return pool_b, kb


def row_rel_err(g, r):
    g = np.asarray(g, np.float64)
    r = np.asarray(r, np.float64)
    den = np.abs(r).max(axis=-1)
    num = np.abs(g - r).max(axis=-1)
    return np.where(den > 0, num / np.where(den > 0, den, 1), num)


def decode_cache_rows(nope, nscale, rope):
    return np.concatenate([mxfp4_decode(nope, nscale), bf16_to_f64(rope)], axis=-1)
