"""The compressor fed from hidden states against the oracle's compress_hidden
([V4.1] "アーキテクチャ", CED paragraph, eq. 1: x = H W^KV, z = H W^Z, then
the pooling of [V4] "ハイブリッド注意：CSAとHCA").

Bounds come from the arithmetic: each projected value is an fp32 sum of
d_model exact bf16 products, off by at most d_model * 2^-24 of the sum of
the absolute products for any summation order (4x that here, the instruction
summing inside itself); through the softmax pooling an error e in x moves
the pooled value by at most e, an error e in a gate logit moves each weight
by at most 2 e of itself (so the pooled value by 2 e * sum_i w_i |x_i|), and
the pooling's own fp32 rounding adds (16 + 4m) 2^-22 * sum_i w_i |x_i|.  The
pooled fp32 rows (in the workspace when an indexer key follows) are checked
against that bound directly; the codes may differ only where the oracle's
pre-image lies within it of a rounding boundary (gpu_check.compare_mxfp4).
"""

import zlib

import numpy as np
import pytest
import torch

import compressed_sparse_attention_compressor_amd as csa
import oracle as O
from gpu_check import compare_bf16_rounding, compare_mxfp4

pytestmark = pytest.mark.gpu
DEV = "cuda"
D = 576

CASES = [
    # (name, B, d_model, m, G, T, tok_begin, d_idx (0: no indexer key), N_cap)
    ("m4-g576-ik", 2, 128, 4, 576, 256, 0, 64, 128),
    ("m4-deep-k-offset", 1, 1024, 4, 576, 192, 64, 128, 128),
    ("m12-g1-ragged", 1, 96, 12, 1, 12 * 23, 0, 64, 40),
    ("m128-g1-hca", 2, 256, 128, 1, 512, 0, 0, 8),
    ("m96-long-offset", 1, 64, 96, 576, 288, 96, 0, 8),
    ("m1", 1, 32, 1, 576, 70, 0, 64, 80),
    ("m64-ik", 1, 160, 64, 576, 192, 0, 128, 4),
]


def _bf16(a):
    return O.f32_to_bf16(np.asarray(a, np.float32))


def _t(u16):
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(torch.bfloat16)


def _np(t):
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def _pool_bound(h, wkv, wz, bias, m):
    """Per-entry, per-channel bound of |GPU pooled - oracle pooled|."""
    hf = np.abs(O.bf16_to_f64(h))
    d_model = hf.shape[1]
    gam = 4.0 * d_model * 2.0 ** -24
    ex = gam * (hf @ np.abs(O.bf16_to_f64(wkv)))                 # [T][D]
    ez = gam * (hf @ np.abs(O.bf16_to_f64(wz)))                  # [T][G]
    x = O.bf16_to_f64(h) @ O.bf16_to_f64(wkv)
    z = O.bf16_to_f64(h) @ O.bf16_to_f64(wz)
    T = x.shape[0]
    N = T // m
    a = np.broadcast_to(z.reshape(N, m, -1) + bias.astype(np.float64)[None, :, None], (N, m, D))
    e = np.exp(a - a.max(axis=1, keepdims=True))
    w = e / e.sum(axis=1, keepdims=True)
    pabs = (w * np.abs(x.reshape(N, m, D))).sum(axis=1)
    bx = (w * ex.reshape(N, m, D)).sum(axis=1)
    bz = np.broadcast_to(ez.reshape(N, m, -1), (N, m, D)).max(axis=1)
    return bx + 2.0 * bz * pabs + (16 + 4 * m) * 2.0 ** -22 * pabs


@pytest.mark.parametrize("name,B,d_model,m,G,T,tok_begin,d_idx,N_cap", CASES, ids=[c[0] for c in CASES])
def test_compress_hidden_parity(name, B, d_model, m, G, T, tok_begin, d_idx, N_cap):
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    h = _bf16(rng.standard_normal((B, T, d_model)))
    wkv = _bf16(rng.standard_normal((d_model, D)) / np.sqrt(d_model))
    wz = _bf16(rng.standard_normal((d_model, G)) / np.sqrt(d_model))
    bias = rng.standard_normal(m).astype(np.float32)
    wik = _bf16(rng.standard_normal((D, d_idx)) / 24) if d_idx else None
    cache = csa.Cache(B, N_cap, m, d_idx, device=DEV)
    ws = csa.compress_hidden(cache, _t(h).to(DEV), _t(wkv).to(DEV), _t(wz).to(DEV), torch.from_numpy(bias).to(DEV),
                             _t(wik).to(DEV) if wik is not None else None, tok_begin=tok_begin)
    torch.cuda.synchronize()
    j0, n = tok_begin // m, T // m
    g_nope, g_nsc, g_rope = _np(cache.nope), _np(cache.nscale), _np(cache.rope)
    for b in range(B):
        o = O.compress_hidden(h[b], wkv, wz, bias, wik, m)
        bnd = _pool_bound(h[b], wkv, wz, bias, m)
        if ws is not None and wik is not None:
            gp = _np(ws.view(torch.float32))[:B * n * D].reshape(B, n, D)[b].astype(np.float64)
            ratio = (np.abs(gp - o["pooled"]) / (bnd + 1e-300)).max()
            print(f"{name} b={b}: pooled error / bound = {ratio:.3e}")
            assert ratio <= 1.0, f"{name} b={b}: pooled values off by {ratio:.3e} x the bound"
        sl = slice(j0, j0 + n)
        compare_mxfp4(g_nope[b, sl], g_nsc[b, sl], o["nope"], o["nscale"], o["pooled"][:, :512], bnd[:, :512],
                      what=f"{name} nope b={b}")
        compare_bf16_rounding(g_rope[b, sl], o["pooled"][:, 512:], bnd[:, 512:], what=f"{name} rope b={b}")
        # nothing outside the written entries
        assert not g_nope[b, :j0].any() and not g_nope[b, j0 + n:].any()
        if wik is not None:
            W = np.abs(O.bf16_to_f64(wik))
            kb = 2.0 ** -14 * o["kI_abs"] + bnd @ W
            compare_mxfp4(_np(cache.ikey)[b, sl], _np(cache.iscale)[b, sl], o["ikey"], o["iscale"], o["kI"], kb,
                          what=f"{name} ikey b={b}")


def test_compress_hidden_identity_matches_stream_compressor():
    """d_model = 576, W^KV = W^Z = I: the projections are the rows
    themselves (exact: one nonzero product per sum), and the pooling and
    the indexer-key projection run the stream compressor's arithmetic
    operation for operation: every plane equals csa_compress's on (h, h)."""
    rng = np.random.default_rng(7)
    B, T, m = 1, 128, 4
    h = _bf16(rng.standard_normal((B, T, D)))
    eye = _bf16(np.eye(D))
    bias = rng.standard_normal(m).astype(np.float32)
    wik = _bf16(rng.standard_normal((D, 64)) / 24)
    a = csa.Cache(B, T // m, m, 64, device=DEV)
    r = csa.Cache(B, T // m, m, 64, device=DEV)
    hd, bd, wd = _t(h).to(DEV), torch.from_numpy(bias).to(DEV), _t(wik).to(DEV)
    csa.compress_hidden(a, hd, _t(eye).to(DEV), _t(eye).to(DEV), bd, wd)
    csa.compress(r, hd, hd, bd, wd)
    torch.cuda.synchronize()
    for k in ("nope", "nscale", "rope", "ikey", "iscale"):
        np.testing.assert_array_equal(_np(getattr(a, k)), _np(getattr(r, k)), err_msg=k)
