"""The C ABI on a machine without a GPU: symbols and host-side argument checks.

Only calls that fail their host-side checks are made here; such calls
return before any HIP call, so no GPU is needed.
"""

import ctypes
import os
import re

import pytest

from compressed_sparse_attention_compressor_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa.h")

OK, ENULL, ESHAPE, EALIGN, EUNSUP, EWS = 0, -1, -2, -3, -4, -5
P = 0x10000          # a fake, 16-byte aligned device address (never dereferenced)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libcsa.so is not built (run __graft_entry__.build())")
    return _lib.lib()


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*((?:csa2?|hca)_\w+)\s*\(", src, flags=re.M)))


def test_every_declared_symbol_is_exported(L):
    names = _declared()
    assert {"csa_compress", "csa_compress_hidden", "csa_index_topk", "csa_sparse_attn", "hca_dense_attn"} <= set(names)
    for n in names:
        assert hasattr(L, n), n
    assert set(_lib._SIGS) == set(names)


def test_status_strings_and_version(L):
    assert L.csa_version() >= 10000
    for s in (OK, ENULL, ESHAPE, EALIGN, EUNSUP, EWS, -6):
        assert L.csa_status_str(s)


def _cache(B=2, N=64, m=4, d_idx=128, **kw):
    c = _lib.CacheT(P, P, P, P if d_idx else None, P if d_idx else None, P, B, N, 512, 64, d_idx, m)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def _compress(L, c, x=P, z=P, G=576, bias=P, w=P, tb=0, T=64, xs=64 * 576, zs=64 * 576):
    return L.csa_compress(x, xs, z, zs, G, bias, w, tb, T, ctypes.byref(c) if c is not None else None, None)


def test_compress_checks(L):
    assert _compress(L, None) == ENULL
    assert _compress(L, _cache(), x=None) == ENULL
    assert _compress(L, _cache(d_idx=0)) == ENULL            # w_ik given, no key planes
    assert _compress(L, _cache(d_nope=256)) == EUNSUP
    assert _compress(L, _cache(m=0)) == EUNSUP
    assert _compress(L, _cache(m=300)) == EUNSUP
    assert _compress(L, _cache(d_idx=96)) == EUNSUP
    assert _compress(L, _cache(), G=7) == EUNSUP
    assert _compress(L, _cache(), tb=2) == ESHAPE             # not a multiple of m
    assert _compress(L, _cache(), T=6) == ESHAPE
    assert _compress(L, _cache(N=8), T=64) == ESHAPE          # beyond N_cap
    assert _compress(L, _cache(), xs=10) == ESHAPE            # rows overlap across sequences
    assert _compress(L, _cache(), x=P + 2) == EALIGN
    assert _compress(L, _cache(nope=P + 8)) == EALIGN
    assert _compress(L, _cache(), T=0) == OK                  # nothing to do, no launch


def _index(L, c, qi=P, w=P, HI=32, qp=P, Q=1, cand=None, C=0, k=8, out=P, ws=P, wsb=1 << 30):
    return L.csa_index_topk(ctypes.byref(c), qi, w, HI, qp, Q, cand, C, k, out, None, ws, wsb, None)


def test_index_topk_checks(L):
    assert _index(L, _cache(ikey=None)) == ENULL
    assert _index(L, _cache(), qi=None) == ENULL
    assert _index(L, _cache(), out=None) == ENULL
    assert _index(L, _cache(), HI=0) == EUNSUP
    assert _index(L, _cache(), HI=65) == EUNSUP
    assert _index(L, _cache(), k=-1) == ESHAPE
    assert _index(L, _cache(), qi=P + 4) == EALIGN
    need = L.csa_workspace_bytes(0, 2, 1, 0, 64, 0)
    assert need == 2 * 64 * 4
    assert _index(L, _cache(), wsb=need - 1) == EWS
    assert _index(L, _cache(), ws=None) == ENULL
    assert _index(L, _cache(), Q=0) == OK
    assert _index(L, _cache(), k=0) == OK


def _attn(L, c, q=P, H=64, qp=P, Q=1, idx=P, k=16, swa=P, s0=P, S=128, nw=128, scale=1.0, od=1, out=P,
          ws=P, wsb=1 << 30, rope=0.0):
    return L.csa_sparse_attn(ctypes.byref(c), q, H, qp, Q, idx, k, swa, s0, S, nw, scale, rope, od, out, None, ws, wsb,
                             None)


def test_attention_checks(L):
    assert _attn(L, _cache(), q=None) == ENULL
    assert _attn(L, _cache(), idx=None) == ENULL
    assert _attn(L, _cache(), swa=None) == ENULL
    assert _attn(L, _cache(), H=48) == EUNSUP
    assert _attn(L, _cache(), H=256) == EUNSUP
    assert _attn(L, _cache(), od=5) == EUNSUP
    assert _attn(L, _cache(), scale=float("nan")) == ESHAPE
    assert _attn(L, _cache(), rope=-1.0) == ESHAPE
    assert _attn(L, _cache(), rope=float("nan")) == ESHAPE
    assert _attn(L, _cache(), rope=float("inf")) == ESHAPE
    assert _attn(L, _cache(), rope=10000.0, Q=0) == OK
    assert _attn(L, _cache(), k=-2) == ESHAPE
    assert _attn(L, _cache(), nw=-1) == ESHAPE
    assert _attn(L, _cache(), out=P + 2) == EALIGN
    need = L.csa_workspace_bytes(1, 2, 1, 64, 16, 128)
    assert need > 0
    assert _attn(L, _cache(), wsb=need - 1) == EWS
    assert _attn(L, _cache(), Q=0) == OK
    assert L.hca_dense_attn(ctypes.byref(_cache(d_idx=0)), None, 64, P, 1, P, P, 128, 128, 1.0, 0.0, 1, P, None, P,
                            1 << 30, None) == ENULL


def test_workspace_sizes_consistent(L):
    # one split (no partials) once there are enough query rows
    assert L.csa_workspace_bytes(1, 1, 65536, 64, 1024, 128) == 0
    # several splits for a single long row, with (O, max, sum) per head
    w = L.csa_workspace_bytes(2, 8, 1, 64, 8192, 128)
    assert w > 0 and w % (8 * 64 * (576 + 2) * 4) == 0


def _pool(L, c, sc=P, qp=P, Q=1, block=8, nb=16, out=P, ws=P, wsb=1 << 30):
    return L.csa_index_pool(ctypes.byref(c), sc, qp, Q, block, nb, out, ws, wsb, None)


def test_index_pool_checks(L):
    assert _pool(L, _cache(), sc=None) == ENULL
    assert _pool(L, _cache(), qp=None) == ENULL
    assert _pool(L, _cache(), out=None) == ENULL
    assert _pool(L, _cache(), ws=None) == ENULL
    assert _pool(L, _cache(), Q=-1) == ESHAPE
    assert _pool(L, _cache(), block=0) == EUNSUP
    assert _pool(L, _cache(), block=65) == EUNSUP
    assert _pool(L, _cache(), nb=0) == EUNSUP
    assert _pool(L, _cache(), block=64, nb=(1 << 14) + 1) == EUNSUP     # pool beyond 2^20 slots
    assert _pool(L, _cache(), ws=P + 8) == EALIGN
    need = L.csa_workspace_bytes(4, 2, 1, 16, 64, 8)
    # block scores (2 rows x 8 blocks), positions, counts, kept blocks: 256-byte aligned pieces
    assert need >= 4 * 256
    assert _pool(L, _cache(), wsb=need - 1) == EWS
    assert _pool(L, _cache(), Q=0) == OK
    assert L.csa_workspace_bytes(4, 2, 1, 16, 64, 0) == 0        # unsupported block


def _layer(mode, cache=None, k=8, cand=0, pool_block=0, pool_blocks=0, q=P, idx=P, pool=P, H=64, od=1):
    e = _lib.Csa2LayerT()
    e.mode, e.cand, e.k, e.pool_block, e.pool_blocks = mode, cand, k, pool_block, pool_blocks
    if cache is not None:
        e.cache = ctypes.pointer(cache)
    e.q_idx, e.w_idx, e.H_I, e.idx_out, e.pool_out = P, P, 32, idx, pool
    e.q, e.H, e.n_win, e.swa, e.swa_pos0, e.S = q, H, 128, P, P, 128
    e.softmax_scale, e.out_dtype, e.out, e.lse = 1.0, od, P, None
    return e


def _arr(layers):
    return (_lib.Csa2LayerT * len(layers))(*layers)


def _stack(L, layers, qp=P, Q=1, ws=P, wsb=1 << 30):
    """Only for stacks that fail a check (a valid one would launch kernels)."""
    return L.csa2_layer_stack(_arr(layers), len(layers), qp, Q, ws, wsb, None)


def test_layer_stack_checks(L):
    c = _cache()
    full, reuse = _layer(0, c), _layer(2)
    assert _stack(L, [full, reuse], Q=0) == OK                 # valid, nothing to launch
    assert _stack(L, [reuse]) == ESHAPE                        # first layer must be Full
    assert _stack(L, [_layer(1)]) == ESHAPE                    # Reindex without a Full layer
    assert _stack(L, [full, _layer(1, cand=3)]) == ESHAPE      # no pool to rescore
    assert _stack(L, [full, _layer(1, cand=9)]) == EUNSUP
    assert _stack(L, [_layer(7, c)]) == EUNSUP
    assert _stack(L, [_layer(0, c, k=0)]) == ESHAPE
    assert _stack(L, [_layer(0)]) == ENULL                     # Full layer without a cache
    assert _stack(L, [full, _layer(2, q=None)]) == ENULL       # a later layer's check fails first
    assert _stack(L, [full, _layer(2, H=48)]) == EUNSUP
    assert _stack(L, [_layer(0, c, pool_block=65, pool_blocks=4)]) == EUNSUP
    assert _stack(L, [_layer(0, c, pool_block=8, pool_blocks=4, pool=None)]) == ENULL
    assert _stack(L, [full, _layer(0, _cache(B=3))]) == ESHAPE  # every cache holds the same sequences
    assert _stack(L, [full, reuse], qp=None) == ENULL
    good = [_layer(0, c, pool_block=8, pool_blocks=4), _layer(1, cand=0), reuse]
    need = L.csa2_stack_workspace_bytes(_arr(good), 3, 1)
    # scores of 2 x 64 entries, then the largest of the pool, top-k and attention workspaces
    assert need >= 2 * 64 * 4
    assert L.csa2_stack_workspace_bytes(_arr([reuse]), 1, 1) == 0      # invalid stack
    assert _stack(L, good, wsb=need - 1) == EWS
    assert _stack(L, good, ws=P + 8) == EALIGN
    assert _stack(L, good, ws=None) == ENULL
    many = [_layer(0, c)] + [_layer(2) for _ in range(256)]          # 257 layers
    assert _stack(L, many) == EUNSUP
    assert L.csa2_stack_workspace_bytes(_arr(many), len(many), 1) == 0


def test_index_pool_grid_limit(L):
    # 2^24 query rows x 128 blocks of 256: beyond a 32-bit flattened grid
    assert _pool(L, _cache(B=1, N=32768), Q=1 << 24, block=1, nb=1) == EUNSUP


def test_fp8_window_checks(L):
    # csa_swa_encode(x, x_stride_b, B, S, codes, scales, rope, stream)
    enc = L.csa_swa_encode
    assert enc(None, 100 * 576, 2, 100, P, P, P, None) == ENULL
    assert enc(P, 100 * 576, 2, 100, P, None, P, None) == ENULL
    assert enc(P, 100 * 576, -1, 100, P, P, P, None) == ESHAPE
    assert enc(P, 50 * 576, 2, 100, P, P, P, None) == ESHAPE          # rows of two sequences overlap
    assert enc(P + 2, 100 * 576, 2, 100, P, P, P, None) == EALIGN
    assert enc(P, 100 * 576 + 4, 2, 100, P, P, P, None) == EALIGN
    assert enc(P, 0, 0, 100, None, None, None, None) == OK            # nothing to do
    # csa_sparse_attn_w8 / hca_dense_attn_w8: the window planes are checked first
    def sw8(codes=P, scales=P, rope=P, nw=128):
        return L.csa_sparse_attn_w8(ctypes.byref(_cache()), P, 64, P, 1, P, 16, codes, scales, rope, P, 128, nw, 1.0,
                                    0.0, 1, P, None, P, 1 << 30, None)
    assert sw8(codes=None) == ENULL
    assert sw8(scales=None) == ENULL
    assert sw8(codes=P + 4) == EALIGN
    assert sw8(rope=P + 8) == EALIGN
    assert L.csa_sparse_attn_w8(ctypes.byref(_cache()), P, 48, P, 1, P, 16, P, P, P, P, 128, 128, 1.0, 0.0, 1, P,
                                None, P, 1 << 30, None) == EUNSUP
    assert L.hca_dense_attn_w8(ctypes.byref(_cache(d_idx=0)), P, 64, P, 1, None, P, P, P, 128, 128, 1.0, 0.0, 1, P,
                               None, P, 1 << 30, None) == ENULL
    assert L.csa_sparse_attn_w8(ctypes.byref(_cache()), P, 64, P, 0, P, 16, P, P, P, P, 128, 128, 1.0, 0.0, 1, P,
                                None, P, 1 << 30, None) == OK                # Q = 0: nothing to launch


def test_compress_hidden_checks(L):
    c = ctypes.byref(_cache())
    def ch(h=P, hs=64 * 128, d=128, wkv=P, wz=P, G=576, bias=P, wik=None, tb=0, T=64, ws=None, wsb=0):
        return L.csa_compress_hidden(h, hs, d, wkv, wz, G, bias, wik, tb, T, c, ws, wsb, None)
    assert ch(h=None) == ENULL
    assert ch(wz=None) == ENULL
    assert ch(d=100) == EUNSUP          # not a multiple of 32
    assert ch(d=0) == EUNSUP
    assert ch(G=7) == EUNSUP
    assert ch(T=6) == ESHAPE            # not a multiple of m
    assert ch(h=P + 2) == EALIGN
    assert ch(T=0) == OK                # nothing to do
    assert L.csa_compress_hidden_ws_bytes(2, 64, 4, 1) == 2 * 16 * 576 * 4
    assert L.csa_compress_hidden_ws_bytes(2, 64, 4, 0) == 0


def test_read_device_flags_null(L):
    # a null output pointer fails before any HIP call
    assert L.csa_read_device_flags(None, None) == ENULL


def test_noalloc_rejects_beyond_the_fixed_scratch(L):
    # 64 rows of 65,536 entries need far more than the fixed scratch: the call
    # is refused on the host, before any HIP call
    c = _cache(B=64, N=65536)
    assert L.csa_index_topk_noalloc(ctypes.byref(c), P, P, 32, P, 1, None, 0, 512, P, None, None) == -7
    assert L.csa_status_str(-7)
    assert L.csa_index_topk_noalloc(None, P, P, 32, P, 1, None, 0, 512, P, None, None) == ENULL
