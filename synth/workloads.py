"""Shapes and input recipes of the five measured workloads, plus small variants.

Input recipe (every value from synth.gen, so CPU and GPU agree bit for bit):
  x   raw KV rows      bf16 N(0,1)                 [B][T][576]
  z   gate logits      bf16 N(0,1)                 [B][T][576]
  bias positional bias fp32 N(0,1)                 [m]
  W_IK projection      bf16 N(0,1)/sqrt(576)       [576][d_idx]
  qI  indexer queries  E4M3 N(0,1) * q_idx_scale   [B][Q][H_I][d_idx]
  w   head weights     fp32 N(0,1)                 [B][Q][H_I]
  q   queries          bf16 N(0,1) * q_scale       [B][Q][H][576]
The sliding-window rows are the raw rows x themselves.  The batched
128K-context decode pre-scales the queries (q by 1/sqrt(576), qI by
1/sqrt(128)) and uses a softmax scale of 1; the other workloads use unit
queries and a softmax scale of 1/sqrt(576).
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

from .gen import TensorId, config_seed, normal_bf16, normal_e4m3, normal_f32

D = 576


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    cfg: int                # seed selector
    B: int
    T: int                  # raw tokens per sequence in the cache
    m: int
    d_idx: int              # 0 = no indexer (HCA)
    H_I: int
    k: int                  # top-k (layer A's k for the two-layer case)
    H: int
    n_win: int
    Q: int = 1              # query tokens per sequence (decode: the last token)
    k_b: int = 0            # second layer's k (two-layer reindex case)
    prescaled: bool = False
    prefill: bool = False   # queries at every position 0..T-1
    pool_block: int = 0     # hierarchical pool: entries per block (0 = no pool)
    pool_blocks: int = 0    # hierarchical pool: blocks kept per query

    @property
    def N(self) -> int:
        return self.T // self.m

    @property
    def seed(self) -> int:
        return config_seed(self.cfg)

    @property
    def softmax_scale(self) -> float:
        return 1.0 if self.prescaled else float(np.float32(1.0 / math.sqrt(D)))

    @property
    def q_scale(self) -> float:
        return 1.0 / math.sqrt(D) if self.prescaled else 1.0

    @property
    def q_idx_scale(self) -> float:
        return 1.0 / math.sqrt(self.d_idx) if (self.prescaled and self.d_idx) else 1.0

    def positions(self) -> np.ndarray:
        if self.prefill:
            return np.tile(np.arange(self.Q, dtype=np.int32), (self.B, 1))
        return np.full((self.B, self.Q), self.T - 1, dtype=np.int32)


TINY_DECODE = Workload("csa-decode-tiny-4k", 1, B=1, T=4096, m=4, d_idx=64, H_I=4, k=64, H=16, n_win=128)
BATCHED_DECODE = Workload("csa-decode-b32-128k", 2, B=32, T=131072, m=4, d_idx=128, H_I=32, k=512, H=64, n_win=128,
                          prescaled=True)
PREFILL = Workload("csa-prefill-64k", 3, B=1, T=65536, m=4, d_idx=128, H_I=32, k=1024, H=64, n_win=128, Q=65536,
                   prefill=True)
HCA_DECODE = Workload("hca-decode-b8-1m", 4, B=8, T=1048576, m=128, d_idx=0, H_I=0, k=0, H=64, n_win=128)
CSA2_DECODE = Workload("csa2-decode-b4-1m", 5, B=4, T=1048576, m=4, d_idx=128, H_I=32, k=2048, H=64, n_win=128,
                       k_b=512)

# The same 1M two-layer decode with the hierarchical pool: the Full layer
# keeps its own top-512 and a pool of 2,048 blocks x 8 entries; the Reindex
# layer rescores the 16,384 pool entries and keeps 512.
CSA2_HIER_DECODE = Workload("csa2-hier-decode-b4-1m", 6, B=4, T=1048576, m=4, d_idx=128, H_I=32, k=512, H=64,
                            n_win=128, k_b=512, pool_block=8, pool_blocks=2048)

ALL = [TINY_DECODE, BATCHED_DECODE, PREFILL, HCA_DECODE, CSA2_DECODE, CSA2_HIER_DECODE]


def raw_rows(w: Workload, t0: int, t1: int, device="cpu", seq0=0, nseq=None):
    """(x, z) rows t0..t1-1 of sequences seq0..seq0+nseq-1: bf16 [nseq][t1-t0][576] each."""
    nseq = w.B if nseq is None else nseq
    x = normal_bf16(w.seed, TensorId.X, (nseq, t1 - t0, D), device=device, first_seq=seq0, first_elem=t0 * D)
    z = normal_bf16(w.seed, TensorId.Z, (nseq, t1 - t0, D), device=device, first_seq=seq0, first_elem=t0 * D)
    return x, z


def params(w: Workload, device="cpu"):
    """bias fp32 [m] and W_IK bf16 [576][d_idx] (None without an indexer)."""
    bias = normal_f32(w.seed, TensorId.BIAS, (1, w.m), device=device)[0]
    wik = None
    if w.d_idx:
        wik = normal_bf16(w.seed, TensorId.W_IK, (1, D, w.d_idx), scale=1.0 / math.sqrt(D), device=device)[0]
    return bias, wik


def queries(w: Workload, device="cpu", second=False, q0=0, nq=None):
    """Per-layer query-side inputs for query tokens q0..q0+nq-1: dict of tensors."""
    nq = w.Q if nq is None else nq
    tq, tqi, tw = (TensorId.Q_B, TensorId.QI_B, TensorId.W_B) if second else (TensorId.Q, TensorId.QI, TensorId.W)
    out = dict(q=normal_bf16(w.seed, tq, (w.B, nq, w.H, D), scale=w.q_scale, device=device,
                             first_elem=q0 * w.H * D))
    if w.d_idx:
        out["qI"] = normal_e4m3(w.seed, tqi, (w.B, nq, w.H_I, w.d_idx), scale=w.q_idx_scale, device=device,
                                first_elem=q0 * w.H_I * w.d_idx)
        out["w"] = normal_f32(w.seed, tw, (w.B, nq, w.H_I), device=device, first_elem=q0 * w.H_I)
    pos = torch.from_numpy(w.positions()[:, q0:q0 + nq].copy())
    out["q_pos"] = pos.to(device)
    return out


def hidden_inputs(w: Workload, d_model: int, G: int = D, t0: int = 0, t1=None, device="cpu"):
    """Hidden states h bf16 [B][t1-t0][d_model] N(0,1) and the projections
    W^KV bf16 [d_model][576], W^Z bf16 [d_model][G], both N(0, 1/d_model), so
    that x = h W^KV and z = h W^Z follow the N(0,1) stream recipe."""
    t1 = w.T if t1 is None else t1
    h = normal_bf16(w.seed, TensorId.HID, (w.B, t1 - t0, d_model), device=device, first_elem=t0 * d_model)
    wkv = normal_bf16(w.seed, TensorId.W_KV, (1, d_model, D), scale=1.0 / math.sqrt(d_model), device=device)[0]
    wz = normal_bf16(w.seed, TensorId.W_Z, (1, d_model, G), scale=1.0 / math.sqrt(d_model), device=device)[0]
    return h, wkv, wz


def second_layer_window(w: Workload, t0: int, t1: int, device="cpu"):
    """The second layer's own window rows (positions t0..t1-1)."""
    return normal_bf16(w.seed, TensorId.SWA_B, (w.B, t1 - t0, D), device=device, first_elem=t0 * D)


def as_u16(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> numpy uint16 bit patterns (CPU copy)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def synthetic_cache(w: Workload, device="cpu", N_cap=None, seq0=0, nseq=None, scales="narrow", rope_zero=False):
    """Cache planes drawn directly (for checking the stages after the compressor
    at full size): uniform E2M1 code bytes, bf16 N(0,1) rope channels and
    E8M0 scale bytes chosen by ``scales``:

    * "narrow": 124..127 (values up to 6 in magnitude, like encoded N(0,1) data);
    * "wide": per 32-channel block, one of five kinds picked by the block's
      hash: a zero block (scale byte 0 and every code 0, as the encoder
      writes for an all-zero block), scale byte 0 with the drawn codes
      (values down to 2^-128, fp32 and bf16 subnormals), 1..100, 128..140
      (values up to 6 * 2^13), or the common 120..127;
    * "tiny": scale bytes 0..3 with the drawn codes and some zero blocks,
      so that whole entries hold values near the bottom of the fp32 range.

    rope_zero: positional channels all zero (so that the MXFP4 channels alone
    set the size of a row)."""
    N_cap = w.N if N_cap is None else N_cap
    nseq = w.B if nseq is None else nseq
    out = {}

    def planes(tid_codes, tid_scales, width):
        codes = _rows_bytes(w, tid_codes, nseq, N_cap, width, device, seq0)
        h = _rows_hash(w, tid_scales, nseq, N_cap, width // 16, device, seq0)
        if scales == "narrow":
            sc = 124 + h % 4
            return codes, sc.to(torch.uint8)
        kind = (h >> 8) % 8
        if scales == "wide":
            sc = torch.where(kind == 2, 1 + h % 100,
                             torch.where(kind == 3, 128 + h % 13, torch.where(kind <= 1, 0, 120 + h % 8)))
            zero = kind == 0
        elif scales == "tiny":
            sc = h % 4
            zero = kind == 0
        else:
            raise ValueError(scales)
        blk = codes.view(nseq, N_cap, width // 16, 16)
        blk = torch.where(zero[..., None], torch.zeros_like(blk), blk)
        return blk.reshape(nseq, N_cap, width), sc.to(torch.uint8)

    out["nope"], out["nscale"] = planes(TensorId.NOPE, TensorId.NSCALE, 256)
    out["rope"] = normal_bf16(w.seed, TensorId.ROPE, (nseq, N_cap, 64), device=device, first_seq=seq0)
    if rope_zero:
        out["rope"] = torch.zeros_like(out["rope"])
    if w.d_idx:
        out["ikey"], out["iscale"] = planes(TensorId.IKEY, TensorId.ISCALE, w.d_idx // 2)
    return out


def _rows_hash(w, tid, nseq, N_cap, width, device, seq0):
    from .gen import hash32
    out = torch.empty((nseq, N_cap * width), dtype=torch.int64, device=device)
    step = 1 << 24
    for b in range(nseq):
        for s in range(0, N_cap * width, step):
            n = min(step, N_cap * width - s)
            out[b, s:s + n] = hash32(w.seed, tid, seq0 + b, s, n, device)
    return out.view(nseq, N_cap, width)


def _rows_bytes(w, tid, nseq, N_cap, width, device, seq0):
    from .gen import hash32
    out = torch.empty((nseq, N_cap * width), dtype=torch.uint8, device=device)
    step = 1 << 24
    for b in range(nseq):
        for s in range(0, N_cap * width, step):
            n = min(step, N_cap * width - s)
            out[b, s:s + n] = (hash32(w.seed, tid, seq0 + b, s, n, device) & 0xFF).to(torch.uint8)
    return out.view(nseq, N_cap, width)
