"""Counter-based synthetic tensors (CPU or GPU, bit-identical on both).

Every element is addressed by (seed, tensor id, sequence b, flat element
index i within that sequence).  The 32-bit hash is Chris Wellons'
"lowbias32" integer mixer (published in his "Prospecting for Hash
Functions" article), evaluated on int64 carriers with explicit 32-bit
masking so that no intermediate overflows on either device.  The top 16
bits of the hash pick an entry of a fixed 65,536-entry table of standard
normal quantiles, Phi^-1((i + 1/2) / 65536), computed once in float64 by the
Python standard library and cast to the target storage type by torch's own
round-to-nearest-even conversions.  Values are therefore a 65,536-level
discretisation of N(0, sigma^2), reaching about +-4.32 sigma.

Because generation is a hash plus a table gather, the GPU can produce the
multi-GB raw streams of the long-context workloads in place while the CPU
regenerates any slice for sampled checks.
"""

from __future__ import annotations

import enum
import functools
import statistics

import numpy as np
import torch

_M32 = 0xFFFFFFFF


class TensorId(enum.IntEnum):
    X = 1          # raw per-token KV rows, bf16 [B][T][576]
    Z = 2          # gate logits, bf16 [B][T][G]
    BIAS = 3       # positional bias, fp32 [m]
    W_IK = 4       # indexer-key projection, bf16 [576][d_idx]
    QI = 5         # indexer queries, E4M3 [B][Q][H_I][d_idx]
    W = 6          # indexer head weights, fp32 [B][Q][H_I]
    Q = 7          # attention queries, bf16 [B][Q][H][576]
    QI_B = 8       # second layer's indexer queries
    W_B = 9        # second layer's head weights
    Q_B = 10       # second layer's attention queries
    SWA_B = 11     # second layer's sliding-window rows
    IDX = 12       # random selections for attention-only tests
    NENT = 13      # random entry counts
    POS = 14       # random query positions
    SWA = 15       # sliding-window rows when they are not the raw stream
    NOPE = 16      # synthetic cache planes for stage-wise checks
    NSCALE = 17
    ROPE = 18
    IKEY = 19
    ISCALE = 20
    HID = 21       # hidden states feeding the projections, bf16 [B][T][d_model]
    W_KV = 22      # raw-row projection, bf16 [d_model][576]
    W_Z = 23       # gate-logit projection, bf16 [d_model][G]


def config_seed(cfg: int) -> int:
    """Seed of workload number ``cfg`` (1-based)."""
    return 0xC5A0 + int(cfg)


def _mul32(x, c: int):
    lo = c & 0xFFFF
    hi = c >> 16
    return (x * lo + (((x * hi) & 0xFFFF) << 16)) & _M32


def _lowbias32(x):
    x = x ^ (x >> 16)
    x = _mul32(x, 0x7FEB352D)
    x = x ^ (x >> 15)
    x = _mul32(x, 0x846CA68B)
    x = x ^ (x >> 16)
    return x


def _stream_key(seed: int, tid: int, b: int) -> int:
    k = _lowbias32((int(seed) * 0x9E3779B9 + int(tid) * 0x85EBCA6B) & _M32)
    return _lowbias32(k ^ (int(b) & _M32))


def hash32(seed: int, tid: int, b: int, start: int, count: int, device="cpu") -> torch.Tensor:
    """Hashes (int64 in [0, 2^32)) of elements [start, start+count) of sequence b."""
    if start < 0 or start + count > (1 << 32):
        raise ValueError("element counter out of the 32-bit range")
    k = _stream_key(seed, tid, b)
    i = torch.arange(start, start + count, dtype=torch.int64, device=device)
    h = _lowbias32(i ^ k)
    return _lowbias32((h + k) & _M32)


@functools.lru_cache(maxsize=None)
def _normal_quantiles() -> np.ndarray:
    nd = statistics.NormalDist()
    return np.array([nd.inv_cdf((i + 0.5) / 65536.0) for i in range(65536)], dtype=np.float64)


_TABLES: dict = {}


def _table(kind: str, scale: float, device) -> torch.Tensor:
    key = (kind, float(scale), str(device))
    t = _TABLES.get(key)
    if t is None:
        q = torch.from_numpy(_normal_quantiles() * float(scale))
        if kind == "bf16":
            t = q.to(torch.bfloat16)
        elif kind == "f32":
            t = q.to(torch.float32)
        elif kind == "e4m3":
            t = q.to(torch.float32).to(torch.float8_e4m3fn).view(torch.uint8)
        else:
            raise ValueError(kind)
        t = t.to(device)
        _TABLES[key] = t
    return t


def _fill(kind, seed, tid, shape, scale, device, first_seq, first_elem):
    shape = tuple(int(s) for s in shape)
    B, inner = shape[0], int(np.prod(shape[1:], dtype=np.int64)) if len(shape) > 1 else 1
    table = _table(kind, scale, device)
    out = torch.empty((B, inner), dtype=table.dtype, device=device)
    # Bound the int64 temporaries to a few hundred MB per pass.
    step = 1 << 24
    for b in range(B):
        for s in range(0, inner, step):
            n = min(step, inner - s)
            h = hash32(seed, tid, first_seq + b, first_elem + s, n, device)
            out[b, s:s + n] = table[h >> 16]
    return out.view(shape)


def normal_bf16(seed, tid, shape, scale=1.0, device="cpu", first_seq=0, first_elem=0):
    """bf16 tensor of ``shape`` = (B, ...); sequence b uses counters from ``first_elem``."""
    return _fill("bf16", seed, tid, shape, scale, device, first_seq, first_elem)


def normal_f32(seed, tid, shape, scale=1.0, device="cpu", first_seq=0, first_elem=0):
    return _fill("f32", seed, tid, shape, scale, device, first_seq, first_elem)


def normal_e4m3(seed, tid, shape, scale=1.0, device="cpu", first_seq=0, first_elem=0):
    """uint8 tensor of OCP E4M3 codes (torch's float8_e4m3fn cast of the quantiles)."""
    return _fill("e4m3", seed, tid, shape, scale, device, first_seq, first_elem)


def uniform_bytes(seed, tid, shape, device="cpu"):
    """uint8 tensor of ``shape`` = (B, ...) with independent uniform bytes."""
    shape = tuple(int(s) for s in shape)
    B = shape[0]
    inner = int(np.prod(shape[1:], dtype=np.int64)) if len(shape) > 1 else 1
    out = torch.empty((B, inner), dtype=torch.uint8, device=device)
    step = 1 << 24
    for b in range(B):
        for s in range(0, inner, step):
            n = min(step, inner - s)
            out[b, s:s + n] = (hash32(seed, tid, b, s, n, device) & 0xFF).to(torch.uint8)
    return out.view(shape)


def uniform_int(seed, tid, shape, low, high, device="cpu"):
    """int64 tensor of ``shape`` = (B, ...) with values in [low, high)."""
    shape = tuple(int(s) for s in shape)
    B = shape[0]
    inner = int(np.prod(shape[1:], dtype=np.int64)) if len(shape) > 1 else 1
    span = int(high) - int(low)
    if span <= 0:
        raise ValueError("empty range")
    out = torch.empty((B, inner), dtype=torch.int64, device=device)
    for b in range(B):
        out[b] = hash32(seed, tid, b, 0, inner, device) % span + int(low)
    return out.view(shape)
