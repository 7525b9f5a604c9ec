"""Storage formats of the cache, decoded exactly to float64.

[V4.1] section "FP4 主 KV キャッシュ" states that the main KV cache is stored
in the OCP MXFP4 format.  The sentence is garbled: it names E2M1 elements
but an "E4M3 scale per 16 channels", which is not MXFP4.  The reading taken
is the OCP Microscaling one: blocks of 32 contiguous channels share one
E8M0 scale byte, and each element is an E2M1 code.  The positional (RoPE)
channels stay bf16, as both [V4] (section "ハイブリッド注意：CSAとHCA",
storage paragraph) and [V4.1] state.  Indexer queries are OCP E4M3.

The sliding-window rows, which [V4.1] keeps in FP8 because they are
sensitive to quantisation, take the same OCP MX form with E4M3 elements
(MXFP8) for their 512 content channels and bf16 for the positional ones;
the pages give no FP8 scale format, and MX keeps the window in the family
of the main cache.

Encoding rule for a block (OCP MX, scale computed from the block maximum):
  X = floor(log2(max |v|)) - 2, clamped to [-127, 127], scale byte X + 127;
  each v / 2^X is rounded to the nearest E2M1 value, ties to the code with an
  even mantissa bit, and saturated at +-6.  A block whose maximum is 0 gets
  scale byte 0 (X = -127).  The code keeps the sign of a negative value even
  when its magnitude rounds to 0 (code 0x8).  Element 2i sits in the low
  nibble of byte i, element 2i+1 in the high nibble.
"""

from __future__ import annotations

import numpy as np

# E2M1 magnitudes of codes 0..7 (1 sign, 2 exponent bits with bias 1, 1 mantissa bit).
E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)

# Rounding boundaries between consecutive E2M1 magnitudes, and, for each
# boundary, whether an exact tie goes up (the upper neighbour has the even
# mantissa bit) or stays down.
_E2M1_BOUNDS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float64)
_E2M1_TIE_UP = np.array([False, True, False, True, False, True, False])


def bf16_to_f64(u16) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly."""
    u = np.asarray(u16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def f32_to_bf16(x) -> np.ndarray:
    """float32 values -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    bias = np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    return ((u + bias) >> np.uint64(16)).astype(np.uint16)


def e4m3_to_f64(u8) -> np.ndarray:
    """OCP E4M3 ("FN") codes -> float64: bias 7, subnormals, S.1111.111 is NaN."""
    u = np.asarray(u8).astype(np.int64)
    sign = np.where(u & 0x80, -1.0, 1.0)
    e = (u >> 3) & 0xF
    mant = (u & 0x7).astype(np.float64)
    mag = np.where(e == 0, mant / 8.0 * 2.0 ** -6, (1.0 + mant / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    mag = np.where((e == 15) & ((u & 0x7) == 7), np.nan, mag)
    return sign * mag


def e2m1_to_f64(nibble) -> np.ndarray:
    """E2M1 codes (0..15) -> float64; bit 3 is the sign."""
    n = np.asarray(nibble).astype(np.int64)
    mag = E2M1_VALUES[n & 7]
    return np.where(n & 8, -mag, mag)


def e8m0_to_f64(u8) -> np.ndarray:
    """E8M0 scale bytes -> 2^(e - 127); byte 255 is NaN."""
    e = np.asarray(u8).astype(np.int64)
    return np.where(e == 255, np.nan, np.exp2(e.astype(np.float64) - 127.0))


def _e2m1_round(mag: np.ndarray) -> np.ndarray:
    """Magnitude (>= 0, already divided by the block scale) -> E2M1 code 0..7."""
    code = np.zeros(mag.shape, dtype=np.int64)
    for bnd, up in zip(_E2M1_BOUNDS, _E2M1_TIE_UP):
        code += (mag > bnd) | ((mag == bnd) & up)
    return code


def mxfp4_encode(v) -> tuple[np.ndarray, np.ndarray]:
    """Values [..., 32*nb] -> (packed codes uint8 [..., 16*nb], scale bytes uint8 [..., nb]).

    The decision is taken on the values exactly as given (callers pass the
    float32 value that the quantiser sees); the arithmetic below is exact in
    float64 for any float32 input.
    """
    v = np.asarray(v, dtype=np.float64)
    if v.shape[-1] % 32:
        raise ValueError("MXFP4 blocks are 32 channels")
    nb = v.shape[-1] // 32
    blk = v.reshape(v.shape[:-1] + (nb, 32))
    amax = np.max(np.abs(blk), axis=-1)
    _, ex = np.frexp(amax)                     # amax = f * 2^ex, f in [0.5, 1)
    x = np.where(amax > 0, ex.astype(np.int64) - 1 - 2, -127)
    x = np.clip(x, -127, 127)
    scaled = blk / np.exp2(x.astype(np.float64))[..., None]
    code = _e2m1_round(np.abs(scaled)) | np.where(scaled < 0, 8, 0)
    code = code.astype(np.uint8)
    packed = (code[..., 0::2] | (code[..., 1::2] << 4)).astype(np.uint8)
    packed = packed.reshape(v.shape[:-1] + (16 * nb,))
    return packed, (x + 127).astype(np.uint8)


# Non-negative finite E4M3 magnitudes of codes 0..126 (code 127 is NaN).
E4M3_VALUES = None  # filled below


def _e4m3_table() -> np.ndarray:
    return e4m3_to_f64(np.arange(127, dtype=np.uint8))


E4M3_VALUES = _e4m3_table()


def _e4m3_round(mag: np.ndarray) -> np.ndarray:
    """Magnitude (>= 0, already divided by the block scale) -> E4M3 code
    0..126: nearest value, ties to the even code (the even mantissa bit),
    saturating at 448 (code 126)."""
    mag = np.asarray(mag, dtype=np.float64)
    hi = np.clip(np.searchsorted(E4M3_VALUES, mag, side="left"), 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    dlo = np.abs(mag - E4M3_VALUES[lo])
    dhi = np.abs(E4M3_VALUES[hi] - mag)
    code = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    return np.where(mag >= E4M3_VALUES[126], 126, code).astype(np.int64)


def mxfp8_encode(v) -> tuple[np.ndarray, np.ndarray]:
    """Values [..., 32*nb] -> (E4M3 codes uint8 [..., 32*nb], scale bytes uint8 [..., nb]).

    OCP MX with E4M3 elements (the largest E4M3 exponent is 8): per block of
    32 channels X = floor(log2(max |v|)) - 8, clamped to [-127, 127], scale
    byte X + 127 (0 for an all-zero block); each v / 2^X is rounded to the
    nearest E4M3 value, ties to even, saturated at 448; the sign bit is set
    for negative values (also when the magnitude rounds to 0).
    """
    v = np.asarray(v, dtype=np.float64)
    if v.shape[-1] % 32:
        raise ValueError("MXFP8 blocks are 32 channels")
    nb = v.shape[-1] // 32
    blk = v.reshape(v.shape[:-1] + (nb, 32))
    amax = np.max(np.abs(blk), axis=-1)
    _, ex = np.frexp(amax)
    x = np.where(amax > 0, ex.astype(np.int64) - 1 - 8, -127)
    x = np.clip(x, -127, 127)
    scaled = blk / np.exp2(x.astype(np.float64))[..., None]
    code = _e4m3_round(np.abs(scaled)) | np.where(scaled < 0, 0x80, 0)
    return code.astype(np.uint8).reshape(v.shape), (x + 127).astype(np.uint8)


def mxfp8_decode(codes, scales) -> np.ndarray:
    """(E4M3 codes [..., 32*nb], scale bytes [..., nb]) -> float64 [..., 32*nb]."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    nb = scales.shape[-1]
    vals = e4m3_to_f64(codes).reshape(codes.shape[:-1] + (nb, 32))
    return (vals * e8m0_to_f64(scales)[..., None]).reshape(codes.shape)


def mxfp4_decode(packed, scales) -> np.ndarray:
    """(packed codes [..., 16*nb], scale bytes [..., nb]) -> float64 [..., 32*nb]."""
    packed = np.asarray(packed, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    nb = scales.shape[-1]
    lo = e2m1_to_f64(packed & 0xF)
    hi = e2m1_to_f64(packed >> 4)
    vals = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.float64)
    vals[..., 0::2] = lo
    vals[..., 1::2] = hi
    vals = vals.reshape(packed.shape[:-1] + (nb, 32)) * e8m0_to_f64(scales)[..., None]
    return vals.reshape(packed.shape[:-1] + (32 * nb,))
