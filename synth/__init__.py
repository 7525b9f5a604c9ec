"""Seeded synthetic inputs, shared by the oracle side and the HIP side.

This package holds no arithmetic of the attention method (no pooling, no
quantisation of the cache, no scoring, no softmax).  It only turns
(seed, tensor id, sequence, element index) counters into values through a
fixed 32-bit integer hash and fixed quantile tables, so that the CPU and
the GPU produce bit-identical tensors and any slice can be regenerated on
its own.
"""

from .gen import (  # noqa: F401
    TensorId,
    hash32,
    normal_bf16,
    normal_f32,
    normal_e4m3,
    uniform_int,
    uniform_bytes,
    config_seed,
)
