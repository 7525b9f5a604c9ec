"""The seeded generators: determinism, slicing and distribution."""

import numpy as np
import torch

from synth import TensorId, hash32, normal_bf16, normal_e4m3, normal_f32, uniform_int


def test_lowbias32_known_values():
    # lowbias32 is a bijection on 32-bit words; 0 maps to 0 and the mixer
    # changes about half of the output bits for a one-bit input change.
    from synth.gen import _lowbias32
    assert _lowbias32(0) == 0
    x = torch.arange(1, 4097, dtype=torch.int64)
    h = _lowbias32(x)
    assert int(h.unique().numel()) == 4096 and int(h.max()) < 2 ** 32
    flips = torch.tensor([bin(int(a) ^ int(b)).count("1") for a, b in zip(_lowbias32(x), _lowbias32(x ^ 1))])
    assert 12 < float(flips.float().mean()) < 20


def test_slices_regenerate():
    full = normal_bf16(7, TensorId.X, (3, 50, 576))
    part = normal_bf16(7, TensorId.X, (1, 10, 576), first_seq=2, first_elem=20 * 576)
    assert torch.equal(full[2, 20:30].view(torch.int16), part[0].view(torch.int16))


def test_distribution_close_to_standard_normal():
    v = normal_f32(3, TensorId.W, (4, 100000)).double()
    assert abs(float(v.mean())) < 0.01 and abs(float(v.std()) - 1.0) < 0.01
    b = normal_bf16(3, TensorId.Q, (1, 100000), scale=1 / 24).double()
    assert abs(float(b.std()) * 24 - 1.0) < 0.02
    e = normal_e4m3(3, TensorId.QI, (1, 50000), scale=1 / 11.3).view(torch.float8_e4m3fn).double()
    assert abs(float(e.std()) * 11.3 - 1.0) < 0.03


def test_streams_are_distinct():
    a = hash32(1, 1, 0, 0, 1000)
    b = hash32(1, 2, 0, 0, 1000)
    c = hash32(1, 1, 1, 0, 1000)
    assert (a == b).sum() < 5 and (a == c).sum() < 5


def test_uniform_int_range():
    u = uniform_int(5, TensorId.IDX, (2, 1000), 3, 17)
    assert int(u.min()) == 3 and int(u.max()) == 16
