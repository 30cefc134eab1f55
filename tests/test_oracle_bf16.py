"""Pins for the oracle's bf16 widening and rounding (CPU only).

The reference point is torch's fp32 -> bf16 cast, which rounds to nearest
even: for inputs that are exact fp32 values the oracle's single rounding
from fp64 must agree with it bit for bit.
"""
import numpy as np
import torch

import oracle


def test_known_values():
    assert oracle.f64_to_bf16_scalar(1.0) == 0x3F80
    assert oracle.f64_to_bf16_scalar(-2.0) == 0xC000
    # ties to even: 1 + 2^-8 sits half way between 1 and 1 + 2^-7
    assert oracle.f64_to_bf16_scalar(1.0 + 2.0 ** -8) == 0x3F80
    assert oracle.f64_to_bf16_scalar(1.0 + 3 * 2.0 ** -8) == 0x3F82
    # just above the tie rounds up
    assert oracle.f64_to_bf16_scalar(1.0 + 2.0 ** -8 + 2.0 ** -30) == 0x3F81
    assert oracle.f64_to_bf16_scalar(float("inf")) == 0x7F80
    assert oracle.f64_to_bf16_scalar(-0.0) == 0x8000
    assert oracle.f64_to_bf16_scalar(3.5e38) == 0x7F80  # overflow


def test_matches_torch_rne_on_fp32_values():
    g = torch.Generator().manual_seed(1)
    x = torch.randn(20000, generator=g) * torch.exp(torch.randn(20000, generator=g) * 20)
    ref = x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.f64_to_bf16_scalar(float(v)) for v in x.double()], dtype=np.uint16)
    assert np.array_equal(ref, got)


def test_subnormals():
    tiny = np.array([2.0 ** -133, 3 * 2.0 ** -134, 2.0 ** -127 + 2.0 ** -133], dtype=np.float32)
    ref = torch.from_numpy(tiny).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.f64_to_bf16_scalar(float(v)) for v in tiny], dtype=np.uint16)
    assert np.array_equal(ref, got)


def test_widening_exact():
    bits = np.arange(0, 65536, 7, dtype=np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]  # finite only
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.array_equal(oracle.bf16_to_f64(bits), ref)
