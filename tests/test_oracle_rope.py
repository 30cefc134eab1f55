"""Pins for the oracle's RoPE (CPU only).

The Spark export page (`_rope`, `_angles`) defines neox-style partial
rotary embedding: the leading ``rot`` dims are split into halves
x1 = x[:rot/2], x2 = x[rot/2:rot] and rotated pairwise (x1[j], x2[j]) by the
angle pos * theta^(-2j/rot); the remaining dims pass through.  The pins
below check the oracle against things fixed independently of its code:
  * the complex-number form of the same rotation (RoFormer's definition),
    evaluated in fp64 numpy with fp64 angles;
  * exact identities (pos 0, pass-through, pos 1 closed forms);
  * invariants (pair norms, relative-position property).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

SHAPES = [(256, 1e4), (64, 5e6)]  # (rot, theta) of sliding and full layers
D = 256


def _x(seed, n=6):
    g = workloads.generator(seed)
    return workloads.bits(workloads.randn_bf16(g, (n, D)))


def _bf16_ulp(y):
    a = np.abs(y)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 7)


@pytest.mark.parametrize("rot,theta", SHAPES)
def test_pos0_identity(rot, theta):
    x = _x(0)
    assert np.array_equal(oracle.rope_apply(x, rot, theta, 0), x)


@pytest.mark.parametrize("rot,theta", SHAPES)
@pytest.mark.parametrize("pos", [1, 1023, 4095, 32767])
def test_pass_through_bit_exact(rot, theta, pos):
    x = _x(1)
    y = oracle.rope_apply(x, rot, theta, pos)
    assert np.array_equal(y[:, rot:], x[:, rot:])


@pytest.mark.parametrize("rot,theta", SHAPES)
@pytest.mark.parametrize("pos", [1, 7, 511, 1023, 4095, 32767])
def test_complex_rotation_form(rot, theta, pos):
    """y[j] + i*y[j+h] == (x[j] + i*x[j+h]) * exp(i * pos * theta^(-2j/rot))."""
    x = _x(2)
    y = oracle.bf16_to_f64(oracle.rope_apply(x, rot, theta, pos))
    xf = oracle.bf16_to_f64(x)
    h = rot // 2
    j = np.arange(h, dtype=np.float64)
    ang = pos * theta ** (-2.0 * j / rot)
    z = (xf[:, :h] + 1j * xf[:, h:rot]) * np.exp(1j * ang)
    ref = np.concatenate([z.real, z.imag], axis=1)
    # the page builds the angle in fp32: rounding the frequency (half an
    # ulp, relative 2^-24) and the product (half an ulp of the angle) moves
    # it slightly, on top of one bf16 rounding of the result
    ang_err = (0.5 * np.spacing(ang.astype(np.float32)).astype(np.float64)
               + ang * 2.0 ** -24) * 1.01
    ang_err = np.concatenate([ang_err, ang_err])[None]
    pair = np.abs(np.concatenate([z, z], axis=1))
    tol = 0.5 * _bf16_ulp(ref) + ang_err * pair + 1e-30
    assert np.all(np.abs(y[:, :rot] - ref) <= tol + 0.5 * _bf16_ulp(ref))


@pytest.mark.parametrize("rot,theta", SHAPES)
def test_pos1_closed_form(rot, theta):
    """Unit vector on dim j rotates by theta^(-2j/rot): j = 0 turns by exactly 1 rad."""
    h = rot // 2
    for j in [0, 1, h - 1]:
        xf = np.zeros(D)
        xf[j] = 1.0
        x = np.array([oracle.f64_to_bf16_scalar(v) for v in xf], dtype=np.uint16)[None]
        y = oracle.bf16_to_f64(oracle.rope_apply(x, rot, theta, 1))[0]
        a = theta ** (-2.0 * j / rot)
        assert y[j] == oracle.bf16_to_f64(np.array([oracle.f64_to_bf16_scalar(np.cos(a))]))[0]
        assert y[j + h] == oracle.bf16_to_f64(np.array([oracle.f64_to_bf16_scalar(np.sin(a))]))[0]
        others = np.delete(y, [j, j + h])
        assert np.all(others == 0.0)


@pytest.mark.parametrize("rot,theta", SHAPES)
def test_pair_norms_preserved(rot, theta):
    x = _x(3)
    y = oracle.bf16_to_f64(oracle.rope_apply(x, rot, theta, 777))
    xf = oracle.bf16_to_f64(x)
    h = rot // 2
    nx = np.hypot(xf[:, :h], xf[:, h:rot])
    ny = np.hypot(y[:, :h], y[:, h:rot])
    assert np.all(np.abs(nx - ny) <= 2.0 ** -8 * nx + 1e-30)


@pytest.mark.parametrize("rot,theta", SHAPES)
def test_relative_position(rot, theta):
    """rope(q, m) . rope(k, n) depends only on m - n (up to bf16 rounding)."""
    q, k = _x(4, 1), _x(5, 1)
    def dot(m, n):
        a = oracle.bf16_to_f64(oracle.rope_apply(q, rot, theta, m))[0]
        b = oracle.bf16_to_f64(oracle.rope_apply(k, rot, theta, n))[0]
        return float(a @ b)
    base = dot(40, 10)
    for shift in [1, 100, 1000]:
        assert abs(dot(40 + shift, 10 + shift) - base) < 0.15
    # and it does change with the offset
    assert abs(dot(41, 10) - base) > 0.15 or abs(dot(50, 10) - base) > 0.15


def test_angles_follow_fp32_recipe():
    """cos/sin come from the fp32 angle pos * fp32(theta^(-2i/rot))."""
    c, s = oracle.rope_angles(1e4, 256, 32767)
    i = np.arange(128)
    inv32 = (1.0 / 1e4 ** (2.0 * i / 256)).astype(np.float32)
    ang32 = np.float32(32767) * inv32
    assert ang32.dtype == np.float32
    assert np.array_equal(c, np.cos(ang32.astype(np.float64)).astype(np.float32))
    assert np.array_equal(s, np.sin(ang32.astype(np.float64)).astype(np.float32))
