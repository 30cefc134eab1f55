"""GPU parity at the long-context shape: batch 16, every sequence at
position 32767 (32768 keys), full-layer caches of 32768 rows (rotary dim
64, theta 5e6) and one sliding layer (ring of 511 + the new token, rotary
dim 256, theta 1e4) at the same positions, per-head sinks drawn near lse.

The full layer runs through hda_decode_step (the streaming kernel's step
form, which rotates q and the new K in registers at pair entry, plus the
merge that scores and appends the new token) and through hda_rope_append +
hda_decode_attn; the sliding layer through hda_decode_step.  Every
sequence is compared with the oracle: out max-abs <= 1e-2 and mean-abs
<= 1e-3, lse within 1e-4, the appended V row bit-exact and the rotated K
row within one bf16 ulp, every other cache row untouched.
"""
import numpy as np
import pytest

from hybrid_case import (FULL, SLIDING, HybridCase, assert_attn_close, assert_rotated_close, bits_of,
                         fused_step, near_lse_sinks, to_f64)

pytestmark = pytest.mark.gpu

B, POS, LMAX = 16, 32767, 32768


def _case(lt):
    return HybridCase(3200 + lt, B, lt, [POS] * B, lmax=LMAX)


def _check_cache(d, h, lt):
    """The appended row (full: row pos; sliding: slot pos mod 511 and the
    evicted-entry row) within one ulp for K, V bit-exact everywhere."""
    assert np.array_equal(bits_of(d["v"]), h["v"])
    k = bits_of(d["k"])
    rows = [POS] if lt == FULL else [POS % 511, 511]
    other = np.ones(k.shape[2], bool)
    other[rows] = False
    assert np.array_equal(k[:, :, other], h["k"][:, :, other])
    assert_rotated_close(k[:, :, rows], h["k"][:, :, rows], max_frac=1e-2)


@pytest.fixture(scope="module")
def full_case():
    case = _case(FULL)
    _, _, lse0 = case.oracle_step()
    sinks = near_lse_sinks(lse0, 3201)
    h, ref, rlse = case.oracle_step(sinks=sinks)
    return case, sinks, h, ref, rlse


def test_long_full_layer_step(full_case):
    print("CASE long full step b=16 pos=32767", flush=True)
    case, sinks, h, ref, rlse = full_case
    d, out, lse = fused_step(case, sinks=sinks)
    assert_attn_close(out, ref)
    np.testing.assert_allclose(to_f64(lse), rlse, rtol=0, atol=1e-4)
    _check_cache(d, h, FULL)


def test_long_full_layer_two_calls(full_case):
    print("CASE long full two calls b=16 pos=32767", flush=True)
    case, sinks, h, ref, rlse = full_case
    d, out, lse = case.gpu_step(sinks=sinks, max_seq_len=LMAX)
    assert_attn_close(out, ref)
    np.testing.assert_allclose(to_f64(lse), rlse, rtol=0, atol=1e-4)
    _check_cache(d, h, FULL)
    assert_rotated_close(bits_of(d["q"]), h["q"])


def test_long_sliding_layer_step():
    print("CASE long sliding step b=16 pos=32767", flush=True)
    case = _case(SLIDING)
    _, _, lse0 = case.oracle_step()
    sinks = near_lse_sinks(lse0, 3202)
    h, ref, rlse = case.oracle_step(sinks=sinks)
    d, out, lse = fused_step(case, sinks=sinks)
    assert_attn_close(out, ref)
    np.testing.assert_allclose(to_f64(lse), rlse, rtol=0, atol=1e-4)
    _check_cache(d, h, SLIDING)
