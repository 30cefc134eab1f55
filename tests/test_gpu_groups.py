"""GPU parity for every query-group size the kernels are built for (G = Hq /
Hkv in 1, 2, 4, 8, 16), on each decomposition: the window kernel (sliding
layer and short full layer), the balanced stream plus merge (full layer
beyond 1024 keys), fixed chunks, and both forms of the fused step.  Same
tolerances as the other decode tests; sinks near lse so they matter."""
import numpy as np
import pytest
import torch

from hybrid_case import (FULL, SLIDING, HybridCase, assert_attn_close, assert_rotated_close,
                         bits_of, fused_step, to_f64)

pytestmark = pytest.mark.gpu

GROUPS = [(4, 4), (8, 4), (16, 2), (32, 2)]  # G = 1, 2, 8, 16 (G = 4 is covered elsewhere)


def _sinks(case, seed):
    _, _, lse0 = case.oracle_step()
    g = np.random.default_rng(seed)
    return (lse0.mean(0) + g.normal(0, 1.5, case.shape.num_q_heads)).astype(np.float32)


@pytest.mark.parametrize("hq,hkv", GROUPS)
@pytest.mark.parametrize("lt,pos,lmax,chunk", [
    (SLIDING, [0, 300, 1000], None, 0),      # window kernel
    (FULL, [5, 700, 1023], 1024, 0),         # window kernel, ragged
    (FULL, [600, 1500, 2047], 2048, 0),      # balanced stream + merge
    (FULL, [600, 1500, 2047], 2048, 64),     # fixed chunks + LSE merge
])
def test_decode_groups(hq, hkv, lt, pos, lmax, chunk):
    print("CASE", hq, hkv, lt, pos, chunk, flush=True)
    case = HybridCase(2000 + hq + 7 * hkv, len(pos), lt, pos, lmax=lmax, poison=True,
                      num_q_heads=hq, num_kv_heads=hkv)
    sinks = _sinks(case, hq)
    h, ref, rlse = case.oracle_step(sinks=sinks)
    d, out, lse = case.gpu_step(sinks=sinks, chunk_keys=chunk, max_seq_len=lmax or 1024)
    assert np.array_equal(bits_of(d["v"]), h["v"])
    assert_rotated_close(bits_of(d["k"]), h["k"])
    assert_attn_close(out, ref)
    np.testing.assert_allclose(to_f64(lse), rlse, rtol=0, atol=1e-4)


@pytest.mark.parametrize("hq,hkv", GROUPS)
@pytest.mark.parametrize("lt,pos,lmax", [(SLIDING, [100, 511, 1300], None), (FULL, [100, 900, 2047], 2048)])
def test_step_groups(hq, hkv, lt, pos, lmax):
    print("CASE step", hq, hkv, lt, pos, flush=True)
    case = HybridCase(2100 + hq + 7 * hkv, len(pos), lt, pos, lmax=lmax, poison=True,
                      num_q_heads=hq, num_kv_heads=hkv)
    sinks = _sinks(case, hq + 1)
    h, ref, rlse = case.oracle_step(sinks=sinks)
    d, out, lse = fused_step(case, sinks=sinks)
    assert np.array_equal(bits_of(d["v"]), h["v"])
    assert_rotated_close(bits_of(d["k"]), h["k"])
    assert_attn_close(out, ref)
    np.testing.assert_allclose(to_f64(lse), rlse, rtol=0, atol=1e-4)
