"""Pins for the oracle's per-head output gate (CPU only).

Spark export page, `_Layer.forward`: each query head's attention output is
multiplied by the logistic sigmoid of that head's g_proj value.  Pinned
against values the definition fixes, not by restating it:
  * gate 0 -> factor 1/2, exact in binary: out halves bit for bit;
  * gate +inf -> factor 1: out unchanged bit for bit; -inf -> out 0;
  * gate ln 3 -> 3/4 (1/4 would mean the exponent's sign is flipped);
  * sigmoid(g) + sigmoid(-g) = 1;
  * one factor per (sequence, head), never mixed across them (B != Hq);
  * the gate leaves lse alone and commutes with the sink;
  * the split-K merge applies the same gate.
"""
import math

import numpy as np
import pytest

import oracle
import workloads

S, FU = workloads.SLIDING, workloads.FULL
W = 512


def _case(seed, B=3, lt=FU, lmax=80):
    shape = workloads.HybridShape(batch=B, lmax=lmax)
    g = workloads.generator(seed)
    t = {k: workloads.bits(v).copy() for k, v in workloads.layer_inputs(g, shape, lt).items()}
    if lt == FU:
        t["kev"] = t["vev"] = None
    else:
        for a in ("k", "v"):
            blk = t[a]
            t[a] = np.ascontiguousarray(blk[:, :, :W - 1])
            t[a + "ev"] = np.ascontiguousarray(blk[:, :, W - 1])
    seq = np.array([lmax, 1 + lmax // 2, 17][:B], dtype=np.int32)
    return shape, t, seq


def _attn(t, seq, lt, sinks=None, gate=None):
    return oracle.decode_attn(t["q"], t["k"], t["v"], t["kev"], t["vev"], seq, lt, W, sinks, 1 / 16,
                              gate=gate)


@pytest.mark.parametrize("lt", [S, FU])
def test_gate_special_values(lt):
    shape, t, seq = _case(1, lt=lt)
    base, lse0 = _attn(t, seq, lt)
    B, Hq = base.shape[:2]
    half, lse = _attn(t, seq, lt, gate=np.zeros((B, Hq), np.float32))
    assert np.array_equal(half, base * 0.5)
    assert np.array_equal(lse, lse0)
    one, _ = _attn(t, seq, lt, gate=np.full((B, Hq), np.inf, np.float32))
    assert np.array_equal(one, base)
    zero, _ = _attn(t, seq, lt, gate=np.full((B, Hq), -np.inf, np.float32))
    assert not zero.any()


def test_gate_sign_and_symmetry():
    shape, t, seq = _case(2)
    base, _ = _attn(t, seq, FU)
    B, Hq = base.shape[:2]
    g3 = np.float32(math.log(3.0))
    out, _ = _attn(t, seq, FU, gate=np.full((B, Hq), g3, np.float32))
    # the fp32 logit is ln 3 to 2^-24 relative; the factor moves by < 1e-7
    np.testing.assert_allclose(out, base * 0.75, rtol=1e-7, atol=0)
    g = np.linspace(-7.5, 7.5, B * Hq, dtype=np.float32).reshape(B, Hq)
    pos, _ = _attn(t, seq, FU, gate=g)
    neg, _ = _attn(t, seq, FU, gate=-g)
    np.testing.assert_allclose(pos + neg, base, rtol=1e-13, atol=1e-15)


def test_gate_per_sequence_and_head():
    shape, t, seq = _case(3)
    base, _ = _attn(t, seq, FU)
    B, Hq = base.shape[:2]
    assert B != Hq
    # each (b, h) gets its own power of two: a factor applied to the wrong
    # (b, h) shows as a different exact ratio
    g = np.zeros((B, Hq), np.float32)
    expect = np.zeros((B, Hq))
    for b in range(B):
        for h in range(Hq):
            f = 2.0 ** -(1 + b * Hq + h)  # exact sigmoid value: g = ln(f / (1 - f))
            g[b, h] = np.float32(math.log(f / (1 - f)))
            expect[b, h] = 1 / (1 + math.exp(-float(g[b, h])))
    out, _ = _attn(t, seq, FU, gate=g)
    ratio = out[:, :, 0] / base[:, :, 0]
    np.testing.assert_allclose(ratio, expect, rtol=1e-12)
    assert np.allclose(expect, [[2.0 ** -(1 + b * Hq + h) for h in range(Hq)] for b in range(B)],
                       rtol=1e-6)


def test_gate_commutes_with_sink():
    shape, t, seq = _case(4)
    base, lse = _attn(t, seq, FU)
    B, Hq = base.shape[:2]
    sinks = (np.arange(Hq, dtype=np.float32) - 1.5) + np.float32(lse.mean())
    g = np.linspace(-2, 2, B * Hq, dtype=np.float32).reshape(B, Hq)
    both, lse_b = _attn(t, seq, FU, sinks=sinks, gate=g)
    sink_only, _ = _attn(t, seq, FU, sinks=sinks)
    gated = sink_only.copy()
    oracle.output_gate(gated, g)
    np.testing.assert_allclose(both, gated, rtol=1e-15, atol=0)
    np.testing.assert_array_equal(lse_b, lse)


def test_gate_in_lse_merge():
    rng = np.random.default_rng(5)
    o = rng.standard_normal((3, 8))
    ls = rng.standard_normal(3)
    base, lse = oracle.lse_merge(o, ls, sink=0.25)
    out, lse_g = oracle.lse_merge(o, ls, sink=0.25, gate=0.0)
    assert np.array_equal(out, base * 0.5) and lse_g == lse
