"""Pins for the oracle's multi-token decode (CPU only).

Spark export page, `SparkStepConfig.cache_len` docstring: the ring holds
the window's previous entries and the new token is scored with them.  A
chunk of T new tokens therefore means: token t (position pos + t) attends
to the entries of its own window -- positions [pos + t - 511, pos + t] on a
sliding layer, [0, pos + t] on a full one -- which are the cached ones plus
new tokens 0..t.  The oracle composes T single-token steps; pinned here
against what does not go through the ring at all:
  * torch's fp64 scaled_dot_product_attention (a library routine) over the
    key list taken from the plain position history (the roll view), with
    the new tokens rotated by the oracle's RoPE (itself pinned), the sink
    as an extra zero-value key, for windows that cross the 511/512 slot
    boundaries inside the chunk;
  * causality: changing token T-1's q, k or v leaves tokens < T-1 bit for
    bit unchanged;
  * the cache after the chunk holds each window's entries where a
    single-token step would find them.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads

S, FU = workloads.SLIDING, workloads.FULL
W = 512
D, HQ, HKV = 256, 8, 2


def _f(bits):
    return workloads.from_bits(np.ascontiguousarray(bits)).double()


def _setup(seed, lt, pos, T, cap=None):
    """History of already-rotated K/V for positions < pos[b], the oracle's
    cache built from it, and T new tokens."""
    B = len(pos)
    g = workloads.generator(seed)
    hist_len = max(pos) + 1
    hk = workloads.bits(workloads.randn_bf16(g, (B, HKV, hist_len, D)))
    hv = workloads.bits(workloads.randn_bf16(g, (B, HKV, hist_len, D)))
    q = workloads.bits(workloads.randn_bf16(g, (B, T, HQ, D)))
    kn = workloads.bits(workloads.randn_bf16(g, (B, T, HKV, D)))
    vn = workloads.bits(workloads.randn_bf16(g, (B, T, HKV, D)))
    if lt == FU:
        cap = cap or max(pos) + T
        k = np.zeros((B, HKV, cap, D), np.uint16)
        v = k.copy()
        for b, p in enumerate(pos):
            k[b, :, :p], v[b, :, :p] = hk[b, :, :p], hv[b, :, :p]
    else:
        k = np.zeros((B, HKV, W - 1, D), np.uint16)
        v = k.copy()
        for b, p in enumerate(pos):
            for qpos in range(max(0, p - (W - 1)), p):
                k[b, :, qpos % (W - 1)], v[b, :, qpos % (W - 1)] = hk[b, :, qpos], hv[b, :, qpos]
    kev = np.zeros((B, HKV, D), np.uint16)
    vev = kev.copy()
    return hk, hv, q, kn, vn, k, v, kev, vev


def _reference(lt, pos, hk, hv, q, kn, vn, sinks, scale, rot, theta):
    B, T = q.shape[:2]
    out = np.zeros((B, T, HQ, D))
    lse = np.zeros((B, T, HQ))
    for b, p in enumerate(pos):
        for t in range(T):
            qr = oracle.rope_apply(q[b, t], rot, theta, p + t)
            new_k = [oracle.rope_apply(kn[b, s], rot, theta, p + s) for s in range(t + 1)]
            lo = 0 if lt == FU else max(0, p + t - (W - 1))
            for h in range(HQ):
                g = h // (HQ // HKV)
                keys = [hk[b, g, x] for x in range(lo, p)] + [nk[g] for nk in new_k]
                vals = [hv[b, g, x] for x in range(lo, p)] + [vn[b, s, g] for s in range(t + 1)]
                K = torch.stack([_f(x) for x in keys])[None, None]
                V = torch.stack([_f(x) for x in vals])[None, None]
                qq = _f(qr[h])[None, None, None]
                lse[b, t, h] = torch.logsumexp(K[0, 0] @ qq[0, 0, 0] * scale, 0).item()
                K = torch.cat([K, torch.zeros(1, 1, 1, D, dtype=torch.float64)], 2)
                V = torch.cat([V, torch.zeros(1, 1, 1, D, dtype=torch.float64)], 2)
                mask = torch.zeros(1, 1, 1, K.shape[2], dtype=torch.float64)
                mask[..., -1] = float(sinks[h])
                out[b, t, h] = F.scaled_dot_product_attention(qq, K, V, attn_mask=mask,
                                                              scale=scale)[0, 0, 0].numpy()
    return out, lse


@pytest.mark.parametrize("lt,pos,T", [
    (S, [0, 509, 2000], 4),     # empty ring; chunk crossing slot 510/511; wrapped ring
    (S, [300, 508], 3),
    (FU, [0, 40, 95], 4),
    (FU, [7, 60], 2),
])
def test_multi_matches_sdpa_over_history(lt, pos, T):
    hk, hv, q, kn, vn, k, v, kev, vev = _setup(10 + T + lt, lt, pos, T)
    shape = workloads.HybridShape(batch=len(pos), lmax=16)
    rot, theta = shape.rot(lt), shape.theta(lt)
    sinks = np.linspace(-1, 2, HQ).astype(np.float32)
    ref, rlse = _reference(lt, pos, hk, hv, q, kn, vn, sinks, 1 / 16, rot, theta)
    out, lse = oracle.decode_multi(q.copy(), kn, vn, np.array(pos), lt, rot, theta, W, k, v, kev,
                                   vev, sinks, 1 / 16)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, rlse, rtol=0, atol=1e-12)


@pytest.mark.parametrize("lt", [S, FU])
def test_multi_causal(lt):
    pos, T = [600, 30], 4
    hk, hv, q, kn, vn, k, v, kev, vev = _setup(20 + lt, lt, pos, T)
    shape = workloads.HybridShape(batch=2, lmax=16)
    args = (np.array(pos), lt, shape.rot(lt), shape.theta(lt), W)
    o1, l1 = oracle.decode_multi(q.copy(), kn, vn, *args, k.copy(), v.copy(), kev.copy(),
                                 vev.copy(), None, 1 / 16)
    q2, kn2, vn2 = q.copy(), kn.copy(), vn.copy()
    q2[:, T - 1] ^= np.uint16(0x8000)
    kn2[:, T - 1] ^= np.uint16(0x4000)
    vn2[:, T - 1] ^= np.uint16(0x4000)
    o2, l2 = oracle.decode_multi(q2, kn2, vn2, *args, k.copy(), v.copy(), kev.copy(), vev.copy(),
                                 None, 1 / 16)
    assert np.array_equal(o1[:, :T - 1], o2[:, :T - 1]) and np.array_equal(l1[:, :T - 1], l2[:, :T - 1])
    assert not np.array_equal(o1[:, T - 1], o2[:, T - 1])


def test_multi_cache_state_sliding():
    """After the chunk, slot (pos + t) mod 511 holds token t (rotated at
    pos + t) and the side row the entry the last token evicted."""
    pos, T = [1000], 3
    hk, hv, q, kn, vn, k, v, kev, vev = _setup(30, S, pos, T)
    shape = workloads.HybridShape(batch=1, lmax=16)
    rot, theta = shape.rot(S), shape.theta(S)
    k0 = k.copy()
    oracle.decode_multi(q.copy(), kn, vn, np.array(pos), S, rot, theta, W, k, v, kev, vev, None,
                        1 / 16)
    for t in range(T):
        slot = (pos[0] + t) % (W - 1)
        assert np.array_equal(k[0, :, slot], oracle.rope_apply(kn[0, t], rot, theta, pos[0] + t))
        assert np.array_equal(v[0, :, slot], vn[0, t])
    last = (pos[0] + T - 1) % (W - 1)
    assert np.array_equal(kev[0], k0[0, :, last])
