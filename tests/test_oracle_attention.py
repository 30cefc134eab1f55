"""Pins for the oracle's decode attention, split-K merge and sink (CPU only).

Independent references:
  * torch's scaled_dot_product_attention and logsumexp in fp64 on CPU over
    the explicitly gathered key set (a library routine, GQA expanded);
  * the sink, [SINK] class docstring out *= exp(lse)/(exp(lse)+exp(sink)),
    is the same as softmax over the keys plus one extra key whose logit is
    the sink and whose value is zero -- checked through SDPA with an
    additive mask;
  * closed forms: one key -> its value exactly; equal keys -> mean of
    values; a -inf sink is a no-op ([SINK] `_sinks_for_query`); sink = lse
    halves the output;
  * invariants: ring order is arbitrary (Spark page ring comment); a split
    softmax merged by LSE equals the single pass, at least as well as the
    page's 140.3 dB (golden/split_softmax_fidelity.json).
"""
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads

HERE = os.path.dirname(os.path.abspath(__file__))
S, FU = workloads.SLIDING, workloads.FULL
W = 512


def _f(bits):
    return torch.from_numpy(oracle.bf16_to_f64(bits))


def _case(seed, B, lt, lmax=96):
    """Oracle-form inputs: a sliding block splits into the 511-slot ring and
    its last row, the side row."""
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
    return shape, t


def _key_set(t, lt, b, g, n):
    """Explicit key/value rows attended by sequence b, kv head g."""
    if lt == FU:
        return t["k"][b, g, :n], t["v"][b, g, :n]
    nr = min(n, W - 1)
    ks, vs = [t["k"][b, g, :nr]], [t["v"][b, g, :nr]]
    if n >= W:
        ks.append(t["kev"][b, g][None])
        vs.append(t["vev"][b, g][None])
    return np.concatenate(ks), np.concatenate(vs)


def _sdpa_ref(t, lt, seq_lens, scale, sinks=None):
    B, Hq, D = t["q"].shape
    Hkv = t["k"].shape[1]
    G = Hq // Hkv
    out = np.zeros((B, Hq, D))
    lse = np.zeros((B, Hq))
    for b in range(B):
        for h in range(Hq):
            kk, vv = _key_set(t, lt, b, h // G, int(seq_lens[b]))
            q = _f(t["q"][b, h])[None, None, None]          # [1,1,1,D]
            K = _f(kk)[None, None]                           # [1,1,n,D]
            V = _f(vv)[None, None]
            if sinks is not None:
                K = torch.cat([K, torch.zeros(1, 1, 1, D, dtype=torch.float64)], 2)
                V = torch.cat([V, torch.zeros(1, 1, 1, D, dtype=torch.float64)], 2)
                mask = torch.zeros(1, 1, 1, K.shape[2], dtype=torch.float64)
                mask[..., -1] = float(sinks[h])
                o = F.scaled_dot_product_attention(q, K, V, attn_mask=mask, scale=scale)
            else:
                o = F.scaled_dot_product_attention(q, K, V, scale=scale)
            out[b, h] = o[0, 0, 0].numpy()
            lse[b, h] = torch.logsumexp(_f(kk) @ _f(t["q"][b, h]) * scale, 0).item()
    return out, lse


@pytest.mark.parametrize("lt", [S, FU])
@pytest.mark.parametrize("seq_lens", [[1, 2], [8, 96], [511, 512], [513, 1024]])
def test_brute_force_sdpa(lt, seq_lens):
    if lt == FU and max(seq_lens) > 96:
        seq_lens = [min(s, 96) for s in seq_lens]
    shape, t = _case(sum(seq_lens) + lt, 2, lt)
    out, lse = oracle.decode_attn(t["q"], t["k"], t["v"], t["kev"], t["vev"], seq_lens, lt, W,
                                  None, 1 / 16)
    ref, rlse = _sdpa_ref(t, lt, seq_lens, 1 / 16)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, rlse, rtol=0, atol=1e-12)


@pytest.mark.parametrize("lt", [S, FU])
def test_sink_is_extra_zero_value_key(lt):
    shape, t = _case(21, 2, lt)
    seq = [300, 90] if lt == S else [50, 96]
    g = workloads.generator(5)
    _, lse0 = oracle.decode_attn(t["q"], t["k"], t["v"], t["kev"], t["vev"], seq, lt, W, None, 1 / 16)
    # sinks near lse actually move the output (N(0,1) sinks barely do)
    sinks = (lse0.mean(0) + 2 * workloads.sinks(g, 8).numpy()).astype(np.float32)
    out, lse = oracle.decode_attn(t["q"], t["k"], t["v"], t["kev"], t["vev"], seq, lt, W, sinks, 1 / 16)
    ref, rlse = _sdpa_ref(t, lt, seq, 1 / 16, sinks)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse0, rtol=0, atol=0)  # lse is pre-sink


def test_sink_special_values():
    shape, t = _case(22, 2, S)
    seq = [512, 200]
    args = (t["q"], t["k"], t["v"], t["kev"], t["vev"], seq, S, W)
    out0, lse0 = oracle.decode_attn(*args, None, 1 / 16)
    o, _ = oracle.decode_attn(*args, np.full(8, -np.inf, np.float32), 1 / 16)
    assert np.array_equal(o, out0)                    # -inf: bitwise no-op
    o, _ = oracle.decode_attn(*args, np.full(8, np.inf, np.float32), 1 / 16)
    assert np.all(o == 0)                             # +inf: everything to the sink
    # sink == lse halves the output; lse per head differs, use one sequence
    o1, l1 = oracle.decode_attn(t["q"][:1], t["k"][:1], t["v"][:1], t["kev"][:1], t["vev"][:1],
                                [512], S, W, None, 1 / 16)
    sk = l1[0].astype(np.float32)
    o2, _ = oracle.decode_attn(t["q"][:1], t["k"][:1], t["v"][:1], t["kev"][:1], t["vev"][:1],
                               [512], S, W, sk, 1 / 16)
    fac = 1.0 / (1.0 + np.exp(sk.astype(np.float64) - l1[0]))
    np.testing.assert_allclose(o2[0], o1[0] * fac[:, None], rtol=1e-15, atol=0)
    assert np.all(np.abs(fac - 0.5) < 1e-6)


def test_one_key_returns_value():
    shape, t = _case(23, 2, S)
    out, lse = oracle.decode_attn(t["q"], t["k"], t["v"], t["kev"], t["vev"], [1, 1], S, W,
                                  None, 1 / 16)
    for b in range(2):
        for h in range(8):
            assert np.array_equal(out[b, h], oracle.bf16_to_f64(t["v"][b, h // 4, 0]))


def test_equal_keys_mean_of_values():
    shape, t = _case(24, 1, FU)
    t["k"][:] = t["k"][:, :, :1]
    out, lse = oracle.decode_attn(t["q"], t["k"], t["v"], None, None, [77], FU, W, None, 1 / 16)
    mean = oracle.bf16_to_f64(t["v"][0, :, :77]).mean(1)
    for h in range(8):
        np.testing.assert_allclose(out[0, h], mean[h // 4], rtol=0, atol=1e-14)
        s = float(oracle.bf16_to_f64(t["q"][0, h]) @ oracle.bf16_to_f64(t["k"][0, h // 4, 0])) / 16
        assert abs(lse[0, h] - (s + np.log(77))) < 1e-12


def test_unwritten_slots_excluded():
    """Poisoned (NaN) rows beyond the valid set never reach the output."""
    shape, t = _case(25, 2, S)
    seq = [300, 40]
    out0, _ = oracle.decode_attn(t["q"], t["k"], t["v"], t["kev"], t["vev"], seq, S, W, None, 1 / 16)
    for b, n in enumerate(seq):
        t["k"][b, :, n:] = 0x7FC0
        t["v"][b, :, n:] = 0x7FC0
    t["kev"][:] = 0x7FC0  # side row is not valid below a full window
    t["vev"][:] = 0x7FC0
    out1, _ = oracle.decode_attn(t["q"], t["k"], t["v"], t["kev"], t["vev"], seq, S, W, None, 1 / 16)
    assert np.array_equal(out0, out1)


def test_ring_order_arbitrary():
    shape, t = _case(26, 1, S)
    args = [t["q"], t["k"], t["v"], t["kev"], t["vev"], [1000], S, W, None, 1 / 16]
    out0, lse0 = oracle.decode_attn(*args)
    perm = np.random.default_rng(0).permutation(511)
    t["k"][:] = t["k"][:, :, perm]
    t["v"][:] = t["v"][:, :, perm]
    out1, lse1 = oracle.decode_attn(t["q"], t["k"], t["v"], t["kev"], t["vev"], [1000], S, W,
                                    None, 1 / 16)
    np.testing.assert_allclose(out1, out0, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse1, lse0, rtol=0, atol=1e-13)


@pytest.mark.parametrize("nchunks", [2, 3, 7, 64])
def test_split_merge_equals_single_pass(nchunks):
    gold = json.load(open(os.path.join(HERE, "golden", "split_softmax_fidelity.json")))
    g = workloads.generator(30 + nchunks)
    n, D = 700, 256
    q = workloads.bits(workloads.randn_bf16(g, (D,)))
    k = workloads.bits(workloads.randn_bf16(g, (n, D)))
    v = workloads.bits(workloads.randn_bf16(g, (n, D)))
    ref, rlse = oracle.attn_chunk(q, k, v, 0, n, 1 / 16)
    edges = np.linspace(0, n, nchunks + 1).astype(int)
    edges[1] = edges[0]  # one empty chunk (lse -inf) must weigh zero
    parts = [oracle.attn_chunk(q, k, v, int(a), int(b), 1 / 16) for a, b in zip(edges[:-1], edges[1:])]
    o = np.stack([p[0] for p in parts])
    l = np.array([p[1] for p in parts])
    assert np.isneginf(l[0])
    out, lse = oracle.lse_merge(o, l)
    snr = 10 * np.log10(np.sum(ref ** 2) / np.sum((out - ref) ** 2 + 1e-300))
    assert snr >= gold["snr_db"]
    assert abs(lse - rlse) < 1e-12
    # chunk order does not matter
    perm = np.random.default_rng(nchunks).permutation(nchunks)
    out2, lse2 = oracle.lse_merge(o[perm], l[perm])
    np.testing.assert_allclose(out2, out, rtol=0, atol=1e-14)
    # the merge's sink matches the one-pass sink
    sk = np.float32(rlse + 0.3)
    o3, _ = oracle.lse_merge(o, l, sk)
    fac = np.exp(rlse) / (np.exp(rlse) + np.exp(np.float64(sk)))
    np.testing.assert_allclose(o3, ref * fac, rtol=0, atol=1e-13)


def test_all_chunks_empty():
    out, lse = oracle.lse_merge(np.zeros((3, 4)), np.full(3, -np.inf))
    assert np.all(out == 0) and np.isneginf(lse)
