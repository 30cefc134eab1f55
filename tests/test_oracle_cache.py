"""Pins for the oracle's cache rules and ring append (CPU only).

Fixed by the Spark export page:
  * `cache_len`: a 512-token window counts the current token, so the ring
    holds 511 previous entries and the roll layout 512; full layers hold
    the whole context;
  * `kv_cache_bytes` and the module docstring's footprint: 81 vs 235 at a
    4k context for the 28-layer model (golden/kv_footprint.json);
  * `_Layer.forward` (ring branch): the new entry goes into the slot for
    its position, evicting the oldest; attention itself equals what the
    roll layout computes over its re-sliced window.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads

HERE = os.path.dirname(os.path.abspath(__file__))
W = 512


def test_kv_footprint_matches_page():
    gold = json.load(open(os.path.join(HERE, "golden", "kv_footprint.json")))
    lt = workloads.layer_pattern(gold["layers"])
    assert lt.count(workloads.FULL) == 7 and lt.count(workloads.SLIDING) == 21
    ring = oracle.kv_cache_bytes(lt, gold["context"], W, True, 2, 256)
    roll = oracle.kv_cache_bytes(lt, gold["context"], W, False, 2, 256)
    div = gold["printed_unit_divisor"]
    for r in (ring, roll):
        assert round(r["hybrid"] / div) == gold["printed_hybrid"]
        assert round(r["uniform"] / div) == gold["printed_uniform"]
    # the exact byte counts these round from
    assert ring["hybrid"] == (7 * 4096 + 21 * 511) * 2048 == 80_697_344
    assert roll["hybrid"] == (7 * 4096 + 21 * 512) * 2048 == 80_740_352
    assert ring["uniform"] == 28 * 4096 * 2048 == 234_881_024


def test_cache_len_rules():
    S, F = workloads.SLIDING, workloads.FULL
    assert oracle.cache_len(S, 100, W, True) == 100
    assert oracle.cache_len(S, 511, W, True) == 511
    assert oracle.cache_len(S, 4096, W, True) == 511
    assert oracle.cache_len(S, 4096, W, False) == 512
    assert oracle.cache_len(F, 4096, W, True) == 4096
    # ring cache plus the new token is exactly one window
    assert oracle.cache_len(S, 4096, W, True) + 1 == W


@pytest.mark.parametrize("pos,slot", [(0, 0), (1, 1), (509, 509), (510, 510), (511, 0),
                                      (512, 1), (1023, 1), (4095, 7), (32767, 63)])
def test_ring_slot(pos, slot):
    # 1023 = 2*511 + 1; 4095 = 8*511 + 7; 32767 = 64*511 + 63
    assert oracle.ring_slot(pos, W) == slot


def _layer(seed, B, lt, lmax=64):
    """Oracle-form inputs: a sliding block splits into the 511-slot ring and
    its last row, the side row."""
    shape = workloads.HybridShape(batch=B, lmax=lmax)
    g = workloads.generator(seed)
    t = {k: workloads.bits(v).copy() for k, v in workloads.layer_inputs(g, shape, lt).items()}
    if lt == workloads.SLIDING:
        for a in ("k", "v"):
            blk = t[a]
            t[a] = np.ascontiguousarray(blk[:, :, :W - 1])
            t[a + "ev"] = np.ascontiguousarray(blk[:, :, W - 1])
    return shape, t


@pytest.mark.parametrize("pos", [0, 1, 509, 510, 511, 512, 1023, 4095])
def test_sliding_append_bit_exact(pos):
    shape, t = _layer(10 + pos, 2, workloads.SLIDING)
    before = {k: v.copy() for k, v in t.items()}
    B = 2
    kev = t["kev"]
    vev = t["vev"]
    posv = np.array([pos, pos], dtype=np.int32)
    oracle.rope_append(t["q"], t["k_new"], t["v_new"], posv, workloads.SLIDING, 256, 1e4, W,
                       t["k"], t["v"], kev, vev)
    s = pos % 511
    for b in range(B):
        for h in range(2):
            # new V lands verbatim in slot s; new K is its rotation
            assert np.array_equal(t["v"][b, h, s], before["v_new"][b, h])
            assert np.array_equal(t["k"][b, h, s],
                                  oracle.rope_apply(before["k_new"][b, h][None], 256, 1e4, pos)[0])
            # every other slot untouched
            mask = np.ones(511, bool)
            mask[s] = False
            assert np.array_equal(t["k"][b, h, mask], before["k"][b, h, mask])
            assert np.array_equal(t["v"][b, h, mask], before["v"][b, h, mask])
            if pos >= 511:
                # side row holds the evicted entry (position pos - 511)
                assert np.array_equal(kev[b, h], before["k"][b, h, s])
                assert np.array_equal(vev[b, h], before["v"][b, h, s])
            else:
                assert np.array_equal(kev[b, h], before["kev"][b, h])
                assert np.array_equal(vev[b, h], before["vev"][b, h])
    assert np.array_equal(t["q"], oracle.rope_apply(before["q"], 256, 1e4, pos))


def test_full_append_bit_exact():
    shape, t = _layer(3, 2, workloads.FULL, lmax=64)
    before = {k: v.copy() for k, v in t.items()}
    posv = np.array([5, 63], dtype=np.int32)
    dummy = np.zeros((2, 2, 256), np.uint16)
    oracle.rope_append(t["q"], t["k_new"], t["v_new"], posv, workloads.FULL, 64, 5e6, W,
                       t["k"], t["v"], dummy, dummy.copy())
    for b, p in enumerate(posv):
        for h in range(2):
            assert np.array_equal(t["v"][b, h, p], before["v_new"][b, h])
            kr = oracle.rope_apply(before["k_new"][b, h][None], 64, 5e6, int(p))[0]
            assert np.array_equal(t["k"][b, h, p], kr)
            assert np.array_equal(t["k"][b, h, p, 64:], before["k_new"][b, h, 64:])
            mask = np.ones(64, bool)
            mask[p] = False
            assert np.array_equal(t["k"][b, h, mask], before["k"][b, h, mask])


@pytest.mark.parametrize("lt", [workloads.SLIDING, workloads.FULL])
def test_append_outside_cache_writes_nothing(lt):
    """A position outside the cache -- negative (an inactive sequence), or
    at or past capacity on a full layer -- writes no row anywhere (the
    block, the side row, and the neighbouring sequences' blocks, which a
    row index of -1 or capacity would reach), while q is still rotated at
    that position; sequences in the cache append as usual."""
    shape, t = _layer(7, 3, lt, lmax=64)
    before = {k: v.copy() for k, v in t.items()}
    cap = t["k"].shape[2]
    posv = np.array([-1, 20, cap if lt == workloads.FULL else -3], dtype=np.int32)
    kev = t.get("kev", np.zeros((3, 2, 256), np.uint16))
    vev = t.get("vev", np.zeros((3, 2, 256), np.uint16))
    kev0, vev0 = kev.copy(), vev.copy()
    rot, theta = (256, 1e4) if lt == workloads.SLIDING else (64, 5e6)
    oracle.rope_append(t["q"], t["k_new"], t["v_new"], posv, lt, rot, theta, W,
                       t["k"], t["v"], kev, vev)
    for b in (0, 2):
        assert np.array_equal(t["k"][b], before["k"][b]) and np.array_equal(t["v"][b], before["v"][b])
        assert np.array_equal(kev[b], kev0[b]) and np.array_equal(vev[b], vev0[b])
        assert np.array_equal(t["q"][b], oracle.rope_apply(before["q"][b], rot, theta, int(posv[b])))
    # sequence 1 appended its row and nothing else
    row = oracle.ring_slot(20, W) if lt == workloads.SLIDING else 20
    assert np.array_equal(t["v"][1, :, row], before["v_new"][1])
    mask = np.ones(cap, bool)
    mask[row] = False
    assert np.array_equal(t["k"][1][:, mask], before["k"][1][:, mask])
    assert np.array_equal(t["v"][1][:, mask], before["v"][1][:, mask])


def _roll_attention(qv, keys, vals, scale):
    """Plain softmax attention over a contiguous window (fp64 torch)."""
    q = torch.from_numpy(oracle.bf16_to_f64(qv))
    k = torch.from_numpy(oracle.bf16_to_f64(np.stack(keys)))
    v = torch.from_numpy(oracle.bf16_to_f64(np.stack(vals)))
    return torch.softmax(k @ q * scale, 0) @ v


def test_ring_equals_roll_streaming():
    """Stream 1100 tokens: the ring (511 slots + side row) always holds
    exactly the roll layout's window, and attention over it equals roll's."""
    g = workloads.generator(7)
    Hkv, D = 1, 256
    k = np.zeros((1, Hkv, 511, D), np.uint16)
    v = np.zeros((1, Hkv, 511, D), np.uint16)
    kev = np.zeros((1, Hkv, D), np.uint16)
    vev = np.zeros((1, Hkv, D), np.uint16)
    win_k, win_v = [], []
    checks = set(range(0, 20)) | set(range(505, 520)) | {700, 1021, 1022, 1023, 1099}
    for pos in range(1100):
        q = workloads.bits(workloads.randn_bf16(g, (1, 1, D))).copy()
        kn = workloads.bits(workloads.randn_bf16(g, (1, Hkv, D))).copy()
        vn = workloads.bits(workloads.randn_bf16(g, (1, Hkv, D))).copy()
        q0 = q.copy()
        oracle.rope_append(q, kn, vn, np.array([pos], np.int32), workloads.SLIDING, 256, 1e4,
                           W, k, v, kev, vev)
        # roll: append the rotated entry, keep the last 512 ([SPARK] roll branch)
        win_k.append(oracle.rope_apply(kn[0, 0][None], 256, 1e4, pos)[0])
        win_v.append(vn[0, 0].copy())
        if len(win_k) > W:
            win_k.pop(0)
            win_v.pop(0)
        if pos in checks:
            n = min(pos + 1, 511)
            ring_rows = {k[0, 0, i].tobytes() + v[0, 0, i].tobytes() for i in range(n)}
            if pos >= 511:
                ring_rows.add(kev[0, 0].tobytes() + vev[0, 0].tobytes())
            roll_rows = {a.tobytes() + b.tobytes() for a, b in zip(win_k, win_v)}
            assert ring_rows == roll_rows
            out, lse = oracle.decode_attn(q, k, v, kev, vev, np.array([pos + 1]),
                                          workloads.SLIDING, W, None, 1 / 16)
            ref = _roll_attention(q[0, 0], win_k, win_v, 1 / 16).numpy()
            np.testing.assert_allclose(out[0, 0], ref, rtol=0, atol=1e-12)
