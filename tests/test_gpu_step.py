"""GPU parity of the fused one-launch decode step (hda_decode_step: RoPE,
append, attention, merge, sink) against the fp64 oracle's append followed
by its attention.

Cache after the call: bit-exact for V and every untouched row, rotated K
within one bf16 ulp (< 0.1% of values off); out max-abs <= 1e-2, mean-abs
<= 1e-3; lse within 1e-4.  Rows the step must not read are NaN-poisoned,
including the stale evicted-entry row of a full sliding window.
"""
import numpy as np
import pytest
import torch

from hybrid_case import (BF16_NAN, FULL, SLIDING, HybridCase, assert_attn_close, assert_rotated_close,
                         bits_of, fused_step, near_lse_sinks, to_f64)

pytestmark = pytest.mark.gpu


def _print_case(**kw):
    print("CASE", " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


def _check_cache(d, h):
    assert np.array_equal(bits_of(d["v"]), h["v"])
    assert_rotated_close(bits_of(d["k"]), h["k"])


def _poison_stale_evicted_row(case):
    """Row window-1 of a sliding block holds the entry evicted one step
    earlier, outside this step's window: the step must not use it."""
    if case.lt != SLIDING:
        return
    W = case.shape.window
    for b, p in enumerate(case.pos):
        if p >= W:
            case.host["k"][b, :, W - 1] = BF16_NAN
            case.host["v"][b, :, W - 1] = BF16_NAN


@pytest.mark.parametrize("pos", [0, 1, 15, 16, 17, 509, 510, 511, 512, 1000, 1021, 4095])
def test_step_sliding_positions(pos):
    _print_case(test="step_sliding", pos=pos)
    case = HybridCase(900 + pos, 3, SLIDING, [pos, max(0, pos - 3), pos + 511], poison=True)
    _poison_stale_evicted_row(case)
    h, ref, rlse = case.oracle_step()
    d, out, lse = fused_step(case)
    _check_cache(d, h)
    assert np.array_equal(bits_of(d["q"]), case.host["q"])  # q is only read
    assert_attn_close(out, ref)
    np.testing.assert_allclose(to_f64(lse), rlse, rtol=0, atol=1e-4)


def test_step_full_ragged():
    pos = [0, 15, 16, 999, 2047, 3000]
    _print_case(test="step_full", pos=pos)
    case = HybridCase(950, len(pos), FULL, pos, lmax=3072, poison=True)
    h, ref, rlse = case.oracle_step()
    d, out, lse = fused_step(case)
    _check_cache(d, h)
    assert_attn_close(out, ref)
    np.testing.assert_allclose(to_f64(lse), rlse, rtol=0, atol=1e-4)


@pytest.mark.parametrize("lt", [SLIDING, FULL])
def test_step_sinks(lt):
    _print_case(test="step_sinks", lt=lt)
    case = HybridCase(960 + lt, 2, lt, [700, 1200], lmax=2048)
    _, ref0, lse0 = case.oracle_step()
    g = np.random.default_rng(2)
    sinks = (lse0.mean(0) + g.normal(0, 2, 8)).astype(np.float32)
    _, ref, _ = case.oracle_step(sinks=sinks)
    _, out, _ = fused_step(case, sinks=sinks)
    assert_attn_close(out, ref)
    _, o_none, _ = fused_step(case)
    _, o_ninf, _ = fused_step(case, sinks=np.full(8, -np.inf, np.float32))
    assert torch.equal(o_none.view(torch.int16), o_ninf.view(torch.int16))
    assert_attn_close(o_none, ref0)
    _, o_pinf, _ = fused_step(case, sinks=np.full(8, np.inf, np.float32))
    assert torch.all(o_pinf.float() == 0)


def test_step_outside_cache():
    """Positions outside a full layer's cache: a negative one attends to
    nothing and writes nothing; one past the capacity attends to the cached
    rows only (q still rotated by its position) and appends nothing.  The
    oracle covers the in-cache sequence and the attention of the other."""
    _print_case(test="step_outside")
    import oracle
    case = HybridCase(970, 3, FULL, [10, 63, 63], lmax=64)
    case.pos = np.array([-1, 63, 80], np.int32)
    d, out, lse = fused_step(case)
    k_gpu, v_gpu = bits_of(d["k"]), bits_of(d["v"])
    for b in (0, 2):  # nothing appended
        assert np.array_equal(k_gpu[b], case.host["k"][b])
        assert np.array_equal(v_gpu[b], case.host["v"][b])
    assert torch.all(out[0].float() == 0) and torch.all(torch.isneginf(lse[0]))
    # sequence 1: an ordinary step at the last row
    sub = HybridCase(970, 3, FULL, [10, 63, 63], lmax=64)
    for key in sub.host:
        sub.host[key] = sub.host[key][1:2].copy()
    sub.pos, sub.seq_lens = np.array([63], np.int32), np.array([64], np.int32)
    sub.shape = sub.shape.__class__(batch=1, lmax=64)
    h, ref, rlse = sub.oracle_step()
    assert np.array_equal(v_gpu[1:2], h["v"])
    assert_rotated_close(k_gpu[1:2], h["k"])
    assert_attn_close(out[1:2], ref)
    np.testing.assert_allclose(to_f64(lse)[1:2], rlse, rtol=0, atol=1e-4)
    # sequence 2: q rotated at 80, keys = the 64 cached rows
    s = case.shape
    q2 = oracle.rope_apply(case.host["q"][2:3], s.rot_full, s.theta_full, 80)
    z = np.zeros((1, 2, 256), np.uint16)
    ref2, rlse2 = oracle.decode_attn(q2, case.host["k"][2:3], case.host["v"][2:3], z, z.copy(),
                                     np.array([64], np.int32), FULL, s.window, None, 1 / 16)
    assert_attn_close(out[2:3], ref2)
    np.testing.assert_allclose(to_f64(lse)[2:3], rlse2, rtol=0, atol=1e-4)


def test_step_full_short_batch_twice():
    """The step's grid is sized from the cache capacity; short sequences in
    a large cache hold far fewer rounds (22) than the grid has waves (512).
    Every pair is still merged, and the arrival counters come back to zero
    so that a second call on the same workspace is right as well."""
    _print_case(test="step_full_short")
    import full_kv_cache_amd as hda
    pos = np.array([0, 3, 20, 100], np.int32)
    case = HybridCase(990, 4, FULL, pos, lmax=4096, poison=True)
    d = case.device()
    ws = torch.zeros(hda.hda_decode_step_workspace_bytes(case.cache(d), FULL), dtype=torch.uint8,
                     device="cuda")
    h, ref, rlse = case.oracle_step()
    for _ in range(2):  # the second call re-appends the same rows
        d, out, lse = fused_step(case, d=d, workspace=ws)
        _check_cache(d, h)
        assert_attn_close(out, ref)
        np.testing.assert_allclose(to_f64(lse), rlse, rtol=0, atol=1e-4)
        assert torch.count_nonzero(ws[: 4 * 4 * 2]).item() == 0


@pytest.mark.parametrize("lt", [SLIDING, FULL])
def test_step_twice_same_workspace(lt):
    """Two consecutive steps on one workspace: the arrival counters come
    back to zero, and the second step sees the first one's append."""
    _print_case(test="step_twice", lt=lt)
    import full_kv_cache_amd as hda
    pos0 = np.array([520, 1500, 2047], np.int32)
    case = HybridCase(980 + lt, 3, lt, pos0, lmax=2049)
    d = case.device()
    ws = torch.zeros(hda.hda_decode_step_workspace_bytes(case.cache(d), lt), dtype=torch.uint8,
                     device="cuda")
    d, _, _ = fused_step(case, d=d, workspace=ws)
    h1, _, _ = case.oracle_step()
    case2 = HybridCase(981 + lt, 3, lt, pos0 + 1, lmax=2049)  # fresh q / k_new / v_new
    for key in ("k", "v"):
        case2.host[key] = h1[key]
    d2 = case2.device()
    d2["k"], d2["v"] = d["k"], d["v"]
    d2, out, lse = fused_step(case2, d=d2, workspace=ws)
    h2, ref, rlse = case2.oracle_step()
    _check_cache(d2, h2)
    assert_attn_close(out, ref)
    np.testing.assert_allclose(to_f64(lse), rlse, rtol=0, atol=1e-4)
    assert torch.count_nonzero(ws[: 4 * 3 * 2]).item() == 0


def test_step_graph_replay():
    """A captured full-layer step replays to the eager result (the full
    layer's append is idempotent for a fixed position)."""
    _print_case(test="step_graph")
    import full_kv_cache_amd as hda
    case = HybridCase(990, 4, FULL, [100, 700, 1300, 2000], lmax=2048)
    d = case.device()
    cache = case.cache(d)
    pos = torch.from_numpy(case.pos).cuda()
    ws = torch.zeros(hda.hda_decode_step_workspace_bytes(cache, FULL), dtype=torch.uint8, device="cuda")
    out = torch.empty(4, 8, 256, dtype=torch.bfloat16, device="cuda")
    sk = torch.randn(8, generator=torch.Generator().manual_seed(0)).cuda()

    def step():
        hda.hda_decode_step(d["q"], d["k_new"], d["v_new"], pos, FULL, cache, sk, 1 / 16, out, None, ws)

    step()
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(4):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16))


def test_step_batch64_all():
    """Headline shape: batch 64, lengths uniform in [512, 4096], sinks drawn
    near lse, in the launch configuration the bench times; every sequence
    is checked against the oracle (the balanced streaming partition of a
    full layer cuts sequences at data-dependent places)."""
    _print_case(test="step_batch64")
    g = np.random.default_rng(64)
    pos = g.integers(511, 4096, 64).astype(np.int32)
    for lt in (SLIDING, FULL):
        case = HybridCase(1000 + lt, 64, lt, pos, lmax=4096)
        _, _, lse0 = case.oracle_step()
        sinks = near_lse_sinks(lse0, 70 + lt)
        h, ref, rlse = case.oracle_step(sinks=sinks)
        d, out, lse = fused_step(case, sinks=sinks)
        assert_attn_close(out, ref)
        np.testing.assert_allclose(to_f64(lse), rlse, rtol=0, atol=1e-4)
        _check_cache(d, h)


@pytest.mark.parametrize("hq", [8, 4])
def test_step_sliding_batch64_edges(hq):
    """A sliding layer at batch 64 takes the head split of the window step
    (two workgroups per (sequence, KV head), each serving half the query
    heads over every key; the last to count in appends; query groups of 4
    and 2): the ring's edge positions
    (empty window, first rows, the fill at 510 / 511, wrap-around) among
    random ones, the stale evicted-entry row poisoned, sinks near lse and
    the output gate, against the oracle; one sequence inactive (pos -1:
    out 0, lse -inf, its block untouched)."""
    _print_case(test="step_sliding_batch64_edges", hq=hq)
    edge = [0, 1, 15, 16, 17, 509, 510, 511, 512, 1000, 1021, 4095]
    g = np.random.default_rng(640)
    pos = np.concatenate([edge, g.integers(0, 4096, 64 - len(edge))]).astype(np.int32)
    neg = 40  # inactive on the device; the oracle runs it at its drawn position
    case = HybridCase(1640 + hq, 64, SLIDING, pos, poison=True, num_q_heads=hq)
    _poison_stale_evicted_row(case)
    _, _, lse0 = case.oracle_step()
    sinks = near_lse_sinks(lse0, 641)
    gate = g.uniform(-3, 3, size=(64, case.shape.num_q_heads)).astype(np.float32)
    h, ref, rlse = case.oracle_step(sinks=sinks, gate=gate)
    case.pos = case.pos.copy()
    case.pos[neg] = -1
    d, out, lse = fused_step(case, sinks=sinks, gate=gate)
    live = np.arange(64) != neg
    assert_attn_close(out[torch.from_numpy(live)], ref[live])
    np.testing.assert_allclose(to_f64(lse)[live], rlse[live], rtol=0, atol=1e-4)
    assert torch.all(out[neg].float() == 0) and torch.all(torch.isneginf(lse[neg]))
    k_gpu, v_gpu = bits_of(d["k"]), bits_of(d["v"])
    assert np.array_equal(v_gpu[live], h["v"][live])
    assert_rotated_close(k_gpu[live], h["k"][live])
    assert np.array_equal(k_gpu[neg], case.host["k"][neg])
    assert np.array_equal(v_gpu[neg], case.host["v"][neg])


def test_step_full_rotary_256():
    """Full layer with the whole head rotated (rotary_dim 256: the q
    operand's chunk j pairs with chunk j + 4 in the step form's in-register
    rotation; the merge rotates 4 dims per lane against dim +- 128)."""
    import dataclasses
    pos = [0, 40, 1100, 2047]
    _print_case(test="step_full_rot256", pos=pos)
    case = HybridCase(1100, len(pos), FULL, pos, lmax=2048, poison=True)
    case.shape = dataclasses.replace(case.shape, rot_full=256, theta_full=1e4)
    h, ref, rlse = case.oracle_step()
    d, out, lse = fused_step(case)
    _check_cache(d, h)
    assert np.array_equal(bits_of(d["q"]), case.host["q"])
    assert_attn_close(out, ref)
    np.testing.assert_allclose(to_f64(lse), rlse, rtol=0, atol=1e-4)


@pytest.mark.parametrize("page_size", [16, 64])
def test_step_full_paged(page_size):
    """The full-layer step on a paged cache: the new row lands in the page
    its table names (no spare page changes), out/lse match the oracle and
    are bit-identical to the same step on the contiguous cache."""
    import full_kv_cache_amd as hda
    import oracle
    import workloads
    from test_gpu_paged import _page
    pos = [0, 15, 16, 300, 2047]
    _print_case(test="step_full_paged", page_size=page_size, pos=pos)
    case = HybridCase(1200 + page_size, len(pos), FULL, pos, lmax=2048, poison=True)
    s = case.shape
    h, ref, rlse = case.oracle_step()
    pk, pv, table, spare = _page(case, page_size)
    pool_k, pool_v = workloads.from_bits(pk).cuda(), workloads.from_bits(pv).cuda()
    d = case.device()
    cache = hda.LayerCache(pool_k, pool_v, s.num_q_heads, s.window, s.rot(FULL), s.theta(FULL),
                           block_table=torch.from_numpy(table).cuda())
    ws = torch.zeros(hda.hda_decode_step_workspace_bytes(cache, FULL), dtype=torch.uint8, device="cuda")
    out = torch.full((s.batch, s.num_q_heads, s.head_dim), float("nan"), dtype=torch.bfloat16,
                     device="cuda")
    lse = torch.full((s.batch, s.num_q_heads), float("nan"), device="cuda")
    hda.hda_decode_step(d["q"], d["k_new"], d["v_new"], torch.from_numpy(case.pos).cuda(), FULL, cache,
                        None, 1 / 16, out, lse, ws)
    torch.cuda.synchronize()
    gk, gv = oracle.page_gather(bits_of(pool_k), table), oracle.page_gather(bits_of(pool_v), table)
    for b, n in enumerate(case.seq_lens):
        assert np.array_equal(gv[b, :, :n], h["v"][b, :, :n]), b
        assert_rotated_close(gk[b, :, :n], h["k"][b, :, :n])
    assert np.array_equal(bits_of(pool_k)[spare], pk[spare])
    assert np.array_equal(bits_of(pool_v)[spare], pv[spare])
    assert_attn_close(out, ref)
    np.testing.assert_allclose(to_f64(lse), rlse, rtol=0, atol=1e-4)
    _, out_c, lse_c = fused_step(case)
    assert torch.equal(out.view(torch.int16), out_c.view(torch.int16))
    assert torch.equal(lse, lse_c)


def test_step_full_matches_two_calls():
    """The full-layer step against hda_rope_append + hda_decode_attn on
    the same inputs: the same cache bit for bit, out within the decode
    tolerance of each other (the new key is scored by the merge instead of
    a round, so the sums differ in order only)."""
    pos = [3, 500, 1999, 4095]
    _print_case(test="step_full_vs_two_calls", pos=pos)
    case = HybridCase(1300, len(pos), FULL, pos, lmax=4096, poison=True)
    d1, out1, lse1 = fused_step(case)
    d2, out2, lse2 = case.gpu_step(max_seq_len=4096)
    assert torch.equal(d1["k"].view(torch.int16), d2["k"].view(torch.int16))
    assert torch.equal(d1["v"].view(torch.int16), d2["v"].view(torch.int16))
    assert_attn_close(out1, to_f64(out2))
    np.testing.assert_allclose(to_f64(lse1), to_f64(lse2), rtol=0, atol=1e-5)


@pytest.mark.parametrize("pos", [[0, 100, 2046, 2047, 5000], [1023, 1024, 4095]])
def test_step_wide_sliding_window(pos):
    """A sliding window of 2048 keys (past one workgroup's 1024): the step
    takes the one-launch streaming form (decode_step_kernel: RoPE, the ring
    append with eviction, attention, last-arriver merge); against the
    oracle, with sinks, twice on one workspace (counters back at zero)."""
    import full_kv_cache_amd as hda
    _print_case(test="step_wide_window", pos=pos)
    case = HybridCase(1400 + len(pos), len(pos), SLIDING, pos, window=2048, poison=True)
    _poison_stale_evicted_row(case)
    sinks = np.linspace(-1.0, 3.0, case.shape.num_q_heads).astype(np.float32)
    h, ref, rlse = case.oracle_step(sinks=sinks)
    ws = None
    for _ in range(2):
        d = case.device()
        if ws is None:
            ws = torch.zeros(hda.hda_decode_step_workspace_bytes(case.cache(d), SLIDING),
                             dtype=torch.uint8, device="cuda")
        d, out, lse = fused_step(case, sinks=sinks, d=d, workspace=ws)
        _check_cache(d, h)
        assert_attn_close(out, ref)
        np.testing.assert_allclose(to_f64(lse), rlse, rtol=0, atol=1e-4)
        assert torch.count_nonzero(ws[: 4 * len(pos) * 2]).item() == 0
