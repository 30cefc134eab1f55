"""GPU parity of the sparse top-k decode (one latent KV head, 64 query
heads, value = leading 512 of 576 dims, per-head sink) against the fp64
oracle, through the C ABI.

Tolerance: attention out max-abs <= 1e-2, mean-abs <= 1e-3 (unit-normal
bf16 inputs, fp32 accumulation); lse within 1e-4.  Pool rows no index names
are NaN-poisoned, so a read of one shows up as a non-finite output.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from hybrid_case import assert_attn_close, to_f64

pytestmark = pytest.mark.gpu

BF16_NAN = 0x7FC0


def _case(seed, T, H, pool, topk, poison=True):
    g = workloads.generator(seed)
    s = workloads.SparseShape(tokens=T, num_q_heads=H, pool=pool, topk=topk)
    t = workloads.sparse_inputs(g, s)
    h = {"q": workloads.bits(t["q"]).copy(), "kv": workloads.bits(t["kv"]).copy(),
         "indices": t["indices"].numpy().copy(), "sinks": t["sinks"].numpy().copy()}
    if poison:
        used = np.zeros(pool, bool)
        used[h["indices"][h["indices"] >= 0]] = True
        h["kv"][~used] = BF16_NAN
    return h


def _gpu(h, topk_length=None, sinks=None, scale=1 / 24):
    import full_kv_cache_amd as hda
    T, H, _ = h["q"].shape
    topk = h["indices"].shape[1]
    q = workloads.from_bits(h["q"]).cuda()
    kv = workloads.from_bits(h["kv"]).cuda()
    idx = torch.from_numpy(h["indices"]).cuda()
    tl = None if topk_length is None else torch.from_numpy(np.asarray(topk_length, np.int32)).cuda()
    sk = None if sinks is None else torch.from_numpy(np.asarray(sinks, np.float32)).cuda()
    out = torch.full((T, H, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    nbytes = hda.hda_sparse_workspace_bytes(T, H, topk)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda") if nbytes else None
    hda.hda_sparse_decode_attn(q, kv, idx, tl, sk, scale, out, lse, ws)
    torch.cuda.synchronize()
    return out, lse


def _ref(h, topk_length=None, sinks=None, scale=1 / 24):
    tl = None if topk_length is None else np.asarray(topk_length, np.int32)
    return oracle.sparse_decode_attn(h["q"], h["kv"], h["indices"], tl, sinks, scale, 512)


def _print_case(**kw):
    print("CASE", " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


@pytest.mark.parametrize("T,H,pool,topk", [(3, 64, 4096, 300), (2, 16, 1000, 77), (64, 64, 8192, 256),
                                           (5, 32, 2048, 1024), (7, 48, 3000, 500), (300, 16, 4096, 2080),
                                           (9, 128, 2048, 700)])
def test_sparse_matches_oracle(T, H, pool, topk):
    """Ragged index rows (not a multiple of 16 or 32), split and unsplit
    plans: 48 heads leave a wave of the shared-tile kernel without heads;
    300 tokens x top-2080 need no split for the grid but two for the
    2048-key cap of a split; 128 heads take the head-group kernel."""
    _print_case(test="sparse", T=T, H=H, pool=pool, topk=topk)
    h = _case(T * 1000 + topk, T, H, pool, topk)
    ref, rlse = _ref(h)
    out, lse = _gpu(h)
    assert_attn_close(out, ref)
    np.testing.assert_allclose(to_f64(lse), rlse, rtol=0, atol=1e-4)


def test_sparse_topk_length_and_invalid_indices():
    """topk_length cuts each row (0 and > topk included); -1 padding and
    indices past the pool are skipped; a token with no key gives 0 / -inf."""
    _print_case(test="sparse_lengths")
    T, H, pool, topk = 6, 64, 3000, 200
    h = _case(7, T, H, pool, topk, poison=False)
    g = np.random.default_rng(3)
    h["indices"][1, g.choice(topk, 50, replace=False)] = -1
    h["indices"][2, :10] = pool + 5
    h["indices"][2, 10:20] = -7
    h["indices"][4, :] = -1
    lengths = [200, 150, 33, 0, 200, 1000]
    used = np.zeros(pool, bool)
    for t in range(T):
        row = h["indices"][t, :min(max(lengths[t], 0), topk)]
        used[row[(row >= 0) & (row < pool)]] = True
    h["kv"][~used] = BF16_NAN
    ref, rlse = _ref(h, lengths)
    out, lse = _gpu(h, lengths)
    live = [0, 1, 2, 5]
    assert_attn_close(out[live], ref[live])
    np.testing.assert_allclose(to_f64(lse)[live], rlse[live], rtol=0, atol=1e-4)
    for t in (3, 4):
        assert torch.all(out[t].float() == 0)
        assert torch.all(torch.isneginf(lse[t]))


def test_sparse_sinks():
    _print_case(test="sparse_sinks")
    T, H, pool, topk = 4, 64, 4096, 512
    h = _case(11, T, H, pool, topk)
    _, rlse = _ref(h)
    g = np.random.default_rng(5)
    sinks = (rlse.mean(0) + g.normal(0, 1.5, H)).astype(np.float32)  # near lse: moves the output
    ref, _ = _ref(h, sinks=sinks)
    out, _ = _gpu(h, sinks=sinks)
    assert_attn_close(out, ref)
    o_none, _ = _gpu(h)
    o_ninf, _ = _gpu(h, sinks=np.full(H, -np.inf, np.float32))
    assert torch.equal(o_none.view(torch.int16), o_ninf.view(torch.int16))
    o_pinf, _ = _gpu(h, sinks=np.full(H, np.inf, np.float32))
    assert torch.all(o_pinf.float() == 0)


def test_sparse_headline_shape_all():
    """32 tokens x 64 heads, pool 32768, top-2048 (the launch the bench
    times), sinks drawn near lse; every token is checked against the
    oracle."""
    _print_case(test="sparse_headline")
    h = _case(0, 32, 64, 32768, 2048, poison=False)
    _, lse0 = _ref(h)
    g = np.random.default_rng(32)
    sinks = (lse0.mean(0) + g.normal(0, 2.0, 64)).astype(np.float32)
    out, lse = _gpu(h, sinks=sinks)
    ref, rlse = _ref(h, sinks=sinks)
    assert_attn_close(out, ref)
    np.testing.assert_allclose(to_f64(lse), rlse, rtol=0, atol=1e-4)


# ------------------------------------------------------------ fp8 pool
# hda_sparse_decode_attn_fp8: e4m3 codes with one fp32 scale per pool row
# (the reading of the flashmla_sparse page's fp8 call), against the oracle's
# fp8 sparse decode; rows no index names hold NaN codes and NaN scales.

NAN8 = 0x7F


def _case8(seed, T, H, pool, topk, poison=True):
    h = _case(seed, T, H, pool, topk, poison=False)
    g = workloads.generator(seed + 1)
    h["codes"] = workloads.fp8_codes(g, (pool, 576)).numpy()
    h["scales"] = workloads.fp8_scales(g, (pool,)).numpy()
    if poison:
        used = np.zeros(pool, bool)
        used[h["indices"][h["indices"] >= 0]] = True
        h["codes"][~used] = NAN8
        h["scales"][~used] = np.nan
    return h


def _gpu8(h, sinks=None, scale=1 / 24):
    import full_kv_cache_amd as hda
    T, H, _ = h["q"].shape
    topk = h["indices"].shape[1]
    q = workloads.from_bits(h["q"]).cuda()
    codes = torch.from_numpy(h["codes"]).cuda()
    scales = torch.from_numpy(h["scales"]).cuda()
    idx = torch.from_numpy(h["indices"]).cuda()
    sk = None if sinks is None else torch.from_numpy(np.asarray(sinks, np.float32)).cuda()
    out = torch.full((T, H, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    nbytes = hda.hda_sparse_workspace_bytes(T, H, topk)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda") if nbytes else None
    hda.hda_sparse_decode_attn_fp8(q, codes, scales, idx, sk, scale, out, lse, ws)
    torch.cuda.synchronize()
    return out, lse


def _ref8(h, sinks=None, scale=1 / 24):
    return oracle.sparse_decode_attn_fp8(h["q"], h["codes"], h["scales"], h["indices"], sinks, scale, 512)


@pytest.mark.parametrize("T,H,pool,topk", [(4, 64, 4096, 512), (3, 16, 1000, 100), (2, 128, 2048, 300),
                                           (1, 64, 600, 17)])
def test_sparse_fp8_parity(T, H, pool, topk):
    _print_case(test="sparse_fp8", T=T, H=H, pool=pool, topk=topk)
    h = _case8(30 + T + H, T, H, pool, topk)
    h["indices"][0, topk // 2] = -1   # padding inside the list
    _, lse0 = _ref8(h)
    g = np.random.default_rng(T + H)
    sinks = (lse0.mean(0) + g.normal(0, 2.0, H)).astype(np.float32)
    ref, rlse = _ref8(h, sinks=sinks)
    out, lse = _gpu8(h, sinks=sinks)
    assert_attn_close(out, ref)
    np.testing.assert_allclose(to_f64(lse), rlse, rtol=0, atol=1e-4)
    o_none, _ = _gpu8(h)
    o_ninf, _ = _gpu8(h, sinks=np.full(H, -np.inf, np.float32))
    assert torch.equal(o_none.view(torch.int16), o_ninf.view(torch.int16))


def test_sparse_fp8_headline_shape_all():
    """32 tokens x 64 heads, pool 32768, top-2048 (the launch the bench
    times), sinks drawn near lse; every token against the oracle."""
    _print_case(test="sparse_fp8_headline")
    h = _case8(40, 32, 64, 32768, 2048, poison=False)
    _, lse0 = _ref8(h)
    g = np.random.default_rng(40)
    sinks = (lse0.mean(0) + g.normal(0, 2.0, 64)).astype(np.float32)
    out, lse = _gpu8(h, sinks=sinks)
    ref, rlse = _ref8(h, sinks=sinks)
    assert_attn_close(out, ref)
    np.testing.assert_allclose(to_f64(lse), rlse, rtol=0, atol=1e-4)


@pytest.mark.parametrize("fp8", [False, True])
def test_sparse_late_large_score(fp8):
    """A key far into the list scoring ~46 above the first tile's maximum
    for one head (more than the 2^32 weight slack against the kernel's
    fixed softmax reference): the wave scores its keys again against the
    exact maximum; results as the oracle's."""
    _print_case(test="sparse_late_large", fp8=fp8)
    # bf16: 64 tokens in 4 key splits of 256, so list position 900 is the
    # fifth 32-key tile of its split, scored after the first set the
    # reference; fp8: 64 tokens x 4 head groups, no split, so it is tile 56
    # of its token, the 15th tile of the wave that scores it
    T, H, pool, topk = 64, 64, 4096, 1024
    h = _case(50, T, H, pool, topk, poison=False)
    qrow = oracle.bf16_to_f64(h["q"][0, 5])
    big = int(h["indices"][0, 900])
    h["kv"][big] = workloads.bits(torch.from_numpy(2.0 * qrow).to(torch.bfloat16))
    if fp8:
        codes, scales = oracle.quant_rows(h["kv"])
        h["codes"], h["scales"] = codes, scales
        ref, rlse = _ref8(h)
        out, lse = _gpu8(h)
    else:
        ref, rlse = _ref(h)
        out, lse = _gpu(h)
    assert rlse[0, 5] > 40
    # head 5 of token 0 is that row's value (2 q, entries up to ~8): its
    # bf16 roundings (the weight times the row scale, out itself) are
    # relative, so the bound scales with |out| there
    got = to_f64(out)
    assert np.all(np.isfinite(got))
    assert np.all(np.abs(got - ref) <= 1e-2 * np.maximum(1.0, np.abs(ref)))
    # the other rows: the planted row is large (entries up to ~8) and many
    # queries put most of their weight on it, so outputs reach |out| ~ 2-8,
    # where a bf16 output's spacing (2^-6 at 2) alone exceeds an absolute
    # 1e-2; the bound is relative there as well, the mean stays absolute
    rest = np.ones(ref.shape[:2], bool)
    rest[0, 5] = False
    err = np.abs(got[rest] - ref[rest])
    assert np.all(err <= 1e-2 * np.maximum(1.0, np.abs(ref[rest])))
    assert err.mean() <= 1e-3
    np.testing.assert_allclose(to_f64(lse), rlse, rtol=0, atol=1e-4)
