"""GPU parity of the FP8 KV cache (e4m3 codes, one fp32 scale per row; the
reading of the flashmla_sparse page's fp8 call) against the fp64 oracle.

The cache starts as seeded random codes (never NaN) with scales in
[1, 2) / 448; q, k_new, v_new are unit-normal bf16 as for the bf16 path.
Rows the step must not read hold NaN codes and NaN scales.  Checked:
  * hda_rope_append: q rotated as on the bf16 path (within one bf16 ulp);
    V codes and scales bit-exact everywhere; K bit-exact on every row but
    the appended one, whose rotated values may differ from the oracle's by
    one bf16 ulp -- there codes within one step and the scale within one
    bf16 ulp; crafted rows pin ties-to-even, subnormal codes, the largest
    code and an all-zero row bit for bit;
  * hda_decode_attn on the window kernel (sliding, short full) and the
    streaming kernel (long full, paged): out max-abs <= 1e-2, mean-abs
    <= 1e-3, lse within 1e-4 of the oracle's attention over its own
    quantized cache; with sinks and the output gate.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from hybrid_case import assert_attn_close, assert_rotated_close, bits_of, to_f64
from workloads import FULL, SLIDING

pytestmark = pytest.mark.gpu
W = 512
NAN8 = 0x7F


class Fp8Case:
    def __init__(self, seed, lt, pos, lmax=None, hq=8, hkv=2):
        self.lt = lt
        self.pos = np.asarray(pos, np.int32)
        B = len(pos)
        lmax = lmax or int(self.pos.max()) + 1
        self.shape = workloads.HybridShape(batch=B, lmax=lmax, num_q_heads=hq, num_kv_heads=hkv)
        s = self.shape
        g = workloads.generator(seed)
        t = workloads.layer_inputs(g, workloads.HybridShape(batch=B, lmax=16, num_q_heads=hq,
                                                            num_kv_heads=hkv), lt)
        self.q, self.k_new, self.v_new = (workloads.bits(t[n]).copy() for n in ("q", "k_new", "v_new"))
        cap = s.capacity(lt)
        g8 = workloads.generator(seed + 1)
        self.kc = workloads.fp8_codes(g8, (B, s.num_kv_heads, cap, s.head_dim)).numpy()
        self.vc = workloads.fp8_codes(g8, (B, s.num_kv_heads, cap, s.head_dim)).numpy()
        self.ks = workloads.fp8_scales(g8, (B, s.num_kv_heads, cap)).numpy()
        self.vs = workloads.fp8_scales(g8, (B, s.num_kv_heads, cap)).numpy()
        for b, p in enumerate(self.pos):  # rows past pos are never read
            for a in (self.kc, self.vc):
                a[b, :, p + 1:] = NAN8
            for a in (self.ks, self.vs):
                a[b, :, p + 1:] = np.nan
        self.seq_lens = self.pos + 1

    # ------------------------------------------------------------ oracle
    def oracle_step(self, sinks=None, gate=None):
        s = self.shape
        q = self.q.copy()
        kc, vc, ks, vs = self.kc.copy(), self.vc.copy(), self.ks.copy(), self.vs.copy()
        if self.lt == SLIDING:
            sl = W - 1
            ring = [np.ascontiguousarray(a[:, :, :sl]) for a in (kc, vc, ks, vs)]
            side = [np.ascontiguousarray(a[:, :, sl]) for a in (kc, vc, ks, vs)]
        else:
            ring = [kc, vc, ks, vs]
            side = [np.zeros(kc.shape[:2] + (s.head_dim,), np.uint8) for _ in range(2)] + \
                   [np.zeros(kc.shape[:2], np.float32) for _ in range(2)]
        oracle.rope_append_fp8(q, self.k_new, self.v_new, self.pos, self.lt, s.rot(self.lt),
                               s.theta(self.lt), W, *ring, *side)
        out, lse = oracle.decode_attn_fp8(q, *ring, *side, self.seq_lens, self.lt, W, sinks,
                                          1 / 16, gate=gate)
        if self.lt == SLIDING:
            blocks = [np.concatenate([r, sd[:, :, None]], axis=2) for r, sd in zip(ring, side)]
        else:
            blocks = ring
        return q, blocks, out, lse

    # --------------------------------------------------------------- GPU
    def device(self):
        d = {n: workloads.from_bits(getattr(self, n)).cuda() for n in ("q", "k_new", "v_new")}
        for n in ("kc", "vc", "ks", "vs"):
            d[n] = torch.from_numpy(getattr(self, n)).cuda()
        return d

    def cache(self, d, block_table=None, kc=None, vc=None, ks=None, vs=None):
        import full_kv_cache_amd as hda
        s = self.shape
        return hda.LayerCache(d["kc"] if kc is None else kc, d["vc"] if vc is None else vc,
                              s.num_q_heads, W, s.rot(self.lt), s.theta(self.lt),
                              block_table=block_table, k_scale=d["ks"] if ks is None else ks,
                              v_scale=d["vs"] if vs is None else vs)

    def gpu_step(self, d=None, cache=None, sinks=None, gate=None, append=True):
        import full_kv_cache_amd as hda
        s = self.shape
        d = d or self.device()
        cache = cache or self.cache(d)
        if append:
            hda.hda_rope_append(d["q"], d["k_new"], d["v_new"], torch.from_numpy(self.pos).cuda(),
                                self.lt, cache)
        msl = int(self.seq_lens.max())
        nbytes = hda.hda_decode_workspace_bytes(cache, self.lt, msl, 0)
        ws = torch.zeros(max(nbytes, 1), dtype=torch.uint8, device="cuda")
        out = torch.full((s.batch, s.num_q_heads, s.head_dim), float("nan"), dtype=torch.bfloat16,
                         device="cuda")
        lse = torch.full((s.batch, s.num_q_heads), float("nan"), device="cuda")
        sk = None if sinks is None else torch.as_tensor(sinks).cuda()
        gt = None if gate is None else torch.as_tensor(gate).cuda()
        hda.hda_decode_attn(d["q"], cache, torch.from_numpy(self.seq_lens).cuda(), self.lt, sk,
                            1 / 16, out, lse, msl, 0, ws, gate=gt)
        torch.cuda.synchronize()
        return d, out, lse


def _check_append(case, d, q_ref, blocks, q_rotated=True):
    kc_ref, vc_ref, ks_ref, vs_ref = blocks
    if q_rotated:
        assert_rotated_close(bits_of(d["q"]), q_ref)
    else:  # the one-launch step only reads q
        assert np.array_equal(bits_of(d["q"]), case.q)
    kc, vc = d["kc"].cpu().numpy(), d["vc"].cpu().numpy()
    ks, vs = d["ks"].cpu().numpy(), d["vs"].cpu().numpy()
    assert np.array_equal(vc, vc_ref)
    assert np.array_equal(vs.view(np.uint32), vs_ref.view(np.uint32))
    cap = kc.shape[2]
    for b, p in enumerate(case.pos):
        row = p % (W - 1) if case.lt == SLIDING else p
        other = np.ones(cap, bool)
        other[row] = False
        assert np.array_equal(kc[b][:, other], kc_ref[b][:, other])
        assert np.array_equal(ks[b][:, other].view(np.uint32), ks_ref[b][:, other].view(np.uint32))
        # the appended K row: codes within one step (same sign), scale within one bf16 ulp
        got, ref = kc[b, :, row].astype(np.int32), kc_ref[b, :, row].astype(np.int32)
        same_sign = (got & 0x80) == (ref & 0x80)
        assert np.all(same_sign | ((got & 0x7F) == 0) | ((ref & 0x7F) == 0))
        assert np.abs((got & 0x7F) - (ref & 0x7F)).max() <= 1
        gs, rs = ks[b, :, row].astype(np.float64), ks_ref[b, :, row].astype(np.float64)
        assert np.all((gs == 0) == (rs == 0))  # an all-zero row has scale 0 on both sides
        nz = rs != 0
        assert np.all(np.abs(gs[nz] / rs[nz] - 1) <= 2.0 ** -7)


@pytest.mark.parametrize("lt,pos,lmax", [
    (SLIDING, [0, 15, 510, 511, 1500], None),   # window kernel; ring wrap and eviction
    (FULL, [0, 17, 300, 1023], 1024),            # window kernel on a short full layer
    (FULL, [5, 700, 2047, 1100], 2048),          # streaming kernel
])
def test_fp8_append_and_attention(lt, pos, lmax):
    print("CASE fp8", lt, pos, lmax, flush=True)
    case = Fp8Case(2000 + len(pos) + lt, lt, pos, lmax)
    Hq = case.shape.num_q_heads
    sk = np.linspace(-1.0, 3.0, Hq).astype(np.float32)
    g = np.random.default_rng(len(pos)).uniform(-3, 3, size=(len(pos), Hq)).astype(np.float32)
    q_ref, blocks, ref, rlse = case.oracle_step(sinks=sk, gate=g)
    d, out, lse = case.gpu_step(sinks=sk, gate=g)
    _check_append(case, d, q_ref, blocks)
    assert_attn_close(out, ref)
    np.testing.assert_allclose(to_f64(lse), rlse, rtol=0, atol=1e-4)


def test_fp8_quantize_ties_subnormals_zero():
    """Rows whose scale is exactly 1 or 1/2 (amax 448 or 224) carry values
    at exact ties between neighbouring codes, in the subnormal range and at
    the top; one sequence appends all-zero rows (scale 0, codes 0)."""
    print("CASE fp8 quantize crafted", flush=True)
    case = Fp8Case(2100, FULL, [3, 40, 77], 128)
    vals = np.array([448.0, 1.0625, 1.1875, -1.0625, 2.0 ** -10, 3 * 2.0 ** -10, -5 * 2.0 ** -11,
                     0.01, 300.0, 232.0, -240.0, 17.0, 2.0 ** -6, 15 * 2.0 ** -10], np.float32)
    row = np.resize(vals, 256).astype(np.float32)
    half = row / 2  # amax 224 -> scale 1/2: the same codes
    bits = lambda a: workloads.bits(torch.from_numpy(a).to(torch.bfloat16))
    case.v_new[0, 0], case.v_new[0, 1] = bits(row), bits(half)
    case.v_new[2], case.k_new[2] = 0, 0
    q_ref, blocks, ref, rlse = case.oracle_step()
    d, out, lse = case.gpu_step()
    _check_append(case, d, q_ref, blocks)
    vc = d["vc"].cpu().numpy()
    assert np.array_equal(vc[0, 0, 3], vc[0, 1, 3])
    assert d["vs"][0, 0, 3].item() == 1.0 and d["vs"][0, 1, 3].item() == 0.5
    assert np.all(vc[2, :, 77] == 0) and torch.all(d["vs"][2, :, 77] == 0)
    assert torch.all(d["ks"][2, :, 77] == 0)
    # sequence 0 attends to values up to 448: its outputs reach ~100, so the
    # bound there is relative -- P.V takes each probability rounded to bf16
    # (2^-9 relative) while the sum keeps fp32 weights (up to 2 x 2^-9), and
    # out itself is bf16 (2^-9): 3 x 2^-9 < 6e-3, bounded by 8e-3
    assert_attn_close(out[1:], ref[1:])
    got0 = to_f64(out[0])
    assert np.all(np.abs(got0 - ref[0]) <= 8e-3 * np.abs(ref[0]) + 1e-2)
    np.testing.assert_allclose(to_f64(lse), rlse, rtol=0, atol=1e-4)


def test_fp8_paged_matches_contiguous():
    """The fp8 cache in a shuffled pool of 64-row pages: the same result as
    the contiguous fp8 cache bit for bit, and the oracle's."""
    import full_kv_cache_amd as hda
    print("CASE fp8 paged", flush=True)
    ps = 64
    case = Fp8Case(2200, FULL, [63, 64, 1500, 5, 2047], 2048)
    s = case.shape
    q_ref, blocks, ref, rlse = case.oracle_step()
    _, out_c, lse_c = case.gpu_step()
    B, Hkv, cap, D = case.kc.shape
    mp = cap // ps
    perm = np.random.default_rng(9).permutation(B * mp + 3)
    def pool(a):
        shp = (B * mp + 3, Hkv, ps) + a.shape[3:]
        out = np.zeros(shp, a.dtype)
        pages = a.reshape((B, Hkv, mp, ps) + a.shape[3:]).swapaxes(1, 2).reshape((B * mp, Hkv, ps) + a.shape[3:])
        out[perm[:B * mp]] = pages
        return torch.from_numpy(out).cuda()
    d = case.device()
    kp, vp, ksp, vsp = (pool(getattr(case, n)) for n in ("kc", "vc", "ks", "vs"))
    table = torch.from_numpy(perm[:B * mp].reshape(B, mp).astype(np.int32)).cuda()
    cache = case.cache(d, block_table=table, kc=kp, vc=vp, ks=ksp, vs=vsp)
    _, out, lse = case.gpu_step(d=d, cache=cache)
    assert torch.equal(out.view(torch.int16), out_c.view(torch.int16))
    assert torch.equal(lse, lse_c)
    assert_attn_close(out, ref)
    np.testing.assert_allclose(to_f64(lse), rlse, rtol=0, atol=1e-4)


@pytest.mark.parametrize("pos", [[0, 15, 510, 511, 1500], [3, 700, 4095, 1022]])
def test_fp8_window_step(pos):
    """hda_decode_step on an fp8 sliding cache (one launch: RoPE, quantized
    append, attention): the cache after it and out / lse as for the
    two-call path; twice, from the same cache, on one workspace (the
    arrival counters return to zero)."""
    import full_kv_cache_amd as hda
    print("CASE fp8 window step", pos, flush=True)
    case = Fp8Case(2300 + len(pos), SLIDING, pos)
    Hq = case.shape.num_q_heads
    sk = np.linspace(-1.0, 3.0, Hq).astype(np.float32)
    g = np.random.default_rng(7).uniform(-3, 3, size=(len(pos), Hq)).astype(np.float32)
    q_ref, blocks, ref, rlse = case.oracle_step(sinks=sk, gate=g)
    ws = None
    for _ in range(2):  # the same step on a fresh copy of the cache, same workspace
        d = case.device()
        cache = case.cache(d)
        if ws is None:
            ws = torch.zeros(hda.hda_decode_step_workspace_bytes(cache, SLIDING), dtype=torch.uint8,
                             device="cuda")
        out = torch.full((len(pos), Hq, 256), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((len(pos), Hq), float("nan"), device="cuda")
        hda.hda_decode_step(d["q"], d["k_new"], d["v_new"], torch.from_numpy(case.pos).cuda(),
                            SLIDING, cache, torch.from_numpy(sk).cuda(), 1 / 16, out, lse, ws,
                            gate=torch.from_numpy(g).cuda())
        torch.cuda.synchronize()
        _check_append(case, d, q_ref, blocks, q_rotated=False)
        assert_attn_close(out, ref)
        np.testing.assert_allclose(to_f64(lse), rlse, rtol=0, atol=1e-4)
        assert torch.count_nonzero(ws[:4 * len(pos) * 2]).item() == 0


@pytest.mark.parametrize("pos,lmax,hq,hkv", [
    ([0, 17, 300, 2047], 2048, 8, 2), ([5, 700, 4095, 1100, 1], 4096, 8, 2),
    ([0, 900, 2047], 2048, 4, 4), ([3, 1500, 640], 2048, 8, 4),      # groups 1, 2
    ([0, 1300, 2047], 2048, 16, 2), ([7, 2000, 129], 2048, 32, 2),  # groups 8, 16
])
def test_fp8_full_step(pos, lmax, hq, hkv):
    """hda_decode_step on an fp8 full-layer cache (the streaming kernel's
    step form: the wave owning a pair's first round quantizes and appends
    the new row; the merge scores it, and for pos 0 -- no held rows --
    quantizes and appends it itself): the cache as the oracle's (one code
    step) and bit-identical to the two-call path's, out / lse within the
    decode tolerance, with sinks and the gate; contiguous and paged."""
    import full_kv_cache_amd as hda
    print("CASE fp8 full step", pos, hq, hkv, flush=True)
    case = Fp8Case(2400 + len(pos) + hq, FULL, pos, lmax, hq=hq, hkv=hkv)
    Hq = case.shape.num_q_heads
    sk = np.linspace(-1.0, 3.0, Hq).astype(np.float32)
    g = np.random.default_rng(8).uniform(-3, 3, size=(len(pos), Hq)).astype(np.float32)
    q_ref, blocks, ref, rlse = case.oracle_step(sinks=sk, gate=g)
    d2, _, _ = case.gpu_step(sinks=sk, gate=g)  # hda_rope_append + hda_decode_attn
    d = case.device()
    cache = case.cache(d)
    ws = torch.zeros(hda.hda_decode_step_workspace_bytes(cache, FULL), dtype=torch.uint8, device="cuda")
    out = torch.full((len(pos), Hq, 256), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((len(pos), Hq), float("nan"), device="cuda")
    hda.hda_decode_step(d["q"], d["k_new"], d["v_new"], torch.from_numpy(case.pos).cuda(), FULL,
                        cache, torch.from_numpy(sk).cuda(), 1 / 16, out, lse, ws,
                        gate=torch.from_numpy(g).cuda())
    torch.cuda.synchronize()
    _check_append(case, d, q_ref, blocks, q_rotated=False)
    for n in ("kc", "vc"):
        assert torch.equal(d[n], d2[n]), n
    for n in ("ks", "vs"):
        assert torch.equal(d[n].view(torch.int32), d2[n].view(torch.int32)), n
    assert_attn_close(out, ref)
    np.testing.assert_allclose(to_f64(lse), rlse, rtol=0, atol=1e-4)


def test_fp8_full_step_paged():
    """The fp8 full-layer step through a shuffled pool of 64-row pages: the
    same out / lse as on the contiguous cache, bit for bit, and the new rows
    in the pages the table names."""
    import full_kv_cache_amd as hda
    print("CASE fp8 full step paged", flush=True)
    ps = 64
    case = Fp8Case(2500, FULL, [0, 63, 64, 1500, 2047], 2048)
    Hq = case.shape.num_q_heads
    B, Hkv, cap, D = case.kc.shape
    mp = cap // ps
    perm = np.random.default_rng(10).permutation(B * mp + 3)

    def pool(a):
        out = np.zeros((B * mp + 3, Hkv, ps) + a.shape[3:], a.dtype)
        pages = a.reshape((B, Hkv, mp, ps) + a.shape[3:]).swapaxes(1, 2).reshape((B * mp, Hkv, ps) + a.shape[3:])
        out[perm[:B * mp]] = pages
        return torch.from_numpy(out).cuda()

    res = []
    for paged in (False, True):
        d = case.device()
        if paged:
            kp, vp, ksp, vsp = (pool(getattr(case, n)) for n in ("kc", "vc", "ks", "vs"))
            table = torch.from_numpy(perm[:B * mp].reshape(B, mp).astype(np.int32)).cuda()
            cache = case.cache(d, block_table=table, kc=kp, vc=vp, ks=ksp, vs=vsp)
        else:
            cache = case.cache(d)
        ws = torch.zeros(hda.hda_decode_step_workspace_bytes(cache, FULL), dtype=torch.uint8,
                         device="cuda")
        out = torch.empty((B, Hq, 256), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((B, Hq), device="cuda")
        hda.hda_decode_step(d["q"], d["k_new"], d["v_new"], torch.from_numpy(case.pos).cuda(), FULL,
                            cache, None, 1 / 16, out, lse, ws)
        torch.cuda.synchronize()
        res.append((out, lse))
        if paged:  # gather the pool back through the table: as the contiguous step left it
            for n, pl in (("kc", kp), ("ks", ksp)):
                back = pl[torch.from_numpy(perm[:B * mp]).cuda()].reshape((B, mp, Hkv, ps) + pl.shape[3:])
                back = back.transpose(1, 2).reshape((B, Hkv, cap) + pl.shape[3:])
                for b, p in enumerate(case.pos):
                    got, want = back[b, :, p].contiguous(), cont[n][b, :, p].contiguous()
                    assert torch.equal(got.view(torch.uint8), want.view(torch.uint8)), n
        else:
            cont = {"kc": d["kc"], "ks": d["ks"]}
    assert torch.equal(res[0][0].view(torch.int16), res[1][0].view(torch.int16))
    assert torch.equal(res[0][1], res[1][1])
