"""GPU parity of the paged full-layer cache (flashmla_sparse page,
`_fp8_flash_mla_kernel`: the cache is read through a block table with
per-sequence lengths).

The contiguous case's blocks are cut into pages, the pages shuffled into a
larger pool whose spare pages hold NaN, and each sequence's table names its
pages; table entries past a sequence's last page point outside the pool
(the kernels clamp and never read them).  Checked against the fp64 oracle:
  * hda_rope_append writes row pos into the page its table names: the pool,
    gathered back through the table, equals the oracle's cache bit for bit
    on every row the sequence holds, and no spare page changes;
  * hda_decode_attn (streaming kernel + merge) is within the decode
    tolerance of the oracle, and bit-identical to the same step on the
    contiguous cache (the same rounds are summed in the same order);
  * page sizes 16, 64 and 256, lengths 1, a page boundary on either side,
    ragged mixes, with sinks and the output gate.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from hybrid_case import BF16_NAN, FULL, HybridCase, assert_attn_close, bits_of, to_f64

pytestmark = pytest.mark.gpu


def _page(case, page_size, spare=5, seed=0):
    """(pool_k, pool_v, table, spare_ids) from the case's contiguous host
    blocks; pages shuffled, `spare` extra NaN pages."""
    k, v = case.host["k"], case.host["v"]
    B, Hkv, cap, D = k.shape
    mp = cap // page_size
    n = B * mp + spare
    rng = np.random.default_rng(seed)
    perm = rng.permutation(n)
    pk = np.full((n, Hkv, page_size, D), BF16_NAN, dtype=np.uint16)
    pv = pk.copy()
    table = np.empty((B, mp), dtype=np.int32)
    for b in range(B):
        used = -(-int(case.seq_lens[b]) // page_size)
        for j in range(mp):
            pg = perm[b * mp + j]
            pk[pg] = k[b, :, j * page_size:(j + 1) * page_size]
            pv[pg] = v[b, :, j * page_size:(j + 1) * page_size]
            table[b, j] = pg if j < used else n + 1000 + j  # never read
    return pk, pv, table, perm[B * mp:]


def _run(case, page_size, sinks=None, gate=None, seed=0):
    import full_kv_cache_amd as hda
    s = case.shape
    pk, pv, table, spare = _page(case, page_size, seed=seed)
    d = case.device()
    pool_k = workloads.from_bits(pk).cuda()
    pool_v = workloads.from_bits(pv).cuda()
    bt = torch.from_numpy(table).cuda()
    cache = hda.LayerCache(pool_k, pool_v, s.num_q_heads, s.window, s.rot(FULL), s.theta(FULL),
                           block_table=bt)
    pos = torch.from_numpy(case.pos).cuda()
    seq = torch.from_numpy(case.seq_lens).cuda()
    hda.hda_rope_append(d["q"], d["k_new"], d["v_new"], pos, FULL, cache)
    msl = int(case.seq_lens.max())
    nbytes = hda.hda_decode_workspace_bytes(cache, FULL, msl, 0)
    ws = torch.zeros(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    out = torch.full((s.batch, s.num_q_heads, s.head_dim), float("nan"), dtype=torch.bfloat16,
                     device="cuda")
    lse = torch.full((s.batch, s.num_q_heads), float("nan"), device="cuda")
    sk = None if sinks is None else torch.as_tensor(sinks).cuda()
    gt = None if gate is None else torch.as_tensor(gate).cuda()
    hda.hda_decode_attn(d["q"], cache, seq, FULL, sk, 1 / 16, out, lse, msl, 0, ws, gate=gt)
    torch.cuda.synchronize()
    return pool_k, pool_v, table, spare, pk, pv, out, lse


@pytest.mark.parametrize("page_size,pos", [
    (16, [0, 15, 16, 300, 2047]),
    (64, [63, 64, 1100, 5, 1000]),
    (256, [255, 256, 1, 1700, 1023]),
])
def test_paged_append_and_attention(page_size, pos):
    print("CASE paged", page_size, pos, flush=True)
    # the longest sequence exceeds 1024 keys, so the contiguous step below
    # takes the streaming kernel as well
    case = HybridCase(1500 + page_size, len(pos), FULL, pos, lmax=2048, poison=True)
    Hq = case.shape.num_q_heads
    sk = np.linspace(-1.0, 3.0, Hq).astype(np.float32)
    g = np.random.default_rng(page_size).uniform(-3, 3, size=(len(pos), Hq)).astype(np.float32)
    h, ref, rlse = case.oracle_step(sinks=sk, gate=g)
    pool_k, pool_v, table, spare, pk0, pv0, out, lse = _run(case, page_size, sk, g)

    # the append: gathered pool == oracle cache on every held row, spare
    # pages untouched
    gk = oracle.page_gather(bits_of(pool_k), table)
    gv = oracle.page_gather(bits_of(pool_v), table)
    for b, n in enumerate(case.seq_lens):
        assert np.array_equal(gk[b, :, :n], h["k"][b, :, :n]), b
        assert np.array_equal(gv[b, :, :n], h["v"][b, :, :n]), b
    assert np.array_equal(bits_of(pool_k)[spare], pk0[spare])
    assert np.array_equal(bits_of(pool_v)[spare], pv0[spare])

    assert_attn_close(out, ref)
    np.testing.assert_allclose(to_f64(lse), rlse, rtol=0, atol=1e-4)

    # the same step on the contiguous cache sums the same rounds in the
    # same order: bit-identical
    _, out_c, lse_c = case.gpu_step(sinks=sk, gate=g)
    assert torch.equal(out.view(torch.int16), out_c.view(torch.int16))
    assert torch.equal(lse, lse_c)


def test_paged_shared_prefix_pages():
    """Sequence 1's table names sequence 0's first four pages instead of
    its own: sequence 0's output is unchanged bit for bit, and sequence 1
    matches the oracle over the shared rows."""
    import full_kv_cache_amd as hda
    print("CASE paged shared prefix", flush=True)
    ps, B = 64, 2
    case = HybridCase(1600, B, FULL, [400, 400], lmax=512)
    s = case.shape
    pk, pv, table, _ = _page(case, ps, spare=0, seed=3)
    # sequence 1 reuses sequence 0's first 4 pages (rows 0..255)
    table_shared = table.copy()
    table_shared[1, :4] = table[0, :4]
    seq = torch.from_numpy(case.seq_lens).cuda()
    q = workloads.from_bits(case.host["q"]).cuda()
    res = []
    for t in (table, table_shared):
        pool_k = workloads.from_bits(pk).cuda()
        pool_v = workloads.from_bits(pv).cuda()
        cache = hda.LayerCache(pool_k, pool_v, s.num_q_heads, s.window, s.rot(FULL),
                               s.theta(FULL), block_table=torch.from_numpy(t).cuda())
        ws = torch.zeros(max(hda.hda_decode_workspace_bytes(cache, FULL, 401, 0), 1),
                         dtype=torch.uint8, device="cuda")
        out = torch.empty((B, s.num_q_heads, s.head_dim), dtype=torch.bfloat16, device="cuda")
        hda.hda_decode_attn(q, cache, seq, FULL, None, 1 / 16, out, None, 401, 0, ws)
        torch.cuda.synchronize()
        res.append(out)
    # sequence 0 is unchanged; sequence 1 now reads sequence 0's prefix
    assert torch.equal(res[0][0].view(torch.int16), res[1][0].view(torch.int16))
    k2, v2 = case.host["k"].copy(), case.host["v"].copy()
    k2[1, :, :256], v2[1, :, :256] = k2[0, :, :256], v2[0, :, :256]
    z = np.zeros((B, s.num_kv_heads, s.head_dim), np.uint16)
    ref, _ = oracle.decode_attn(case.host["q"], k2, v2, z, z, case.seq_lens, FULL, s.window,
                                None, 1 / 16)
    assert_attn_close(res[1], ref)
