"""Pins for the oracle's paged-cache gather (CPU only).

flashmla_sparse page, `_fp8_flash_mla_kernel`: the attention call reads
the cache through a block table with per-sequence lengths.  Reading: row r
of sequence b is row r % page_size of pool page block_table[b][r / page_size].
Pinned by what that addressing fixes, not by restating it:
  * pages laid out in table order reproduce the contiguous blocks exactly
    (a swapped head/page order or page/offset split would not);
  * a marker row lands at exactly one (sequence, head, row);
  * element-by-element brute force on a tiny case;
  * relabelling the pool's pages (pool and table permuted together) changes
    nothing; a table entry outside the pool leaves its rows zero;
  * attention over a gathered paged cache equals attention over the same
    rows stored contiguously, bit for bit.
"""
import numpy as np
import pytest

import oracle
import workloads


def _paged_from_blocks(k, page_size):
    """Contiguous [B, Hkv, cap, D] -> (pool, table) with page b*max_pages + j
    holding rows j*page_size .. of sequence b."""
    B, Hkv, cap, D = k.shape
    mp = cap // page_size
    pool = np.ascontiguousarray(
        k.reshape(B, Hkv, mp, page_size, D).transpose(0, 2, 1, 3, 4).reshape(B * mp, Hkv,
                                                                             page_size, D))
    table = np.arange(B * mp, dtype=np.int32).reshape(B, mp)
    return pool, table


@pytest.mark.parametrize("page_size", [16, 32, 64])
def test_in_order_pages_are_identity(page_size):
    rng = np.random.default_rng(1)
    k = rng.integers(0, 1 << 16, size=(3, 2, 128, 8), dtype=np.uint16)
    pool, table = _paged_from_blocks(k, page_size)
    assert np.array_equal(oracle.page_gather(pool, table), k)


def test_marker_row_position():
    pool = np.zeros((7, 2, 16, 4), dtype=np.uint16)
    pool[5, 1, 3, :] = 7
    table = np.array([[2, 5], [0, 1]], dtype=np.int32)
    out = oracle.page_gather(pool, table)
    hit = np.argwhere(out != 0)
    # sequence 0, head 1, row 16 + 3 (second page of sequence 0, offset 3)
    assert {tuple(x[:3]) for x in hit} == {(0, 1, 19)}
    assert np.all(out[0, 1, 19] == 7)


def test_brute_force_tiny():
    rng = np.random.default_rng(2)
    P, Hkv, ps, D, B, mp = 5, 2, 16, 3, 2, 3
    pool = rng.integers(0, 1 << 16, size=(P, Hkv, ps, D), dtype=np.uint16)
    table = np.array([[4, 0, 2], [1, 1, 3]], dtype=np.int32)  # page 1 used twice
    out = oracle.page_gather(pool, table)
    for b in range(B):
        for h in range(Hkv):
            for r in range(mp * ps):
                page, off = table[b][r // ps], r % ps
                for d in range(D):
                    assert out[b, h, r, d] == pool[page, h, off, d]


def test_relabelled_pool_is_invariant():
    rng = np.random.default_rng(3)
    P, Hkv, ps, D = 9, 2, 32, 8
    pool = rng.integers(0, 1 << 16, size=(P, Hkv, ps, D), dtype=np.uint16)
    table = rng.permutation(P)[:8].astype(np.int32).reshape(2, 4)
    perm = rng.permutation(P)
    pool2 = np.empty_like(pool)
    pool2[perm] = pool
    table2 = perm[table].astype(np.int32)
    assert np.array_equal(oracle.page_gather(pool2, table2), oracle.page_gather(pool, table))


def test_out_of_pool_entry_reads_zero():
    pool = np.full((2, 1, 16, 4), 9, dtype=np.uint16)
    out = oracle.page_gather(pool, np.array([[1, -1, 2]], dtype=np.int32))
    assert np.all(out[0, 0, :16] == 9)
    assert np.all(out[0, 0, 16:] == 0)


def test_attention_over_paged_equals_contiguous():
    shape = workloads.HybridShape(batch=3, lmax=96)
    g = workloads.generator(4)
    t = {k: workloads.bits(v).copy()
         for k, v in workloads.layer_inputs(g, shape, workloads.FULL).items()}
    sinks = workloads.sinks(g, shape.num_q_heads).numpy()
    k, v = t["k"], t["v"]
    pool_k, table = _paged_from_blocks(k, 32)
    pool_v, _ = _paged_from_blocks(v, 32)
    # shuffle the pool so the gather has real work to do
    perm = np.random.default_rng(5).permutation(pool_k.shape[0])
    pk, pv = np.empty_like(pool_k), np.empty_like(pool_v)
    pk[perm], pv[perm] = pool_k, pool_v
    table = perm[table].astype(np.int32)
    seq = np.array([96, 49, 17], dtype=np.int32)
    args = dict(seq_lens=seq, layer_type=workloads.FULL, window=512, sinks=sinks,
                scale=0.0625)
    o1, l1 = oracle.decode_attn(t["q"], k, v, None, None, **args)
    o2, l2 = oracle.decode_attn(t["q"], oracle.page_gather(pk, table),
                                oracle.page_gather(pv, table), None, None, **args)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
