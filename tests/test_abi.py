"""The C-ABI library loads, exports every entry point of include/hda.h, and
rejects bad arguments on the host before touching a GPU (CPU only).

Error conventions follow the pages: the Spark export page's config checks
(`__post_init__`: query heads not a multiple of KV heads, unknown layer
types -> ValueError) and the flashmla_sparse page's sink checks
(`_validate_sinks`, `_sinks_for_query`: fp32, shape (num_heads,), same
device).  No call here reaches a kernel launch.
"""
import ctypes
import os
import re
import subprocess

import pytest
import torch

import full_kv_cache_amd as hda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "hda.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hda_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert {"hda_rope_append", "hda_decode_attn", "hda_decode_workspace_bytes",
            "hda_status_string", "hda_last_error_message"} <= set(names)
    out = subprocess.check_output(["nm", "-D", "--defined-only", str(hda.LIB_PATH)], text=True)
    exported = {l.split()[-1] for l in out.splitlines() if l.strip()}
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    L = hda.lib()
    for n in names:
        assert hasattr(L, n)


def test_status_strings():
    L = hda.lib()
    for code, name in [(0, b"HDA_OK"), (1, b"HDA_ERR_INVALID_ARGUMENT"),
                       (2, b"HDA_ERR_UNSUPPORTED"), (3, b"HDA_ERR_WORKSPACE"), (4, b"HDA_ERR_HIP")]:
        assert L.hda_status_string(code) == name


FAKE = 0x10000  # aligned, never dereferenced: every call below fails validation


def _desc(**kw):
    d = dict(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=256, window=512, rotary_dim=256,
             capacity=512, rope_theta=1e4, k=FAKE, v=FAKE)
    d.update(kw)
    return hda.CacheDesc(**d)


def _decode(desc, layer=hda.SLIDING, max_seq_len=512, chunk=0, q=FAKE, out=FAKE, ws=None, wsb=0,
            scale=0.0625):
    L = hda.lib()
    return L.hda_decode_attn(ctypes.c_void_p(q), ctypes.byref(desc), ctypes.c_void_p(FAKE), layer,
                             None, None, scale, ctypes.c_void_p(out), None, max_seq_len, chunk,
                             ctypes.c_void_p(ws) if ws else None, wsb, None)


def _append(desc, layer=hda.SLIDING, q=FAKE):
    L = hda.lib()
    return L.hda_rope_append(ctypes.c_void_p(q), ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE),
                             ctypes.c_void_p(FAKE), layer, ctypes.byref(desc), None)


def _msg():
    return hda.lib().hda_last_error_message().decode()


@pytest.mark.parametrize("fn", [_append, _decode])
def test_heads_not_multiple(fn):
    assert fn(_desc(num_q_heads=6, num_kv_heads=4)) == 1
    assert "not a multiple" in _msg()


@pytest.mark.parametrize("fn", [_append, _decode])
def test_unknown_layer_type(fn):
    assert fn(_desc(), layer=2) == 1
    assert "unknown layer type" in _msg()


def test_rotary_dim_checks():
    assert _append(_desc(rotary_dim=255)) == 1
    assert _append(_desc(rotary_dim=258)) == 1


def test_sliding_capacity_must_be_window():
    assert _append(_desc(capacity=511)) == 1
    assert "must equal window" in _msg()


def test_rotary_dim_granularity_unsupported():
    assert _append(_desc(rotary_dim=24)) == 2


def test_null_and_misaligned_pointers():
    assert _append(_desc(), q=0) == 1
    assert _append(_desc(k=FAKE + 2)) == 1
    assert _decode(_desc(), q=FAKE + 8) == 1


def test_decode_unsupported_shapes():
    assert _decode(_desc(head_dim=128, rotary_dim=128)) == 2
    assert _decode(_desc(num_q_heads=6, num_kv_heads=2)) == 2  # group of 3
    tiny = _desc(capacity=8, rotary_dim=64, rope_theta=5e6)
    assert _decode(tiny, layer=hda.FULL, max_seq_len=8) == 2  # fewer than 16 rows


def test_decode_bounds():
    full = _desc(capacity=1024, rotary_dim=64, rope_theta=5e6)
    assert _decode(full, layer=hda.FULL, max_seq_len=1025) == 1
    assert "capacity" in _msg()
    assert _decode(full, layer=hda.FULL, max_seq_len=0) == 1
    assert _decode(full, layer=hda.FULL, max_seq_len=64, chunk=24) == 1
    assert _decode(full, layer=hda.FULL, max_seq_len=64, chunk=1024) == 1
    assert _decode(full, layer=hda.FULL, max_seq_len=64, scale=float("nan")) == 1


def test_workspace_sizing_and_errors():
    L = hda.lib()
    full = _desc(capacity=4096, rotary_dim=64, rope_theta=5e6)
    need = L.hda_decode_workspace_bytes(ctypes.byref(full), hda.FULL, 4096, 256)
    # a 256-byte header (one counter per sequence x KV head, rounded up), then
    # 2 sequences x 8 heads x 16 chunks of (256 floats out + 1 float lse)
    assert need == 256 + (2 * 8 * 16 * 256 * 4) + 2 * 8 * 16 * 4
    assert _decode(full, layer=hda.FULL, max_seq_len=4096, chunk=256) == 3
    assert _decode(full, layer=hda.FULL, max_seq_len=4096, chunk=256, ws=FAKE, wsb=need - 1) == 3
    assert "workspace" in _msg()
    # one chunk covering every key needs no workspace
    assert L.hda_decode_workspace_bytes(ctypes.byref(full), hda.FULL, 512, 512) == 0
    # invalid description -> 0
    bad = _desc(num_q_heads=6, num_kv_heads=4)
    assert L.hda_decode_workspace_bytes(ctypes.byref(bad), hda.SLIDING, 512, 0) == 0


def test_batch_zero_is_noop():
    assert _append(_desc(batch=0)) == 0
    assert _decode(_desc(batch=0)) == 0


def test_sink_validation_in_binding():
    q = torch.zeros(2, 8, 256, dtype=torch.bfloat16)
    hda.validate_sinks(None, q)
    hda.validate_sinks(torch.zeros(8), q)
    with pytest.raises(ValueError, match="float32"):
        hda.validate_sinks(torch.zeros(8, dtype=torch.float16), q)
    with pytest.raises(ValueError, match="shape"):
        hda.validate_sinks(torch.zeros(4), q)
    with pytest.raises(ValueError, match="shape"):
        hda.validate_sinks(torch.zeros(8, 1), q)


# ------------------------------------------------------------- sparse entry
def _sparse(tokens=32, heads=64, topk=2048, dqk=576, dv=512, pool=32768, q=FAKE, kv=FAKE,
            idx=FAKE, out=FAKE, ws=None, wsb=0, scale=1 / 24):
    L = hda.lib()
    return L.hda_sparse_decode_attn(ctypes.c_void_p(q), ctypes.c_void_p(kv), pool,
                                    ctypes.c_void_p(idx), tokens, topk, None, heads, dqk, dv, None,
                                    scale, ctypes.c_void_p(out), None,
                                    ctypes.c_void_p(ws) if ws else None, wsb, None)


def test_sparse_shape_checks():
    assert _sparse(heads=24) == 1 and "multiple of 16" in _msg()
    assert _sparse(heads=0) == 1
    assert _sparse(tokens=-1) == 1
    assert _sparse(topk=-5) == 1
    assert _sparse(dqk=512) == 2 and "576" in _msg()
    assert _sparse(dv=256) == 2
    assert _sparse(pool=0) == 1 and "pool_rows" in _msg()
    assert _sparse(q=0) == 1
    assert _sparse(out=FAKE + 8) == 1 and "aligned" in _msg()
    assert _sparse(idx=FAKE + 2) == 1


def test_sparse_workspace_plan():
    """Split only when the workgroups would leave the GPU short (fewer than
    256): one per token for a bf16 pool and up to 64 heads (the shared-tile
    kernel), one per (token, 16 heads) otherwise; the size covers either
    pool.  The headline shape (32 tokens, 64 heads, top-2048) splits in
    eight for the bf16 pool: partials fp32 [32, 64, 8, 512] plus lse
    [32, 64, 8]."""
    ws = hda.hda_sparse_workspace_bytes
    assert ws(32, 64, 2048) == 32 * 64 * 8 * 512 * 4 + 32 * 64 * 8 * 4
    assert ws(128, 64, 2048) == 128 * 64 * 2 * 512 * 4 + 128 * 64 * 2 * 4  # bf16: 2 splits; fp8: none
    assert ws(256, 64, 2048) == 0       # 256 workgroups already: no split
    assert ws(256, 16, 4096) == 256 * 16 * 2 * 512 * 4 + 256 * 16 * 2 * 4  # splits of at most 2048 keys
    assert ws(1, 16, 64) == 0           # too few keys to split
    assert ws(1, 16, 2048) == 1 * 16 * 32 * 512 * 4 + 16 * 32 * 4  # 32 splits of 64 keys
    assert ws(32, 64, 2048, dv=256) == 0  # invalid shape
    need = ws(32, 64, 2048)
    assert _sparse() == 3 and "workspace" in _msg()
    assert _sparse(ws=FAKE, wsb=need - 1) == 3
    assert _sparse(ws=FAKE + 4, wsb=need) == 1 and "aligned" in _msg()
    assert _sparse(tokens=0) == 0       # no tokens: nothing to do, nothing needed


def test_sparse_sink_validation_in_binding():
    q = torch.zeros(2, 16, 576, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="float32"):
        hda.hda_sparse_decode_attn(q, None, None, None, torch.zeros(16, dtype=torch.float64), 1.0, None)
    with pytest.raises(ValueError, match="shape"):
        hda.hda_sparse_decode_attn(q, None, None, None, torch.zeros(8), 1.0, None)


# -------------------------------------------------------- fused step entry
def _step(desc, layer=hda.SLIDING, q=FAKE, ws=None, wsb=0, scale=0.0625):
    L = hda.lib()
    return L.hda_decode_step(ctypes.c_void_p(q), ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE),
                             ctypes.c_void_p(FAKE), layer, ctypes.byref(desc), None, None, scale,
                             ctypes.c_void_p(FAKE), None, ctypes.c_void_p(ws) if ws else None, wsb,
                             None)


def test_step_shape_checks():
    assert _step(_desc(num_q_heads=6, num_kv_heads=4)) == 1
    assert _step(_desc(), layer=7) == 1
    assert _step(_desc(capacity=1024)) == 1 and "must equal window" in _msg()
    assert _step(_desc(rotary_dim=128)) == 2 and "rotary_dim" in _msg()
    assert _step(_desc(head_dim=128, rotary_dim=64)) == 2
    assert _step(_desc(batch=5000)) == 2
    assert _step(_desc(), q=0) == 1
    assert _step(_desc(), q=FAKE + 8) == 1 and "aligned" in _msg()


def test_step_workspace():
    """Counter header first (shared with hda_decode_attn's layouts); the
    window form (sliding layers) adds, for a key split over S workgroups, a
    partial (o fp32 [G, 256], lse fp32 [G]) per workgroup; the streaming
    form (full layers) adds one partial slot per wave and per (sequence,
    KV head), and one new-key score per (sequence, query head)."""
    L = hda.lib()
    d = _desc()
    need = L.hda_decode_step_workspace_bytes(ctypes.byref(d), hda.SLIDING)
    # 2 sequences x 2 KV heads: 4 pairs, too few for 256 workgroups, so a
    # 512-key window splits 8 ways (4 rounds each); group 4
    pairs, S, G = 4, 8, 4
    assert need == 256 + pairs * S * G * 256 * 4 + 512
    full = _desc(capacity=4096, rotary_dim=64, rope_theta=5e6)
    need_full = L.hda_decode_step_workspace_bytes(ctypes.byref(full), hda.FULL)
    assert need_full > 256 and need_full % 256 == 0
    assert _step(d) == 3 and "workspace" in _msg()
    assert _step(d, ws=FAKE, wsb=need - 1) == 3
    assert _step(d, ws=FAKE + 4, wsb=need) == 1
    assert L.hda_decode_step_workspace_bytes(ctypes.byref(_desc(rotary_dim=128)), hda.SLIDING) == 0
    assert _step(_desc(batch=0), ws=FAKE, wsb=need) == 0  # nothing to do


# ------------------------------------------------------------ output gate
def test_gate_pointer_alignment():
    """A misaligned gate pointer is refused before anything is enqueued."""
    L = hda.lib()
    r = L.hda_decode_attn(ctypes.c_void_p(FAKE), ctypes.byref(_desc()), ctypes.c_void_p(FAKE),
                          hda.SLIDING, None, ctypes.c_void_p(FAKE + 2), 0.0625, ctypes.c_void_p(FAKE),
                          None, 512, 0, None, 0, None)
    assert r == 1 and "gate" in _msg()
    r = L.hda_lse_merge(ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), 2, 8, 2, 256, None,
                        ctypes.c_void_p(FAKE + 1), ctypes.c_void_p(FAKE), None, None)
    assert r == 1 and "gate" in _msg()
    r = L.hda_decode_step(ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE),
                          ctypes.c_void_p(FAKE), hda.SLIDING, ctypes.byref(_desc()), None,
                          ctypes.c_void_p(FAKE + 2), 0.0625, ctypes.c_void_p(FAKE), None, None, 0,
                          None)
    assert r == 1 and "gate" in _msg()


def test_gate_binding_checks():
    """The binding checks the gate's dtype, shape and device like the sinks'."""
    q = torch.zeros(2, 8, 256, dtype=torch.bfloat16)
    out = torch.zeros(2, 8, 256, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="dtype"):
        hda.validate_gate(torch.zeros(2, 8, dtype=torch.float16), out)
    with pytest.raises(ValueError, match="shape"):
        hda.validate_gate(torch.zeros(8, dtype=torch.float32), out)
    with pytest.raises(ValueError, match="contiguous"):
        hda.validate_gate(torch.zeros(8, 2, dtype=torch.float32).t(), out)
    hda.validate_gate(torch.zeros(2, 8, dtype=torch.float32), out)
    hda.validate_gate(None, q)


# ------------------------------------------------------------- paged cache
_PAGED = dict(capacity=1024, rotary_dim=64, rope_theta=5e6, block_table=FAKE, page_size=64,
              max_pages=16, num_pages=40)


def test_paged_descriptor_checks():
    """The paged layout is refused on sliding layers and checked for a
    page size that keeps each 16-key round inside one page, a capacity of
    max_pages * page_size, and an aligned table."""
    assert _append(_desc(block_table=FAKE, page_size=64, max_pages=8, num_pages=8)) == 2
    assert "full layers" in _msg()
    for bad in (dict(page_size=24), dict(page_size=0), dict(page_size=-16),
                dict(max_pages=0, capacity=0), dict(num_pages=0), dict(capacity=1040),
                dict(block_table=FAKE + 2)):
        d = _desc(**{**_PAGED, **bad})
        assert _append(d, layer=hda.FULL) == 1, bad
        assert _decode(d, layer=hda.FULL, max_seq_len=16) == 1, bad


def test_paged_routing():
    """A paged cache is read only by the streaming kernel: split-K chunks,
    the partials stage and batches above the streaming limit are refused
    before anything is enqueued; the full-layer step (the streaming
    kernel's step form) takes it, with the streaming path's workspace."""
    L = hda.lib()
    d = _desc(**_PAGED)
    assert _decode(d, layer=hda.FULL, max_seq_len=1024, chunk=256) == 2
    assert "paged" in _msg()
    big = _desc(**{**_PAGED, "batch": 5000})
    assert _decode(big, layer=hda.FULL, max_seq_len=1024) == 2
    r = L.hda_decode_attn_partials(ctypes.c_void_p(FAKE), ctypes.byref(d), ctypes.c_void_p(FAKE),
                                   hda.FULL, 0.0625, 1024, 256, ctypes.c_void_p(FAKE),
                                   ctypes.c_void_p(FAKE), None)
    assert r == 2 and "contiguous" in _msg()
    assert _step(d, layer=hda.FULL) == 3 and "workspace" in _msg()
    # the streaming path's workspace, then one score per (sequence, query head)
    assert L.hda_decode_step_workspace_bytes(ctypes.byref(d), hda.FULL) == \
        L.hda_decode_workspace_bytes(ctypes.byref(d), hda.FULL, 1024, 0) + 256 > 256
    assert _decode(_desc(**{**_PAGED, "batch": 0}), layer=hda.FULL, max_seq_len=16) == 0


def test_paged_binding_desc():
    """LayerCache with a block table describes the pool and the table."""
    import torch
    pool = torch.zeros(12, 2, 32, 256, dtype=torch.bfloat16)
    table = torch.arange(12, dtype=torch.int32).reshape(3, 4)
    c = hda.LayerCache(pool, pool, 8, 512, 64, 5e6, block_table=table).desc()
    assert (c.batch, c.num_kv_heads, c.capacity, c.page_size, c.max_pages, c.num_pages) == \
        (3, 2, 128, 32, 4, 12)
    assert c.block_table == table.data_ptr()
    with pytest.raises(ValueError):
        hda.LayerCache(pool, pool, 8, 512, 64, 5e6, block_table=table.long()).desc()


# ---------------------------------------------------------------- fp8 cache
_FP8 = dict(kv_dtype=1, k_scale=FAKE, v_scale=FAKE)


def test_fp8_descriptor_checks():
    """An fp8 cache needs both scale arrays, 4-byte aligned, and head_dim 256;
    an unknown element type is refused."""
    assert _append(_desc(kv_dtype=2)) == 1 and "kv_dtype" in _msg()
    assert _append(_desc(kv_dtype=1)) == 1 and "scale" in _msg()
    assert _append(_desc(kv_dtype=1, k_scale=FAKE)) == 1
    assert _append(_desc(**{**_FP8, "v_scale": FAKE + 2})) == 1 and "aligned" in _msg()
    assert _append(_desc(**{**_FP8, "head_dim": 128, "rotary_dim": 128})) == 2


def test_fp8_routing():
    """The fp8 cache is read by the window and streaming kernels only: the
    full-layer step (streaming step form) takes it, a sliding window past
    one workgroup's 1024 keys does not."""
    L = hda.lib()
    full = _desc(**{**_FP8, "capacity": 4096, "rotary_dim": 64, "rope_theta": 5e6})
    assert _decode(full, layer=hda.FULL, max_seq_len=4096, chunk=256) == 2 and "fp8" in _msg()
    assert _step(full, layer=hda.FULL) == 3 and "workspace" in _msg()
    assert L.hda_decode_step_workspace_bytes(ctypes.byref(full), hda.FULL) > 0
    wide = _desc(**{**_FP8, "window": 2048, "capacity": 2048})
    assert _step(wide) == 2 and "fp8" in _msg()
    assert L.hda_decode_step_workspace_bytes(ctypes.byref(wide), hda.SLIDING) == 0
    # the window form takes an fp8 cache: the same workspace as on bf16
    assert L.hda_decode_step_workspace_bytes(ctypes.byref(_desc(**_FP8)), hda.SLIDING) == \
        L.hda_decode_step_workspace_bytes(ctypes.byref(_desc()), hda.SLIDING)
    r = L.hda_decode_attn_partials(ctypes.c_void_p(FAKE), ctypes.byref(full), ctypes.c_void_p(FAKE),
                                   hda.FULL, 0.0625, 4096, 256, ctypes.c_void_p(FAKE),
                                   ctypes.c_void_p(FAKE), None)
    assert r == 2 and "bf16" in _msg()


def test_fp8_binding_desc():
    import torch
    codes = torch.zeros(2, 2, 512, 256, dtype=torch.uint8)
    sc = torch.zeros(2, 2, 512, dtype=torch.float32)
    c = hda.LayerCache(codes, codes, 8, 512, 256, 1e4, k_scale=sc, v_scale=sc).desc()
    assert c.kv_dtype == 1 and c.k_scale == sc.data_ptr() and c.v_scale == sc.data_ptr()
    assert hda.LayerCache(torch.zeros(2, 2, 512, 256, dtype=torch.bfloat16),
                          torch.zeros(2, 2, 512, 256, dtype=torch.bfloat16), 8, 512, 256,
                          1e4).desc().kv_dtype == 0
    with pytest.raises(ValueError):
        hda.LayerCache(codes, codes, 8, 512, 256, 1e4).desc()  # scales missing
    with pytest.raises(ValueError):
        hda.LayerCache(codes, codes, 8, 512, 256, 1e4, k_scale=sc[:, :, :10],
                       v_scale=sc).desc()


# ------------------------------------------------------------- chunk decode
def _multi(desc, tokens=2, layer=hda.SLIDING, q=FAKE, pos=FAKE, scale=0.0625, msl=16, ws=None,
           wsb=0):
    L = hda.lib()
    return L.hda_decode_multi(ctypes.c_void_p(q), ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE),
                              ctypes.c_void_p(pos), tokens, layer, ctypes.byref(desc), None, None,
                              scale, ctypes.c_void_p(FAKE), None, msl,
                              ctypes.c_void_p(ws) if ws else None, wsb, None)


def test_multi_checks():
    """Chunk decode: 1..512 tokens, a cache of at least 16 rows (32 for
    chunks of more than 16 query rows per KV head), contiguous bf16 caches,
    the usual pointer and shape checks."""
    assert _multi(_desc(), tokens=0) == 2 and "tokens" in _msg()
    assert _multi(_desc(), tokens=513) == 2 and "512" in _msg()
    assert _multi(_desc(), tokens=512) == 3  # accepted: only the workspace is missing
    tiny = _desc(capacity=16, rotary_dim=64, rope_theta=5e6)
    assert _multi(tiny, layer=hda.FULL, tokens=4, msl=16) == 3
    assert _multi(tiny, layer=hda.FULL, tokens=5, msl=16) == 2 and "32 rows" in _msg()
    assert _multi(_desc(), q=0) == 1
    assert _multi(_desc(), pos=FAKE + 2) == 1 and "aligned" in _msg()
    assert _multi(_desc(), scale=0.0) == 1
    assert _multi(_desc(head_dim=128, rotary_dim=128)) == 2
    assert _multi(_desc(rotary_dim=24)) == 2
    assert _multi(_desc(**_FP8)) == 2 and "bf16" in _msg()
    assert _multi(_desc(**{**_PAGED, "rotary_dim": 64}), layer=hda.FULL) == 2
    assert _multi(_desc(batch=0)) == 0
    assert _multi(_desc(), msl=0) == 1


def test_multi_workspace():
    """The workspace holds the rotated new K rows (bf16 [B, T, Hkv, D]);
    long contexts also split each pair's keys over several workgroups, whose
    partials (fp32 out + lse per query row) follow.  Prefill-sized chunks
    (more than 16 query rows per KV head) split their key tiles (up to 4
    ranges, at least 8 tiles of 32 keys each) while the row blocks leave
    fewer than 256 workgroups."""
    L = hda.lib()
    full = _desc(capacity=4096, rotary_dim=64, rope_theta=5e6)
    krot = lambda T: (2 * T * 2 * 256 * 2 + 255) // 256 * 256
    assert L.hda_decode_multi_workspace_bytes(ctypes.byref(full), hda.FULL, 2, 20) == krot(2)
    need = L.hda_decode_multi_workspace_bytes(ctypes.byref(full), hda.FULL, 2, 4096)
    # 4 pairs: 128 / 4 = 32 workgroups wanted and 256 rounds allow 32 (8 rounds each);
    # partial rows = pairs x 32 x (2 tokens x 4 heads)
    rows = 2 * 2 * 32 * 2 * 4
    assert need == krot(2) + (rows * 256 * 4 + 255) // 256 * 256 + rows * 4
    assert _multi(full, layer=hda.FULL, msl=4096) == 3 and "workspace" in _msg()
    assert _multi(full, layer=hda.FULL, msl=4096, ws=FAKE, wsb=need - 1) == 3
    assert _multi(full, layer=hda.FULL, msl=4096, ws=FAKE + 4, wsb=need) == 1
    # 5 tokens x 4 heads: one 128-row block per pair, 4 pairs, 128 key tiles:
    # 4 ranges; partial rows = pairs x 4 x 20
    prows = 2 * 2 * 4 * 5 * 4
    assert L.hda_decode_multi_workspace_bytes(ctypes.byref(full), hda.FULL, 5, 4096) == \
        krot(5) + (prows * 256 * 4 + 255) // 256 * 256 + prows * 4
    assert L.hda_decode_multi_workspace_bytes(ctypes.byref(full), hda.FULL, 5, 200) == krot(5)  # 7 tiles
    # sliding window, 64 sequences (128 pairs): one token keeps one workgroup
    # per pair (no partials); from two tokens on the 511 held keys (32
    # rounds) split in 2 (256 workgroups, 16 rounds each)
    slide = _desc(batch=64)
    krot64 = lambda T: (64 * T * 2 * 256 * 2 + 255) // 256 * 256
    assert L.hda_decode_multi_workspace_bytes(ctypes.byref(slide), hda.SLIDING, 1, 4096) == krot64(1)
    srows = 64 * 2 * 2 * 4 * 4  # pairs x 2 parts x (4 tokens x 4 heads)
    assert L.hda_decode_multi_workspace_bytes(ctypes.byref(slide), hda.SLIDING, 4, 4096) == \
        krot64(4) + (srows * 256 * 4 + 255) // 256 * 256 + srows * 4
