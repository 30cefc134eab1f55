"""GPU parity of the hybrid decode path against the CPU oracle (MI355X).

Every case runs the same seeded inputs through libhda (C ABI, gfx950
kernels) and through the fp64 oracle, then compares:
  * cache placement, eviction and pass-through dims: bit-exact;
  * rotated q / new-K values: within one bf16 ulp, < 0.1% of them off;
  * attention out: max-abs <= 1e-2 and mean-abs <= 1e-3 (unit-normal
    bf16 inputs, fp32 accumulation); lse within 1e-4.
Sizes span several 16-key tiles, several chunks and ragged tails; rows the
step must not read are NaN-poisoned.
"""
import numpy as np
import pytest
import torch

from hybrid_case import (FULL, SLIDING, HybridCase, assert_attn_close, assert_rotated_close,
                         bits_of, near_lse_sinks, to_f64)

pytestmark = pytest.mark.gpu


def _print_case(**kw):
    print("CASE", " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


def _check_append(case, d):
    """Cache and q after hda_rope_append vs the oracle's append."""
    h, _, _ = case.oracle_step()
    assert np.array_equal(bits_of(d["v"]), h["v"])
    for name in ("k", "q"):
        assert_rotated_close(bits_of(d[name]), h[name])
    rot = case.shape.rot(case.lt)
    assert np.array_equal(bits_of(d["q"])[..., rot:], case.host["q"][..., rot:])


@pytest.mark.parametrize("pos", [[0, 1, 7], [509, 510, 511], [512, 1023, 4095], [32767, 600, 2]])
def test_rope_append_sliding(pos):
    _print_case(test="rope_append_sliding", pos=pos)
    import full_kv_cache_amd as hda
    case = HybridCase(100 + pos[0], 3, SLIDING, pos)
    d = case.device()
    hda.hda_rope_append(d["q"], d["k_new"], d["v_new"], torch.tensor(pos, dtype=torch.int32).cuda(),
                        SLIDING, case.cache(d))
    torch.cuda.synchronize()
    _check_append(case, d)


@pytest.mark.parametrize("pos", [[0, 5, 1023], [4095, 17, 2048]])
def test_rope_append_full(pos):
    _print_case(test="rope_append_full", pos=pos)
    import full_kv_cache_amd as hda
    case = HybridCase(200 + pos[0], 3, FULL, pos, lmax=4096)
    d = case.device()
    hda.hda_rope_append(d["q"], d["k_new"], d["v_new"], torch.tensor(pos, dtype=torch.int32).cuda(),
                        FULL, case.cache(d))
    torch.cuda.synchronize()
    _check_append(case, d)


@pytest.mark.parametrize("lt", [SLIDING, FULL])
def test_tiny_config(lt):
    """One sequence at position 1023: one sliding and one full layer, no sink."""
    _print_case(test="tiny", lt=lt)
    case = HybridCase(0, 1, lt, [1023], lmax=1024, poison=True)
    _, ref, rlse = case.oracle_step()
    _, out, lse = case.gpu_step()
    assert_attn_close(out, ref)
    np.testing.assert_allclose(to_f64(lse), rlse, rtol=0, atol=1e-4)


@pytest.mark.parametrize("pos", [0, 1, 7, 15, 16, 17, 509, 510, 511, 512, 1000])
def test_sliding_edge_positions(pos):
    _print_case(test="sliding_edge", pos=pos)
    case = HybridCase(300 + pos, 2, SLIDING, [pos, max(0, pos - 3)], poison=True)
    _, ref, rlse = case.oracle_step()
    for chunk in (0, 16, 48, 512):
        _, out, lse = case.gpu_step(chunk_keys=chunk)
        assert_attn_close(out, ref)
        np.testing.assert_allclose(to_f64(lse), rlse, rtol=0, atol=1e-4)
    if pos == 0:  # a single key: out is the new value
        assert np.array_equal(bits_of(out)[0], np.repeat(case.host["v_new"][0], 4, axis=0))


@pytest.mark.parametrize("chunk", [0, 16, 64, 112, 256, 512])
def test_full_chunks_ragged(chunk):
    """Full layer over lengths that leave ragged tiles and chunks."""
    pos = [0, 15, 16, 999, 2047, 3000]
    _print_case(test="full_chunks", chunk=chunk, pos=pos)
    case = HybridCase(400, len(pos), FULL, pos, lmax=3072, poison=True)
    _, ref, rlse = case.oracle_step()
    _, out, lse = case.gpu_step(chunk_keys=chunk)
    assert_attn_close(out, ref)
    np.testing.assert_allclose(to_f64(lse), rlse, rtol=0, atol=1e-4)


@pytest.mark.parametrize("pos", [
    [0, 15, 16, 300, 2047],            # 302 rounds for a 320-wave grid
    [0, 0, 0, 0, 0, 0, 0, 2047],      # 270 rounds for a 512-wave grid
])
def test_stream_fewer_rounds_than_waves(pos):
    """The streaming grid is sized from max_seq_len for every sequence; a
    ragged batch can hold fewer rounds than the grid has waves.  Every
    sequence must still be merged from exactly its own segments."""
    _print_case(test="stream_few_rounds", pos=pos)
    case = HybridCase(410 + len(pos), len(pos), FULL, pos, lmax=2048, poison=True)
    _, ref, rlse = case.oracle_step()
    _, out, lse = case.gpu_step()
    assert_attn_close(out, ref)
    np.testing.assert_allclose(to_f64(lse), rlse, rtol=0, atol=1e-4)


@pytest.mark.parametrize("lt", [SLIDING, FULL])
def test_sinks(lt):
    _print_case(test="sinks", lt=lt)
    pos = [700, 1200]
    case = HybridCase(500 + lt, 2, lt, pos, lmax=2048)
    _, ref0, lse0 = case.oracle_step()
    # sinks near lse actually move the output
    g = np.random.default_rng(1)
    sinks = (lse0.mean(0) + g.normal(0, 2, 8)).astype(np.float32)
    _, ref, _ = case.oracle_step(sinks=sinks)
    for chunk in (0, 64):
        _, out, lse = case.gpu_step(sinks=sinks, chunk_keys=chunk)
        assert_attn_close(out, ref)
        # -inf sink: bit-for-bit the no-sink output
        _, o_inf, _ = case.gpu_step(sinks=np.full(8, -np.inf, np.float32), chunk_keys=chunk)
        _, o_none, _ = case.gpu_step(sinks=None, chunk_keys=chunk)
        assert torch.equal(o_inf.view(torch.int16), o_none.view(torch.int16))
        assert_attn_close(o_none, ref0)
        # +inf sink absorbs everything
        _, o_pinf, _ = case.gpu_step(sinks=np.full(8, np.inf, np.float32), chunk_keys=chunk)
        assert torch.all(o_pinf.float() == 0)


def test_zero_length_sequence():
    _print_case(test="zero_length")
    case = HybridCase(600, 2, FULL, [10, 20], lmax=64)
    case.seq_lens = np.array([0, 21], np.int32)
    for chunk in (0, 16):
        _, out, lse = case.gpu_step(chunk_keys=chunk, max_seq_len=64, append=False)
        assert torch.all(out[0].float() == 0)
        assert torch.all(torch.isneginf(lse[0]))
        assert torch.all(torch.isfinite(out[1].float()))


def test_ring_order_and_resume():
    """Permuting the window's rows (ring slots and evicted-entry row) leaves
    the output unchanged up to summation order; copying the cache resumes
    exactly."""
    _print_case(test="ring_order")
    import full_kv_cache_amd as hda
    case = HybridCase(700, 2, SLIDING, [900, 2000])
    d, out0, _ = case.gpu_step()
    perm = torch.randperm(512, generator=torch.Generator().manual_seed(0)).cuda()
    d2 = {k: v.clone() for k, v in d.items()}
    d2["k"] = d["k"][:, :, perm].contiguous()
    d2["v"] = d["v"][:, :, perm].contiguous()
    _, out1, _ = case.gpu_step(d=d2, append=False)
    assert (out1.float() - out0.float()).abs().max().item() <= 2e-3
    d3 = {k: v.clone() for k, v in d.items()}
    _, out2, _ = case.gpu_step(d=d3, append=False)
    assert torch.equal(out2.view(torch.int16), out0.view(torch.int16))
    assert hda is not None


def test_batch64_throughput_shape_all():
    """Headline shape: batch 64, lengths uniform in [512, 4096], sinks drawn
    near lse; one sliding and one full layer through hda_rope_append +
    hda_decode_attn in the launch configuration of the two-call path; every
    sequence is checked against the oracle."""
    _print_case(test="batch64_all")
    g = np.random.default_rng(64)
    pos = g.integers(511, 4096, 64).astype(np.int32)
    for lt in (SLIDING, FULL):
        case = HybridCase(800 + lt, 64, lt, pos, lmax=4096)
        _, _, lse0 = case.oracle_step()
        sinks = near_lse_sinks(lse0, 80 + lt)
        _, ref, rlse = case.oracle_step(sinks=sinks)
        _, out, lse = case.gpu_step(sinks=sinks, max_seq_len=4096)
        assert_attn_close(out, ref)
        np.testing.assert_allclose(to_f64(lse), rlse, rtol=0, atol=1e-4)


def test_window_path_ragged():
    """Full layer at most 1024 keys long with a ragged length mix: the
    default split takes the window decomposition (one workgroup per sequence,
    KV head and half query group, no partials)."""
    pos = [0, 15, 16, 100, 511, 1000]
    _print_case(test="window_ragged", pos=pos)
    case = HybridCase(410, len(pos), FULL, pos, lmax=1024, poison=True)
    _, ref, rlse = case.oracle_step()
    _, out, lse = case.gpu_step(chunk_keys=0, max_seq_len=1024)
    assert_attn_close(out, ref)
    np.testing.assert_allclose(to_f64(lse), rlse, rtol=0, atol=1e-4)
