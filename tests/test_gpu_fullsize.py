"""Parity at the headline shape for the paged, fp8 and chunk-decode paths:
batch 64, context lengths uniform in [512, 4096] (the bench's workload),
in the launch configuration the bench times (one-launch window step for
fp8 sliding layers, streaming kernel for full layers, 64-row shuffled
pages, 4-token chunks with the workgroup split max_seq_len 4096 selects).
Every sequence is checked against the oracle, with per-head sinks drawn
near the heads' lse (so the sink factor spreads over (0, 1)).
Tolerances as everywhere: out max-abs <= 1e-2, mean-abs <= 1e-3; lse 1e-4.
"""
import numpy as np
import pytest
import torch

from hybrid_case import FULL, SLIDING, HybridCase, assert_attn_close, near_lse_sinks, to_f64
from test_gpu_fp8 import Fp8Case
from test_gpu_multi import MultiCase
from test_gpu_paged import _run as paged_run

pytestmark = pytest.mark.gpu


def _positions(seed):
    return np.random.default_rng(seed).integers(511, 4096, 64).astype(np.int32)


def _close(out, lse, ref, rlse):
    assert_attn_close(out, ref)
    np.testing.assert_allclose(to_f64(lse), rlse, rtol=0, atol=1e-4)


def test_fp8_full_layer_batch64():
    print("CASE fullsize fp8 full", flush=True)
    case = Fp8Case(5000, FULL, _positions(1), 4096)
    *_, lse0 = case.oracle_step()
    sinks = near_lse_sinks(lse0, 5000)
    _, _, ref, rlse = case.oracle_step(sinks=sinks)
    _, out, lse = case.gpu_step(sinks=sinks)
    _close(out, lse, ref, rlse)


def test_fp8_sliding_step_batch64():
    import full_kv_cache_amd as hda
    print("CASE fullsize fp8 sliding step", flush=True)
    case = Fp8Case(5001, SLIDING, _positions(2))
    *_, lse0 = case.oracle_step()
    sinks = near_lse_sinks(lse0, 5001)
    _, _, ref, rlse = case.oracle_step(sinks=sinks)
    d = case.device()
    cache = case.cache(d)
    ws = torch.zeros(hda.hda_decode_step_workspace_bytes(cache, SLIDING), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((64, 8, 256), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((64, 8), device="cuda")
    hda.hda_decode_step(d["q"], d["k_new"], d["v_new"], torch.from_numpy(case.pos).cuda(), SLIDING,
                        cache, torch.from_numpy(sinks).cuda(), 1 / 16, out, lse, ws)
    torch.cuda.synchronize()
    _close(out, lse, ref, rlse)


def test_paged_full_layer_batch64():
    print("CASE fullsize paged", flush=True)
    case = HybridCase(5002, 64, FULL, _positions(3), lmax=4096, poison=True)
    _, _, lse0 = case.oracle_step()
    sinks = near_lse_sinks(lse0, 5002)
    _, ref, rlse = case.oracle_step(sinks=sinks)
    *_, out, lse = paged_run(case, 64, sinks=sinks)
    _close(out, lse, ref, rlse)


@pytest.mark.parametrize("lt", [SLIDING, FULL])
def test_chunk_decode_batch64(lt):
    """4-token chunks, token 0 at seq_len - 4 (as the bench), max_seq_len
    4096: the split the bench runs (two workgroups per pair here)."""
    import full_kv_cache_amd as hda
    import workloads
    print("CASE fullsize chunk", lt, flush=True)
    pos = _positions(4) - 3
    case = MultiCase(5003 + lt, lt, pos, 4, cap=4096 if lt == FULL else None)
    *_, lse0 = case.oracle()
    sinks = near_lse_sinks(lse0, 5003 + lt)
    _, _, _, ref, rlse = case.oracle(sinks=sinks)
    dev = {n: workloads.from_bits(getattr(case, n)).cuda() for n in ("q", "k_new", "v_new", "k", "v")}
    cache = hda.LayerCache(dev["k"], dev["v"], case.hq, 512, case.rot, case.theta)
    nbytes = hda.hda_decode_multi_workspace_bytes(cache, lt, 4, 4096)
    assert nbytes > 0  # split
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    out = torch.empty(case.q.shape, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(case.q.shape[:3], device="cuda")
    hda.hda_decode_multi(dev["q"], dev["k_new"], dev["v_new"], torch.from_numpy(case.pos).cuda(), lt,
                         cache, torch.from_numpy(sinks).cuda(), 1 / 16, out, lse, max_seq_len=4096,
                         workspace=ws)
    torch.cuda.synchronize()
    _close(out, lse, ref, rlse)
