"""Parity at the headline shape for the paged, fp8 and chunk-decode paths:
batch 64, context lengths uniform in [512, 4096] (the bench's workload),
in the launch configuration the bench times (one-launch window step for
fp8 sliding layers, streaming kernel for full layers, 64-row shuffled
pages, 4-token chunks with the workgroup split max_seq_len 4096 selects).
The oracle checks a sample of 8 sequences, computed from the same inputs
restricted to them (every kernel treats sequences independently).
Tolerances as everywhere: out max-abs <= 1e-2, mean-abs <= 1e-3; lse 1e-4.
"""
import copy

import numpy as np
import pytest
import torch

from hybrid_case import FULL, SLIDING, HybridCase, assert_attn_close, to_f64
from test_gpu_fp8 import Fp8Case
from test_gpu_multi import MultiCase
from test_gpu_paged import _run as paged_run

pytestmark = pytest.mark.gpu
SAMPLE = np.array([0, 1, 7, 20, 33, 47, 62, 63])


def _positions(seed):
    return np.random.default_rng(seed).integers(511, 4096, 64).astype(np.int32)


def _restrict(case, names, sample=SAMPLE):
    sub = copy.copy(case)
    for n in names:
        setattr(sub, n, np.ascontiguousarray(getattr(case, n)[sample]))
    sub.pos = case.pos[sample]
    if hasattr(case, "seq_lens"):
        sub.seq_lens = sub.pos + 1
    if hasattr(case, "shape"):
        sub.shape = case.shape.__class__(batch=len(sample), lmax=case.shape.lmax,
                                         num_q_heads=case.shape.num_q_heads,
                                         num_kv_heads=case.shape.num_kv_heads)
    return sub


def _close(out, lse, ref, rlse):
    idx = torch.from_numpy(SAMPLE).cuda()
    assert_attn_close(out[idx], ref)
    np.testing.assert_allclose(to_f64(lse)[SAMPLE], rlse, rtol=0, atol=1e-4)


def test_fp8_full_layer_batch64():
    print("CASE fullsize fp8 full", flush=True)
    case = Fp8Case(5000, FULL, _positions(1), 4096)
    _, out, lse = case.gpu_step()
    sub = _restrict(case, ("q", "k_new", "v_new", "kc", "vc", "ks", "vs"))
    _, _, ref, rlse = sub.oracle_step()
    _close(out, lse, ref, rlse)


def test_fp8_sliding_step_batch64():
    import full_kv_cache_amd as hda
    print("CASE fullsize fp8 sliding step", flush=True)
    case = Fp8Case(5001, SLIDING, _positions(2))
    d = case.device()
    cache = case.cache(d)
    ws = torch.zeros(hda.hda_decode_step_workspace_bytes(cache, SLIDING), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((64, 8, 256), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((64, 8), device="cuda")
    hda.hda_decode_step(d["q"], d["k_new"], d["v_new"], torch.from_numpy(case.pos).cuda(), SLIDING,
                        cache, None, 1 / 16, out, lse, ws)
    torch.cuda.synchronize()
    sub = _restrict(case, ("q", "k_new", "v_new", "kc", "vc", "ks", "vs"))
    _, _, ref, rlse = sub.oracle_step()
    _close(out, lse, ref, rlse)


def test_paged_full_layer_batch64():
    print("CASE fullsize paged", flush=True)
    case = HybridCase(5002, 64, FULL, _positions(3), lmax=4096, poison=True)
    *_, out, lse = paged_run(case, 64)
    sub = HybridCase(5002, 64, FULL, case.pos, lmax=4096, poison=True)
    for k in sub.host:
        sub.host[k] = sub.host[k][SAMPLE].copy()
    sub.pos, sub.seq_lens = case.pos[SAMPLE], case.seq_lens[SAMPLE]
    sub.shape = sub.shape.__class__(batch=len(SAMPLE), lmax=4096)
    _, ref, rlse = sub.oracle_step()
    _close(out, lse, ref, rlse)


@pytest.mark.parametrize("lt", [SLIDING, FULL])
def test_chunk_decode_batch64(lt):
    """4-token chunks, token 0 at seq_len - 4 (as the bench), max_seq_len
    4096: the split the bench runs (two workgroups per pair here)."""
    import full_kv_cache_amd as hda
    print("CASE fullsize chunk", lt, flush=True)
    pos = _positions(4) - 3
    case = MultiCase(5003 + lt, lt, pos, 4, cap=4096 if lt == FULL else None)
    import workloads
    dev = {n: workloads.from_bits(getattr(case, n)).cuda() for n in ("q", "k_new", "v_new", "k", "v")}
    cache = hda.LayerCache(dev["k"], dev["v"], case.hq, 512, case.rot, case.theta)
    nbytes = hda.hda_decode_multi_workspace_bytes(cache, lt, 4, 4096)
    assert nbytes > 0  # split
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    out = torch.empty(case.q.shape, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(case.q.shape[:3], device="cuda")
    hda.hda_decode_multi(dev["q"], dev["k_new"], dev["v_new"], torch.from_numpy(case.pos).cuda(), lt,
                         cache, None, 1 / 16, out, lse, max_seq_len=4096, workspace=ws)
    torch.cuda.synchronize()
    sub = _restrict(case, ("q", "k_new", "v_new", "k", "v"))
    _, _, _, ref, rlse = sub.oracle()
    _close(out, lse, ref, rlse)
