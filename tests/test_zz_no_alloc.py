"""hda_decode_step_noalloc (the step with the library's static per-device
scratch as its workspace) against hda_decode_step with a caller workspace,
through the C ABI: the same kernels, so out, lse and the cache must agree
bit for bit; both checked against the oracle at the decode tolerance.  Two
calls in a row, the second with a smaller batch, for a sliding layer (the
head-split window step at batch 64, the key split at batch 5) and a full
layer (the streaming step form); a step too large for the scratch is
refused on the host."""
import ctypes

import numpy as np
import pytest
import torch

from hybrid_case import FULL, SLIDING, HybridCase, assert_attn_close, fused_step, to_f64

pytestmark = pytest.mark.gpu


def _noalloc(case, d, sinks):
    import full_kv_cache_amd as hda
    s = case.shape
    out = torch.full((s.batch, s.num_q_heads, s.head_dim), float("nan"), dtype=torch.bfloat16,
                     device="cuda")
    lse = torch.full((s.batch, s.num_q_heads), float("nan"), dtype=torch.float32, device="cuda")
    hda.hda_decode_step_noalloc(d["q"], d["k_new"], d["v_new"], torch.from_numpy(case.pos).cuda(),
                                case.lt, case.cache(d), torch.from_numpy(sinks).cuda(), 1 / 16, out, lse)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("lt,batches,lmax", [(SLIDING, (64, 5), None), (FULL, (64, 7), 4096)])
def test_noalloc_matches_step(lt, batches, lmax):
    for call, B in enumerate(batches):
        print(f"CASE noalloc lt={lt} call={call} batch={B}", flush=True)
        rng = np.random.default_rng(100 * lt + call)
        pos = rng.integers(0, 4096, B).astype(np.int32)
        pos[:2] = [0, 511]
        case = HybridCase(7000 + 10 * lt + call, B, lt, pos, lmax=lmax or 4096)
        sinks = np.linspace(4.0, 9.0, case.shape.num_q_heads).astype(np.float32)
        h, ref, rlse = case.oracle_step(sinks=sinks)
        d1 = case.device()
        out1, lse1 = _noalloc(case, d1, sinks)
        d2, out2, lse2 = fused_step(case, sinks=sinks)
        assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
        assert torch.equal(lse1, lse2)
        for k in ("k", "v"):
            assert torch.equal(d1[k].view(torch.int16), d2[k].view(torch.int16))
        assert_attn_close(out1, ref)
        np.testing.assert_allclose(to_f64(lse1), rlse, rtol=0, atol=1e-4)


def test_noalloc_refuses_a_step_beyond_the_scratch():
    import full_kv_cache_amd as hda
    L = hda.lib()
    fake = 0x10000  # never dereferenced: the call is refused on the host
    d = hda.CacheDesc(batch=4096, num_q_heads=8, num_kv_heads=2, head_dim=256, window=512,
                      rotary_dim=64, capacity=4096, rope_theta=5e6, k=fake, v=fake)
    assert L.hda_decode_step_workspace_bytes(ctypes.byref(d), FULL) > 16 << 20
    P = ctypes.c_void_p
    r = L.hda_decode_step_noalloc(P(fake), P(fake), P(fake), P(fake), FULL, ctypes.byref(d), None, None,
                                  0.0625, P(fake), None, None)
    assert r == 3 and b"static scratch" in L.hda_last_error_message()
