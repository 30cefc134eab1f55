"""GPU parity of the per-head output gate (Spark export page,
`_Layer.forward`: out of head h times the sigmoid of its g_proj value)
against the fp64 oracle, on every kernel epilogue that writes out:
the window kernel (sliding hda_decode_attn), the streaming kernel + merge
(full), the chunk kernel with one chunk and with the LSE merge, the fused
step in its window and streaming forms, and hda_lse_merge alone.

Gate logits span [-6, 6] (factors 0.0025 .. 0.9975), distinct per
(sequence, head), with sinks near lse so that both factors matter.
Tolerances as for the ungated paths (out max-abs <= 1e-2, mean-abs <= 1e-3;
lse within 1e-4, and lse does not depend on the gate).
"""
import numpy as np
import pytest
import torch

from hybrid_case import FULL, SLIDING, HybridCase, assert_attn_close, fused_step, to_f64

pytestmark = pytest.mark.gpu


def _gate(B, Hq, seed):
    rng = np.random.default_rng(seed)
    return rng.uniform(-6, 6, size=(B, Hq)).astype(np.float32)


def _sinks(Hq):
    return np.linspace(4.5, 8.5, Hq).astype(np.float32)


def _check(out, lse, ref, rlse):
    assert_attn_close(out, ref)
    np.testing.assert_allclose(to_f64(lse), rlse, rtol=0, atol=1e-4)


@pytest.mark.parametrize("lt,chunk,pos,lmax", [
    (SLIDING, 0, [5, 511, 1500], 2048),    # window kernel
    (FULL, 0, [5, 700, 2047], 2048),       # streaming kernel + merge
    (FULL, 512, [5, 300, 511], 512),       # one chunk: the chunk kernel writes out
    (FULL, 128, [5, 700, 2047], 2048),     # chunks + LSE merge kernel
])
def test_gate_decode_attn(lt, chunk, pos, lmax):
    print("CASE gate_decode_attn", lt, chunk, pos, flush=True)
    case = HybridCase(1200 + chunk + lt, len(pos), lt, pos, lmax=lmax, poison=True)
    B, Hq = len(pos), case.shape.num_q_heads
    g, sk = _gate(B, Hq, 7 + chunk), _sinks(Hq)
    _, ref, rlse = case.oracle_step(sinks=sk, gate=g)
    _, ref0, rlse0 = case.oracle_step(sinks=sk)
    assert np.array_equal(rlse, rlse0)
    d, out, lse = case.gpu_step(sinks=sk, gate=g, chunk_keys=chunk, max_seq_len=lmax)
    _check(out, lse, ref, rlse)


@pytest.mark.parametrize("lt,pos", [(SLIDING, [5, 511, 1500]), (FULL, [5, 700, 2047])])
def test_gate_decode_step(lt, pos):
    print("CASE gate_decode_step", lt, pos, flush=True)
    case = HybridCase(1300 + lt, len(pos), lt, pos, lmax=2048, poison=True)
    B, Hq = len(pos), case.shape.num_q_heads
    g, sk = _gate(B, Hq, 11 + lt), _sinks(Hq)
    _, ref, rlse = case.oracle_step(sinks=sk, gate=g)
    _, out, lse = fused_step(case, sinks=sk, gate=g)
    _check(out, lse, ref, rlse)


def test_gate_lse_merge_and_limits():
    """hda_lse_merge with a gate equals the gated one-call result bit for
    bit; gate +inf reproduces the ungated output bit for bit, gate 0 halves
    it, and -inf gives 0."""
    print("CASE gate_lse_merge", flush=True)
    import full_kv_cache_amd as hda
    pos = [100, 700, 1500, 2047]
    case = HybridCase(1400, 4, FULL, pos, lmax=2048)
    Hq = case.shape.num_q_heads
    g = _gate(4, Hq, 13)
    d, out, lse = case.gpu_step(gate=g, chunk_keys=64)
    cache = case.cache(d)
    seq = torch.from_numpy(case.seq_lens).cuda()
    c, n = hda.hda_decode_split_plan(cache, FULL, 2048, 64)
    po = torch.full((4, Hq, n, 256), float("nan"), device="cuda")
    pl = torch.full((4, Hq, n), float("nan"), device="cuda")
    hda.hda_decode_attn_partials(d["q"], cache, seq, FULL, 1 / 16, 2048, 64, po, pl)
    out2 = torch.empty_like(out)
    hda.hda_lse_merge(po, pl, None, out2, None, gate=torch.from_numpy(g).cuda())
    torch.cuda.synchronize()
    assert torch.equal(out2.view(torch.int16), out.view(torch.int16))
    base = torch.empty_like(out)
    hda.hda_lse_merge(po, pl, None, base)
    for val, check in ((np.inf, lambda o: torch.equal(o.view(torch.int16), base.view(torch.int16))),
                       (0.0, lambda o: torch.equal(o.float(), (base.float() * 0.5))),
                       (-np.inf, lambda o: not o.float().abs().any())):
        o = torch.empty_like(out)
        gv = torch.full((4, Hq), val, dtype=torch.float32, device="cuda")
        hda.hda_lse_merge(po, pl, None, o, gate=gv)
        torch.cuda.synchronize()
        assert check(o), val
