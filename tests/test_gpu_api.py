"""GPU checks of the two-stage API and of graph replay (MI355X).

* hda_decode_attn_partials + hda_lse_merge give exactly the one-call
  result, and the partials themselves match the oracle's per-chunk
  softmax (Spark ring-branch comment: softmax over key subsets, merged).
* A HIP graph of a two-layer step, replayed several times with eager work
  and synchronisations between replays, reproduces the eager output bit
  for bit on every replay.
"""
import numpy as np
import pytest
import torch

import oracle
from hybrid_case import FULL, SLIDING, HybridCase, assert_attn_close, to_f64

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("lt,chunk", [(FULL, 64), (FULL, 256), (SLIDING, 128), (SLIDING, 512)])
def test_partials_then_merge(lt, chunk):
    print("CASE partials_then_merge", lt, chunk, flush=True)
    import full_kv_cache_amd as hda
    pos = [100, 700, 1500, 2047]
    case = HybridCase(900 + chunk, 4, lt, pos, lmax=2048)
    sinks = np.linspace(4, 9, 8).astype(np.float32)
    d, out, lse = case.gpu_step(sinks=sinks, chunk_keys=chunk)
    cache = case.cache(d)
    seq = torch.from_numpy(case.seq_lens).cuda()
    msl = int(case.seq_lens.max())
    c, n = hda.hda_decode_split_plan(cache, lt, msl, chunk)
    assert c == chunk
    po = torch.full((4, 8, n, 256), float("nan"), device="cuda")
    pl = torch.full((4, 8, n), float("nan"), device="cuda")
    hda.hda_decode_attn_partials(d["q"], cache, seq, lt, 1 / 16, msl, chunk, po, pl)
    out2 = torch.empty_like(out)
    lse2 = torch.empty_like(lse)
    sk = torch.from_numpy(sinks).cuda()
    hda.hda_lse_merge(po, pl, sk, out2, lse2)
    torch.cuda.synchronize()
    assert torch.equal(out2.view(torch.int16), out.view(torch.int16))
    assert torch.equal(lse2, lse)
    # per-chunk partials against the oracle, full layers (contiguous rows)
    if lt == FULL:
        q = case.host["q"].copy()
        from workloads import bits
        qb = bits(d["q"])
        kb, vb = bits(d["k"]), bits(d["v"])
        for b in (0, 3):
            for h in (0, 5):
                for ci in range(n):
                    r0, r1 = ci * chunk, min((ci + 1) * chunk, int(case.seq_lens[b]))
                    o_ref, l_ref = oracle.attn_chunk(qb[b, h], kb[b, h // 4], vb[b, h // 4], r0, r1,
                                                     1 / 16)
                    if r1 <= r0:
                        assert np.isneginf(pl[b, h, ci].item())
                        continue
                    got = po[b, h, ci].cpu().double().numpy()
                    assert np.abs(got - o_ref).max() < 2e-3
                    assert abs(pl[b, h, ci].item() - l_ref) < 1e-4
        assert q is not None


def test_graph_replay_matches_eager():
    print("CASE graph_replay", flush=True)
    import full_kv_cache_amd as hda
    cases = [HybridCase(950, 3, SLIDING, [511, 1000, 20]),
             HybridCase(951, 3, FULL, [511, 1000, 20], lmax=1024)]
    pristine = [c.device() for c in cases]
    live = [{k: v.clone() for k, v in p.items()} for p in pristine]
    pos = torch.tensor([511, 1000, 20], dtype=torch.int32, device="cuda")
    seq = pos + 1
    sinks = torch.linspace(-1, 8, 8, device="cuda")
    outs = [torch.empty(3, 8, 256, dtype=torch.bfloat16, device="cuda") for _ in cases]
    ws = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda")

    def step():
        for c, d, o in zip(cases, live, outs):
            cache = c.cache(d)
            hda.hda_rope_append(d["q"], d["k_new"], d["v_new"], pos, c.lt, cache)
            hda.hda_decode_attn(d["q"], cache, seq, c.lt, sinks, 1 / 16, o, None, 1001, 64, ws)

    def reset():
        for d, p in zip(live, pristine):
            for k in d:
                d[k].copy_(p[k])

    reset()
    step()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    eager_cache = [{k: v.clone() for k, v in d.items()} for d in live]
    for c, o in zip(cases, eager):
        _, ref, _ = c.oracle_step(sinks=sinks.cpu().numpy())
        assert_attn_close(o, ref)
    reset()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        reset()
        torch.cuda.synchronize()
        for o in outs:
            o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        _ = (torch.randn(1000, device="cuda") @ torch.randn(1000, device="cuda"))  # eager work
        for o, e in zip(outs, eager):
            assert torch.equal(o.view(torch.int16), e.view(torch.int16)), rep
        for d, e in zip(live, eager_cache):
            for k in d:
                assert torch.equal(d[k].view(torch.int16), e[k].view(torch.int16)), (rep, k)


def test_stream_workspace_reuse():
    """One workspace serves call after call of the default (streaming) path
    with identical results."""
    print("CASE workspace_reuse", flush=True)
    import full_kv_cache_amd as hda
    case = HybridCase(960, 5, FULL, [100, 4000, 17, 2500, 900], lmax=4096)
    d = case.device()
    cache = case.cache(d)
    seq = torch.from_numpy(case.seq_lens).cuda()
    nbytes = hda.hda_decode_workspace_bytes(cache, FULL, 4096, 0)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(3):
        out = torch.empty(5, 8, 256, dtype=torch.bfloat16, device="cuda")
        hda.hda_decode_attn(d["q"], cache, seq, FULL, None, 1 / 16, out, None, 4096, 0, ws)
        torch.cuda.synchronize()
        outs.append(out)
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    assert torch.equal(outs[0].view(torch.int16), outs[2].view(torch.int16))


def test_one_workspace_serves_both_paths():
    """One workspace serves the streaming and the chunked path in any order
    (a chunked call once overwrote state a later streaming call relied on)."""
    print("CASE workspace_both_paths", flush=True)
    import full_kv_cache_amd as hda
    case = HybridCase(961, 6, FULL, [3000, 20, 4095, 700, 1, 2200], lmax=4096)
    _, ref, _ = case.oracle_step()
    d = case.device()
    cache = case.cache(d)
    pos = torch.from_numpy(case.pos).cuda()
    hda.hda_rope_append(d["q"], d["k_new"], d["v_new"], pos, FULL, cache)
    seq = torch.from_numpy(case.seq_lens).cuda()
    nbytes = max(hda.hda_decode_workspace_bytes(cache, FULL, 4096, c) for c in (0, 64, 256))
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    for chunk in (0, 64, 0, 256, 0):
        out = torch.full((6, 8, 256), float("nan"), dtype=torch.bfloat16, device="cuda")
        hda.hda_decode_attn(d["q"], cache, seq, FULL, None, 1 / 16, out, None, 4096, chunk, ws)
        torch.cuda.synchronize()
        assert_attn_close(out, ref)
