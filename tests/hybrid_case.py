"""Test helper: one hybrid-layer case on both sides.

Draws a layer's inputs with ``workloads``, keeps host bit copies for the
oracle and device copies for the library, and runs the step (append, then
attention) on each side.  Only tests import this module.

The library keeps a sliding layer as one block of `window` rows (ring slots
0..window-2, evicted-entry row window-1); the oracle keeps the ring and the
side row apart.  `to_oracle` / `from_oracle` convert between the two.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import workloads
from workloads import FULL, SLIDING

BF16_NAN = 0x7FC0


class HybridCase:
    def __init__(self, seed, batch, layer_type, pos, lmax=None, window=512, poison=False,
                 num_q_heads=8, num_kv_heads=2):
        self.lt = layer_type
        self.pos = np.asarray(pos, dtype=np.int32)
        assert self.pos.shape == (batch,)
        lmax = lmax or int(self.pos.max()) + 1
        self.shape = workloads.HybridShape(batch=batch, lmax=lmax, window=window,
                                           num_q_heads=num_q_heads, num_kv_heads=num_kv_heads)
        g = workloads.generator(seed)
        t = workloads.layer_inputs(g, self.shape, layer_type)
        self.host = {k: workloads.bits(v).copy() for k, v in t.items()}
        if poison:
            self._poison()
        self.seq_lens = self.pos + 1

    def _poison(self):
        """NaN in every row the step must not read: unwritten ring slots
        and the evicted-entry row below a full window (all rows past pos in
        the block), full-layer rows past pos."""
        h = self.host
        for b, p in enumerate(self.pos):
            h["k"][b, :, p + 1:] = BF16_NAN
            h["v"][b, :, p + 1:] = BF16_NAN

    # ------------------------------------------------ block <-> oracle form
    def to_oracle(self, h):
        """(k, v, kev, vev) in the oracle's form from a host block dict."""
        if self.lt == SLIDING:
            slots = self.shape.window - 1
            return (np.ascontiguousarray(h["k"][:, :, :slots]), np.ascontiguousarray(h["v"][:, :, :slots]),
                    np.ascontiguousarray(h["k"][:, :, slots]), np.ascontiguousarray(h["v"][:, :, slots]))
        z = np.zeros((self.shape.batch, self.shape.num_kv_heads, self.shape.head_dim), np.uint16)
        return h["k"], h["v"], z, z.copy()

    def from_oracle(self, k, v, kev, vev):
        """Block form (k, v) of the oracle's cache arrays."""
        if self.lt == SLIDING:
            return (np.concatenate([k, kev[:, :, None]], axis=2), np.concatenate([v, vev[:, :, None]], axis=2))
        return k, v

    # ---------------------------------------------------------- oracle side
    def oracle_step(self, sinks=None, scale=1 / 16, gate=None):
        """Append then attention in the oracle; returns the block-form host
        state after the append, out and lse.  gate: fp32 [B, Hq] logits."""
        h = {k: v.copy() for k, v in self.host.items()}
        s = self.shape
        k, v, kev, vev = self.to_oracle(h)
        oracle.rope_append(h["q"], h["k_new"], h["v_new"], self.pos, self.lt, s.rot(self.lt),
                           s.theta(self.lt), s.window, k, v, kev, vev)
        out, lse = oracle.decode_attn(h["q"], k, v, kev, vev, self.seq_lens, self.lt, s.window,
                                      sinks, scale, gate=gate)
        h["k"], h["v"] = self.from_oracle(k, v, kev, vev)
        return h, out, lse

    # ------------------------------------------------------------- GPU side
    def device(self, dev="cuda"):
        return {k: workloads.from_bits(v).to(dev) for k, v in self.host.items()}

    def cache(self, d):
        import full_kv_cache_amd as hda
        s = self.shape
        return hda.LayerCache(d["k"], d["v"], s.num_q_heads, s.window, s.rot(self.lt),
                              s.theta(self.lt))

    def gpu_step(self, sinks=None, scale=1 / 16, chunk_keys=0, max_seq_len=None, d=None,
                 append=True, gate=None):
        import full_kv_cache_amd as hda
        d = d or self.device()
        cache = self.cache(d)
        pos = torch.from_numpy(self.pos).cuda()
        seq = torch.from_numpy(self.seq_lens).cuda()
        if append:
            hda.hda_rope_append(d["q"], d["k_new"], d["v_new"], pos, self.lt, cache)
        msl = int(max_seq_len or self.seq_lens.max())
        ws_bytes = hda.hda_decode_workspace_bytes(cache, self.lt, msl, chunk_keys)
        ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device="cuda") if ws_bytes else None
        s = self.shape
        out = torch.full((s.batch, s.num_q_heads, s.head_dim), float("nan"), dtype=torch.bfloat16,
                         device="cuda")
        lse = torch.full((s.batch, s.num_q_heads), float("nan"), dtype=torch.float32, device="cuda")
        sk = None if sinks is None else torch.as_tensor(sinks, dtype=torch.float32).cuda()
        gt = None if gate is None else torch.as_tensor(gate, dtype=torch.float32).cuda()
        hda.hda_decode_attn(d["q"], cache, seq, self.lt, sk, scale, out, lse, msl, chunk_keys, ws,
                            gate=gt)
        torch.cuda.synchronize()
        return d, out, lse


def fused_step(case: "HybridCase", sinks=None, scale=1 / 16, d=None, workspace=None, gate=None):
    """hda_decode_step on the case's device tensors (q is not modified)."""
    import full_kv_cache_amd as hda
    d = d or case.device()
    cache = case.cache(d)
    pos = torch.from_numpy(case.pos).cuda()
    if workspace is None:
        nbytes = hda.hda_decode_step_workspace_bytes(cache, case.lt)
        workspace = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    s = case.shape
    out = torch.full((s.batch, s.num_q_heads, s.head_dim), float("nan"), dtype=torch.bfloat16,
                     device="cuda")
    lse = torch.full((s.batch, s.num_q_heads), float("nan"), dtype=torch.float32, device="cuda")
    sk = None if sinks is None else torch.as_tensor(sinks, dtype=torch.float32).cuda()
    gt = None if gate is None else torch.as_tensor(gate, dtype=torch.float32).cuda()
    hda.hda_decode_step(d["q"], d["k_new"], d["v_new"], pos, case.lt, cache, sk, scale, out, lse,
                        workspace, gate=gt)
    torch.cuda.synchronize()
    return d, out, lse


def near_lse_sinks(lse, seed, spread=2.0):
    """Per-head sinks drawn near the heads' lse (mean over sequences plus
    N(0, spread)): factors 1/(1+exp(sink-lse)) spread over (0, 1), so the
    sink moves the output (an N(0, 1) sink next to lse ~ 8 barely does)."""
    g = np.random.default_rng(seed)
    lse = np.asarray(lse, np.float64)
    return (lse.reshape(-1, lse.shape[-1]).mean(0) + g.normal(0, spread, lse.shape[-1])).astype(np.float32)


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().double().numpy()


def bits_of(t: torch.Tensor) -> np.ndarray:
    return workloads.bits(t)


def assert_attn_close(out_gpu, out_ref, max_abs=1e-2, mean_abs=1e-3):
    """The decode tolerance for unit-normal bf16 inputs with fp32 accumulation."""
    got = to_f64(out_gpu)
    assert np.all(np.isfinite(got)), "non-finite output"
    err = np.abs(got - out_ref)
    assert err.max() <= max_abs, f"max abs err {err.max():.3e}"
    assert err.mean() <= mean_abs, f"mean abs err {err.mean():.3e}"
    return float(err.max()), float(err.mean())


def bf16_ulp_diff(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """|a - b| in bf16 ulps (same-sign finite values; order-preserving map)."""
    def key(x):
        x = x.astype(np.int32)
        return np.where(x & 0x8000, 0x8000 - (x & 0x7FFF), 0x8000 + (x & 0x7FFF))
    return np.abs(key(a_bits) - key(b_bits))


def assert_rotated_close(got_bits, ref_bits, rot=None, max_frac=1e-3):
    """Rotated bf16 values (last axis = head dims, rotary pairs j and
    j + rot/2) against the oracle's.  Both sides use the same fp32 cos /
    sin; the kernel forms x1 c - x2 s in fp32 (one rounded product, one
    fma), the oracle in fp64, and each rounds once to bf16.  So a value is
    within one bf16 ulp of the oracle's, except where the rotation cancels
    (a result far below its pair's norm): there the fp32 product's rounding,
    at most 2^-24 of the pair's norm, can be many ulps of the small result,
    and the bound is 2^-22 of the norm.  Fewer than max_frac of the values
    differ at all."""
    got_bits = np.asarray(got_bits)
    ref_bits = np.asarray(ref_bits)
    ulps = bf16_ulp_diff(got_bits, ref_bits)
    g, r = oracle.bf16_to_f64(got_bits), oracle.bf16_to_f64(ref_bits)
    rot = rot or r.shape[-1]
    h = rot // 2
    norm = np.zeros_like(r)
    pn = np.sqrt(r[..., :h] ** 2 + r[..., h:rot] ** 2)
    norm[..., :h] = pn
    norm[..., h:rot] = pn
    ok = (ulps <= 1) | (np.abs(g - r) <= 2.0 ** -22 * norm)
    assert ok.all(), f"{(~ok).sum()} rotated values off by more than the fp32 rounding bound"
    frac = (ulps > 0).mean()
    assert frac < max_frac, f"{frac:.2e} of rotated values differ"

