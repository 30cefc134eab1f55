"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module draws random numbers and nothing else: it holds none of the
attention, RoPE or cache arithmetic.  Both the HIP library and the CPU
oracle consume what it returns.

Every tensor comes from one ``torch.Generator`` in a fixed order, as fp32
``randn`` cast to bf16 (unit-normal values, the distribution the decode
workloads are quoted on).  Shapes follow the hybrid model of the Spark
export page: 8 query heads, 2 KV heads, head dim 256, a 512-token window
held as a 512-row block (511 ring slots plus the evicted-entry row), full
layers of ``lmax`` rows; and
the sparse MLA layer of the FlashMLA sparse page: 64 query heads over one
576-dim latent head.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

SLIDING = 0
FULL = 1


@dataclass(frozen=True)
class HybridShape:
    batch: int
    lmax: int                  # rows of each full-layer cache
    num_q_heads: int = 8
    num_kv_heads: int = 2
    head_dim: int = 256
    window: int = 512          # sliding window incl. the current token
    rot_sliding: int = 256
    theta_sliding: float = 1e4
    rot_full: int = 64
    theta_full: float = 5e6

    @property
    def ring_slots(self) -> int:
        return self.window - 1

    def capacity(self, layer_type: int) -> int:
        return self.window if layer_type == SLIDING else self.lmax

    def rot(self, layer_type: int) -> int:
        return self.rot_sliding if layer_type == SLIDING else self.rot_full

    def theta(self, layer_type: int) -> float:
        return self.theta_sliding if layer_type == SLIDING else self.theta_full


def layer_pattern(n_layers: int = 28) -> list[int]:
    """Three sliding layers then one full layer, repeated (index % 4 == 3 is full)."""
    return [FULL if i % 4 == 3 else SLIDING for i in range(n_layers)]


def generator(seed: int = 0, device: str | torch.device = "cpu") -> torch.Generator:
    return torch.Generator(device=device).manual_seed(seed)


def randn_bf16(gen: torch.Generator, shape, device="cpu", scale: float = 1.0) -> torch.Tensor:
    x = torch.randn(*shape, generator=gen, device=device, dtype=torch.float32)
    if scale != 1.0:
        x.mul_(scale)
    return x.to(torch.bfloat16)


def uniform_seq_lens(gen: torch.Generator, batch: int, lo: int, hi: int, device="cpu") -> torch.Tensor:
    """Per-sequence lengths uniform on [lo, hi] inclusive, int32."""
    return torch.randint(lo, hi + 1, (batch,), generator=gen, device=device, dtype=torch.int32)


def layer_inputs(gen: torch.Generator, shape: HybridShape, layer_type: int, device="cpu") -> dict:
    """One layer's step inputs, drawn in the order q, k_new, v_new, K, V."""
    B, Hq, Hkv, D = shape.batch, shape.num_q_heads, shape.num_kv_heads, shape.head_dim
    cap = shape.capacity(layer_type)
    out = {
        "q": randn_bf16(gen, (B, Hq, D), device),
        "k_new": randn_bf16(gen, (B, Hkv, D), device),
        "v_new": randn_bf16(gen, (B, Hkv, D), device),
        "k": randn_bf16(gen, (B, Hkv, cap, D), device),
        "v": randn_bf16(gen, (B, Hkv, cap, D), device),
    }
    return out


def sinks(gen: torch.Generator, num_heads: int, device="cpu") -> torch.Tensor:
    return torch.randn(num_heads, generator=gen, device=device, dtype=torch.float32)


def gate_logits(gen: torch.Generator, batch: int, num_heads: int, device="cpu") -> torch.Tensor:
    """Synthetic g_proj outputs for the per-head output gate: N(0, 1) fp32 [B, Hq]."""
    return torch.randn(batch, num_heads, generator=gen, device=device, dtype=torch.float32)


def fp8_codes(gen: torch.Generator, shape, device="cpu") -> torch.Tensor:
    """Uniformly random e4m3 codes, uint8, never NaN (0x7F / 0xFF): every
    sign, exponent and mantissa equally likely."""
    c = torch.randint(0, 254, tuple(shape), generator=gen, device=device, dtype=torch.int32)
    c = c + (c >= 0x7F).to(torch.int32)  # skip 0x7F; 0xFF is never reached
    return c.to(torch.uint8)


def fp8_scales(gen: torch.Generator, shape, device="cpu") -> torch.Tensor:
    """Per-row scales, fp32 uniform in [1, 2) / 448 (largest values 1 .. 2)."""
    return (torch.rand(tuple(shape), generator=gen, device=device, dtype=torch.float32) + 1.0) / 448.0


@dataclass(frozen=True)
class SparseShape:
    tokens: int = 32
    num_q_heads: int = 64
    dqk: int = 576
    dv: int = 512
    pool: int = 32768
    topk: int = 2048


def sparse_inputs(gen: torch.Generator, shape: SparseShape, device="cpu") -> dict:
    """q, the latent pool, per-token indices drawn without replacement, sinks."""
    T, H = shape.tokens, shape.num_q_heads
    q = randn_bf16(gen, (T, H, shape.dqk), device)
    kv = randn_bf16(gen, (shape.pool, shape.dqk), device)
    idx = torch.stack([
        torch.rand(shape.pool, generator=gen, device=device).argsort()[: shape.topk]
        for _ in range(T)
    ]).to(torch.int32)
    s = sinks(gen, H, device)
    return {"q": q, "kv": kv, "indices": idx, "sinks": s}


def bits(t: torch.Tensor):
    """bf16 tensor -> numpy uint16 bit patterns (host copy)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view("uint16")


def from_bits(a) -> torch.Tensor:
    """numpy uint16 bit patterns -> bf16 tensor (host)."""
    import numpy as np
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
