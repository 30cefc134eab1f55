"""Pins for the oracle's sparse top-k decode with sink (CPU only).

[SINK] `_bf16_flash_mla_kernel`: every query head of a token shares one
latent KV head and the token's top-k index list; keys are whole rows,
values their leading ``head_dim_v`` dims.  References:
  * top-k = whole pool with identity indices reduces to dense multi-query
    attention -- torch SDPA in fp64;
  * random indices: SDPA over the explicitly gathered rows;
  * topk_length keeps only the prefix of the index list; negative indices
    are skipped; a -inf sink is a bitwise no-op; the sink equals an extra
    zero-value key.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads


def _f(bits):
    return torch.from_numpy(oracle.bf16_to_f64(bits))


def _inputs(seed, T, H, dqk, dv, N, topk):
    shape = workloads.SparseShape(tokens=T, num_q_heads=H, dqk=dqk, dv=dv, pool=N, topk=topk)
    t = workloads.sparse_inputs(workloads.generator(seed), shape)
    return {"q": workloads.bits(t["q"]), "kv": workloads.bits(t["kv"]),
            "indices": t["indices"].numpy(), "sinks": t["sinks"].numpy()}


def _ref(t, scale, dv, lens=None, sinks=None):
    T, H, D = t["q"].shape
    out = np.zeros((T, H, dv))
    for i in range(T):
        idx = t["indices"][i]
        if lens is not None:
            idx = idx[: lens[i]]
        idx = idx[idx >= 0]
        K = _f(t["kv"][idx])[None, None]           # [1,1,n,D]
        V = K[..., :dv]
        q = _f(t["q"][i])[None, :, None]           # [1,H,1,D]
        mask = None
        if sinks is not None:
            K = torch.cat([K, torch.zeros(1, 1, 1, D, dtype=torch.float64)], 2)
            V = torch.cat([V, torch.zeros(1, 1, 1, dv, dtype=torch.float64)], 2)
            mask = torch.zeros(1, H, 1, K.shape[2], dtype=torch.float64)
            mask[0, :, 0, -1] = torch.from_numpy(sinks.astype(np.float64))
        o = F.scaled_dot_product_attention(q, K.expand(1, H, -1, -1), V.expand(1, H, -1, -1),
                                           attn_mask=mask, scale=scale)
        out[i] = o[0, :, 0].numpy()
    return out


def test_dense_reduction():
    T, H, dqk, dv, N = 2, 8, 64, 48, 40
    t = _inputs(1, T, H, dqk, dv, N, N)
    t["indices"] = np.tile(np.arange(N, dtype=np.int32), (T, 1))
    scale = 1 / np.sqrt(dqk)
    out, lse = oracle.sparse_decode_attn(t["q"], t["kv"], t["indices"], None, None, scale, dv)
    np.testing.assert_allclose(out, _ref(t, scale, dv), rtol=0, atol=1e-12)
    for i in range(T):
        s = _f(t["kv"]) @ _f(t["q"][i]).T * scale    # [N, H]
        np.testing.assert_allclose(lse[i], torch.logsumexp(s, 0).numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("with_sink", [False, True])
def test_gathered_brute_force(with_sink):
    T, H, dqk, dv, N, topk = 3, 16, 576, 512, 300, 64
    t = _inputs(2, T, H, dqk, dv, N, topk)
    scale = 1 / np.sqrt(dqk)
    sinks = t["sinks"] if with_sink else None
    out, _ = oracle.sparse_decode_attn(t["q"], t["kv"], t["indices"], None, sinks, scale, dv)
    np.testing.assert_allclose(out, _ref(t, scale, dv, sinks=sinks), rtol=0, atol=1e-12)


def test_topk_length_and_negative_indices():
    T, H, dqk, dv, N, topk = 3, 4, 64, 32, 100, 20
    t = _inputs(3, T, H, dqk, dv, N, topk)
    t["indices"][1, 3] = -1
    lens = np.array([20, 7, 0], np.int32)
    scale = 0.125
    out, lse = oracle.sparse_decode_attn(t["q"], t["kv"], t["indices"], lens, None, scale, dv)
    ref = _ref(t, scale, dv, lens=lens[:2].tolist() + [1])
    np.testing.assert_allclose(out[:2], ref[:2], rtol=0, atol=1e-12)
    assert np.all(out[2] == 0) and np.all(np.isneginf(lse[2]))   # empty key set


def test_neg_inf_sink_noop():
    t = _inputs(4, 2, 8, 64, 64, 50, 10)
    a, la = oracle.sparse_decode_attn(t["q"], t["kv"], t["indices"], None, None, 0.1, 64)
    b, lb = oracle.sparse_decode_attn(t["q"], t["kv"], t["indices"], None,
                                      np.full(8, -np.inf, np.float32), 0.1, 64)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


# ------------------------------------------------------------ fp8 pool
# [SINK] `_fp8_flash_mla_kernel`: the same sparse attention over a pool handed
# to the kernel as bytes.  Reading: e4m3 codes with one fp32 scale per row
# (value = code x scale, key and value dims alike).  The codes are decoded
# here with torch's float8_e4m3fn, independently of the oracle's decoder.


def _fp8_pool(seed, N, D, pow2):
    g = workloads.generator(seed)
    codes = workloads.fp8_codes(g, (N, D))
    if pow2:
        e = torch.randint(-12, 1, (N,), generator=g).to(torch.float32)
        scales = torch.pow(2.0, e)
    else:
        scales = workloads.fp8_scales(g, (N,))
    return codes.numpy(), scales.numpy()


def _dequant_torch(codes, scales):
    v = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64)
    return v * torch.from_numpy(scales.astype(np.float64))[:, None]


def test_fp8_pool_pow2_scales_equal_bf16_pool():
    """Power-of-two scales keep every value a bf16 number: the fp8 oracle
    equals the bf16 one on the pool holding those values, bit for bit."""
    T, H, dqk, dv, N, topk = 3, 16, 576, 512, 200, 48
    t = _inputs(20, T, H, dqk, dv, N, topk)
    codes, scales = _fp8_pool(21, N, dqk, pow2=True)
    vals = _dequant_torch(codes, scales)
    kv_bits = workloads.bits(vals.to(torch.bfloat16))
    assert np.array_equal(oracle.bf16_to_f64(kv_bits), vals.numpy())  # exact in bf16
    t["indices"][0, 5] = -1
    for sinks in (None, t["sinks"]):
        a, la = oracle.sparse_decode_attn_fp8(t["q"], codes, scales, t["indices"], sinks, 1 / 24, dv)
        b, lb = oracle.sparse_decode_attn(t["q"], kv_bits, t["indices"], None, sinks, 1 / 24, dv)
        assert np.array_equal(a, b) and np.array_equal(la, lb)


@pytest.mark.parametrize("with_sink", [False, True])
def test_fp8_pool_brute_force(with_sink):
    T, H, dqk, dv, N, topk = 2, 16, 576, 512, 150, 40
    t = _inputs(22, T, H, dqk, dv, N, topk)
    codes, scales = _fp8_pool(23, N, dqk, pow2=False)
    vals = _dequant_torch(codes, scales)
    scale = 1 / np.sqrt(dqk)
    sinks = t["sinks"] if with_sink else None
    out, lse = oracle.sparse_decode_attn_fp8(t["q"], codes, scales, t["indices"], sinks, scale, dv)
    for i in range(T):
        K = vals[t["indices"][i]]                                   # [n, dqk]
        s = (K @ _f(t["q"][i]).T) * scale                           # [n, H]
        ref_lse = torch.logsumexp(s, 0)
        p = torch.softmax(s, 0)
        o = p.T @ K[:, :dv]                                         # [H, dv]
        if sinks is not None:
            o = o / (1 + torch.exp(torch.from_numpy(sinks.astype(np.float64)) - ref_lse))[:, None]
        np.testing.assert_allclose(out[i], o.numpy(), rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[i], ref_lse.numpy(), rtol=0, atol=1e-12)


def test_fp8_pool_skips_negative_indices_and_neg_inf_sink():
    T, H, dqk, dv, N, topk = 2, 16, 576, 512, 80, 12
    t = _inputs(24, T, H, dqk, dv, N, topk)
    codes, scales = _fp8_pool(25, N, dqk, pow2=False)
    a, la = oracle.sparse_decode_attn_fp8(t["q"], codes, scales, t["indices"], None, 0.05, dv)
    b, lb = oracle.sparse_decode_attn_fp8(t["q"], codes, scales, t["indices"],
                                          np.full(H, -np.inf, np.float32), 0.05, dv)
    assert np.array_equal(a, b) and np.array_equal(la, lb)
    idx2 = t["indices"].copy()
    idx2[:, 3:] = -1
    c, _ = oracle.sparse_decode_attn_fp8(t["q"], codes, scales, idx2, None, 0.05, dv)
    d, _ = oracle.sparse_decode_attn_fp8(t["q"], codes, scales, np.ascontiguousarray(t["indices"][:, :3]),
                                         None, 0.05, dv)
    assert np.array_equal(c, d)
