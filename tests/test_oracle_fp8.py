"""Pins for the oracle's FP8 KV cache (CPU only).

flashmla_sparse page, `_fp8_flash_mla_kernel`: the cache reaches the
kernel as raw bytes with an fp8 flag; the element format and scaling are
not printed.  Reading: e4m3 codes (bias 7, no infinities, S.1111.111 NaN,
largest finite 448), one fp32 scale per cached row, scale = amax / 448.
Pinned against what fixes them independently of the oracle's own code:
  * every one of the 256 codes decodes as torch's float8_e4m3fn does;
  * encoding agrees with torch's float8_e4m3fn cast on |x| <= 448,
    including every exact tie between neighbouring codes and the
    subnormal range; beyond 448 (where torch gives NaN) it saturates;
  * row quantization: the largest element maps to +-448, negation flips
    only sign bits, a zero row stays zero, the dequantized error is within
    half a code step, and codes equal torch's cast of x / scale;
  * the fp8 append equals the bf16 append followed by quantizing the
    written rows, eviction included;
  * attention over an fp8 cache whose values are bf16-representable
    (power-of-two scales) equals the bf16 oracle bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

FP8 = torch.float8_e4m3fn


def _torch_decode(codes):
    return torch.from_numpy(np.asarray(codes, dtype=np.uint8)).view(FP8).double().numpy()


def _torch_encode(x_f32):
    return torch.from_numpy(np.asarray(x_f32, dtype=np.float32)).to(FP8).view(torch.uint8).numpy()


def test_decode_every_code():
    ref = _torch_decode(np.arange(256))
    got = np.array([oracle.e4m3_to_f64(c) for c in range(256)])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))  # -0 is 0x80
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9


def _finite_values():
    v = np.array([oracle.e4m3_to_f64(c) for c in range(0x7F)])  # 0 .. 448, increasing
    assert np.all(np.diff(v) > 0)
    return v


def test_encode_matches_torch_including_ties():
    rng = np.random.default_rng(0)
    v = _finite_values()
    ties = (v[:-1] + v[1:]) / 2                          # exact midpoints
    near = np.concatenate([np.nextafter(ties.astype(np.float32), np.float32(0)),
                           np.nextafter(ties.astype(np.float32), np.float32(1e9))])
    rand = np.exp(rng.uniform(np.log(2.0 ** -12), np.log(448.0), 20000))
    x = np.concatenate([v, ties, near, rand, [2.0 ** -10, 3 * 2.0 ** -11]]).astype(np.float32)
    x = x[np.abs(x) <= 448]
    x = np.concatenate([x, -x])
    got = np.array([oracle.f32_to_e4m3(t) for t in x], dtype=np.uint8)
    assert np.array_equal(got, _torch_encode(x))


def test_encode_saturates_and_nan():
    for t, c in [(449.0, 0x7E), (464.0, 0x7E), (1e6, 0x7E), (float("inf"), 0x7E),
                 (-1e6, 0xFE), (float("-inf"), 0xFE)]:
        assert oracle.f32_to_e4m3(t) == c, t
    assert oracle.f32_to_e4m3(float("nan")) == 0x7F


def _bf16_rows(seed, shape):
    g = workloads.generator(seed)
    return workloads.bits(workloads.randn_bf16(g, shape))


def test_quant_rows_properties():
    x = _bf16_rows(1, (64, 256))
    codes, scales = oracle.quant_rows(x)
    xf = workloads.from_bits(x).double().numpy()
    amax = np.abs(xf).max(axis=1)
    i = np.abs(xf).argmax(axis=1)
    assert np.all(np.isin(codes[np.arange(64), i], [0x7E, 0xFE]))
    assert np.array_equal(scales, (amax.astype(np.float32) / np.float32(448.0)))
    # codes are torch's cast of the fp32 quotient
    q = (xf.astype(np.float32) / scales[:, None]).astype(np.float32)
    assert np.array_equal(codes, _torch_encode(q))
    # error within half a step: 2^-4 relative for normal codes, 2^-10 * scale below
    deq = oracle.dequant_rows(codes, scales)
    err = np.abs(deq - xf)
    bound = np.maximum(np.abs(xf) * 2.0 ** -4, scales[:, None].astype(np.float64) * 2.0 ** -10)
    assert np.all(err <= bound)
    # negation flips only the sign bits of nonzero codes
    cn, sn = oracle.quant_rows(x ^ np.uint16(0x8000))
    assert np.array_equal(sn, scales)
    nz = codes & 0x7F != 0
    assert np.array_equal(cn[nz], codes[nz] ^ 0x80)


def test_quant_zero_row():
    codes, scales = oracle.quant_rows(np.zeros((2, 256), np.uint16))
    assert np.all(codes == 0) and np.all(scales == 0)
    assert np.all(oracle.dequant_rows(codes, scales) == 0)


def _fp8_cache_from_bf16(k):
    c, s = oracle.quant_rows(k)
    return c, s


@pytest.mark.parametrize("lt,pos", [(workloads.SLIDING, [3, 510, 511, 1500]),
                                    (workloads.FULL, [0, 17, 200, 255])])
def test_fp8_append_is_bf16_append_then_quantize(lt, pos):
    W = 512
    shape = workloads.HybridShape(batch=len(pos), lmax=256)
    g = workloads.generator(7)
    t = {k: workloads.bits(v).copy() for k, v in workloads.layer_inputs(g, shape, lt).items()}
    pos = np.array(pos, np.int32)
    rot, theta = shape.rot(lt), shape.theta(lt)
    B, Hkv, cap, D = t["k"].shape
    if lt == workloads.SLIDING:
        k, v = t["k"][:, :, :W - 1].copy(), t["v"][:, :, :W - 1].copy()
        kev, vev = t["k"][:, :, W - 1].copy(), t["v"][:, :, W - 1].copy()
    else:
        k, v = t["k"].copy(), t["v"].copy()
        kev = np.zeros((B, Hkv, D), np.uint16)
        vev = kev.copy()
    # fp8 side: the starting cache quantized row by row
    kc, ks = _fp8_cache_from_bf16(k)
    vc, vs = _fp8_cache_from_bf16(v)
    kevc, kevs = _fp8_cache_from_bf16(kev)
    vevc, vevs = _fp8_cache_from_bf16(vev)
    kc0, ks0 = kc.copy(), ks.copy()
    q8 = t["q"].copy()
    oracle.rope_append_fp8(q8, t["k_new"], t["v_new"], pos, lt, rot, theta, W, kc, vc, ks, vs,
                           kevc, vevc, kevs, vevs)
    # bf16 side, then quantize the rows it wrote
    q16 = t["q"].copy()
    oracle.rope_append(q16, t["k_new"], t["v_new"], pos, lt, rot, theta, W, k, v, kev, vev)
    assert np.array_equal(q8, q16)
    for b, p in enumerate(pos):
        row = p % (W - 1) if lt == workloads.SLIDING else p
        ck, sk = oracle.quant_rows(k[b, :, row])
        cv, sv = oracle.quant_rows(v[b, :, row])
        assert np.array_equal(kc[b, :, row], ck) and np.array_equal(ks[b, :, row], sk)
        assert np.array_equal(vc[b, :, row], cv) and np.array_equal(vs[b, :, row], sv)
        if lt == workloads.SLIDING and p >= W - 1:  # side row = the slot's prior content
            assert np.array_equal(kevc[b], kc0[b, :, row]) and np.array_equal(kevs[b], ks0[b, :, row])
        others = np.ones(kc.shape[2], bool)
        others[row] = False
        assert np.array_equal(kc[b][:, others], kc0[b][:, others])


@pytest.mark.parametrize("lt", [workloads.SLIDING, workloads.FULL])
def test_fp8_attention_equals_bf16_when_exact(lt):
    """Power-of-two scales keep every dequantized value a bf16 value."""
    W, B, Hkv, D = 512, 3, 2, 256
    cap = W - 1 if lt == workloads.SLIDING else 300
    rng = np.random.default_rng(3)
    finite = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    kc = rng.choice(finite, size=(B, Hkv, cap, D))
    vc = rng.choice(finite, size=(B, Hkv, cap, D))
    ks = (2.0 ** rng.integers(-9, -4, size=(B, Hkv, cap))).astype(np.float32)
    vs = (2.0 ** rng.integers(-9, -4, size=(B, Hkv, cap))).astype(np.float32)
    kevc, vevc = kc[:, :, 0].copy(), vc[:, :, 1].copy()
    kevs, vevs = ks[:, :, 5].copy(), vs[:, :, 6].copy()
    q = _bf16_rows(4, (B, 8, D))
    seq = np.array([1, 200, 300] if lt == workloads.FULL else [1, 511, 900], np.int32)
    sinks = np.linspace(-2, 2, 8).astype(np.float32)
    to_bf16 = np.vectorize(oracle.f64_to_bf16_scalar, otypes=[np.uint16])
    k16 = to_bf16(oracle.dequant_rows(kc, ks))
    v16 = to_bf16(oracle.dequant_rows(vc, vs))
    kev16 = to_bf16(oracle.dequant_rows(kevc, kevs))
    vev16 = to_bf16(oracle.dequant_rows(vevc, vevs))
    assert np.array_equal(workloads.from_bits(k16).double().numpy(), oracle.dequant_rows(kc, ks))
    o8, l8 = oracle.decode_attn_fp8(q, kc, vc, ks, vs, kevc, vevc, kevs, vevs, seq, lt, W, sinks,
                                    1 / 16)
    o16, l16 = oracle.decode_attn(q, k16, v16, kev16, vev16, seq, lt, W, sinks, 1 / 16)
    assert np.array_equal(o8, o16) and np.array_equal(l8, l16)
