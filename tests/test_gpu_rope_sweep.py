"""GPU sweep of the RoPE evaluation through hda_rope_append: 4096 distinct
positions in [0, 40000] per call, for both RoPE configurations of the Spark
export page (rotary dim 256 with theta 1e4 -- sliding layers; rotary dim 64
with theta 5e6 -- full layers), on a 16-row sliding block (the append's
slot arithmetic as on a 512-row one).  Against the oracle's rope_append:
rotated q and the appended K within one bf16 ulp (or, where the rotation
cancels, within the fp32 rounding of the kernel's products) with fewer than
0.1% of values off, V and the evicted-entry row bit-exact, pass-through dims
bit-exact."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from hybrid_case import SLIDING, HybridCase, assert_rotated_close, bits_of

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("rot,theta", [(256, 1e4), (64, 5e6)])
def test_rope_append_position_sweep(rot, theta):
    import full_kv_cache_amd as hda
    print(f"CASE rope sweep rot={rot} theta={theta}", flush=True)
    rng = np.random.default_rng(rot)
    pos = rng.choice(40001, 4096, replace=False).astype(np.int32)
    case = HybridCase(4000 + rot, len(pos), SLIDING, pos, window=16)
    case.shape = dataclasses.replace(case.shape, rot_sliding=rot, theta_sliding=theta)
    s = case.shape
    h = {k: v.copy() for k, v in case.host.items()}
    k, v, kev, vev = case.to_oracle(h)
    oracle.rope_append(h["q"], h["k_new"], h["v_new"], case.pos, SLIDING, rot, theta, s.window,
                       k, v, kev, vev)
    kb, vb = case.from_oracle(k, v, kev, vev)
    d = case.device()
    hda.hda_rope_append(d["q"], d["k_new"], d["v_new"], torch.from_numpy(case.pos).cuda(), SLIDING,
                        case.cache(d))
    torch.cuda.synchronize()
    q = bits_of(d["q"])
    assert np.array_equal(q[..., rot:], h["q"][..., rot:])
    assert_rotated_close(q, h["q"], rot)
    assert np.array_equal(bits_of(d["v"]), vb)
    kg = bits_of(d["k"])
    bi = np.arange(len(pos))
    slot = pos % (s.window - 1)
    new_g, new_o = kg[bi, :, slot], kb[bi, :, slot]  # [B, Hkv, D]: the appended rows
    assert np.array_equal(new_g[..., rot:], new_o[..., rot:])
    assert_rotated_close(new_g, new_o, rot)
    kg[bi, :, slot] = kb[bi, :, slot]
    assert np.array_equal(kg, kb)  # every other row, the evicted-entry row included
