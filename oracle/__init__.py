"""CPU oracle for hybrid decode attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline
leg may import this package.  The product path (``full_kv_cache_amd``)
never imports, links or calls it, and shares no code with it.

The arithmetic lives in ``oracle.c`` (plain C, fp64); this module builds it
with gcc and marshals numpy arrays through ctypes.  bf16 tensors travel as
``numpy.uint16`` bit patterns.

Parity status: every exported function is pinned by the ``-m "not gpu"``
tests listed in its C header comment; none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "oracle.c"
_LIB = _HERE / "liboracle.so"

SLIDING = 0
FULL = 1

_lib = None


def build(force: bool = False) -> Path:
    """Compile ``oracle.c`` into ``liboracle.so`` with gcc and OpenMP."""
    if force or not _LIB.exists() or _LIB.stat().st_mtime < _SRC.stat().st_mtime:
        tmp = _LIB.with_suffix(".so.tmp%d" % os.getpid())
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
             "-Wall", "-Wextra", "-o", str(tmp), str(_SRC), "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        # HDA_ORACLE_LIB: a build of oracle.c made elsewhere (the sanitizer
        # test loads an AddressSanitizer / UBSan build this way)
        path = os.environ.get("HDA_ORACLE_LIB")
        if not path:
            path = str(build())
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        lib.or_bf16_to_f64.restype = f64
        lib.or_bf16_to_f64.argtypes = [ctypes.c_uint16]
        lib.or_f64_to_bf16.restype = ctypes.c_uint16
        lib.or_f64_to_bf16.argtypes = [f64]
        lib.or_cache_len.restype = i64
        lib.or_cache_len.argtypes = [i32, i64, i32, i32]
        lib.or_kv_cache_bytes.restype = None
        lib.or_kv_cache_bytes.argtypes = [P, i32, i64, i32, i32, i32, i32, i32, P]
        lib.or_ring_slot.restype = i64
        lib.or_ring_slot.argtypes = [i64, i32]
        lib.or_rope_angles.restype = None
        lib.or_rope_angles.argtypes = [f64, i32, i64, P, P]
        lib.or_rope_apply.restype = None
        lib.or_rope_apply.argtypes = [P, P, i64, i32, i32, f64, i64]
        lib.or_rope_append.restype = None
        lib.or_rope_append.argtypes = [P, P, P, P, i32, i32, i32, i32, i32, i32, f64,
                                       i32, i64, P, P, P, P]
        lib.or_decode_attn.restype = None
        lib.or_decode_attn.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, i32, i32,
                                       i64, P, f64, P, P]
        lib.or_attn_chunk.restype = None
        lib.or_attn_chunk.argtypes = [P, P, P, i64, i64, i32, f64, P, P]
        lib.or_lse_merge.restype = None
        lib.or_lse_merge.argtypes = [P, P, i32, i32, P, P, P]
        lib.or_output_gate.restype = None
        lib.or_output_gate.argtypes = [P, i32, i32, i32, P]
        lib.or_e4m3_to_f64.restype = f64
        lib.or_e4m3_to_f64.argtypes = [ctypes.c_uint8]
        lib.or_f32_to_e4m3.restype = ctypes.c_uint8
        lib.or_f32_to_e4m3.argtypes = [ctypes.c_float]
        lib.or_quant_rows.restype = None
        lib.or_quant_rows.argtypes = [P, i64, i32, P, P]
        lib.or_dequant_rows.restype = None
        lib.or_dequant_rows.argtypes = [P, P, i64, i32, P]
        lib.or_rope_append_fp8.restype = None
        lib.or_rope_append_fp8.argtypes = [P, P, P, P, i32, i32, i32, i32, i32, i32, f64, i32,
                                           i64, P, P, P, P, P, P, P, P]
        lib.or_decode_attn_f64.restype = None
        lib.or_decode_attn_f64.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, i32, i32,
                                           i64, P, f64, P, P]
        lib.or_page_gather.restype = None
        lib.or_page_gather.argtypes = [P, P, i32, i32, i32, i32, i32, i64, P]
        lib.or_sparse_decode_attn.restype = None
        lib.or_sparse_decode_attn.argtypes = [P, P, i64, P, i32, P, i32, i32, i32, i32,
                                              P, f64, P, P]
        lib.or_sparse_decode_attn_fp8.restype = None
        lib.or_sparse_decode_attn_fp8.argtypes = [P, P, P, i64, P, i32, i32, i32, i32, i32,
                                                  P, f64, P, P]
        lib.or_num_threads.restype = ctypes.c_int
        lib.or_num_threads.argtypes = []
        _lib = lib
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _u16(a):
    a = np.ascontiguousarray(a)
    assert a.dtype == np.uint16, a.dtype
    return a


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def _f32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float32)


# ---------------------------------------------------------------- scalars

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (vectorised, same rule as C)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16_scalar(x: float) -> int:
    return int(_load().or_f64_to_bf16(float(x)))


def cache_len(layer_type: int, context: int, window: int, ring: bool) -> int:
    return int(_load().or_cache_len(layer_type, context, window, int(ring)))


def kv_cache_bytes(layer_types, context, window, ring, kv_heads, head_dim, bytes_per_elem=2):
    lt = _i32(layer_types)
    out = np.zeros(2, dtype=np.int64)
    _load().or_kv_cache_bytes(_p(lt), len(lt), context, window, int(ring), kv_heads,
                              head_dim, bytes_per_elem, _p(out))
    return {"hybrid": int(out[0]), "uniform": int(out[1])}


def ring_slot(pos: int, window: int) -> int:
    return int(_load().or_ring_slot(pos, window))


def num_threads() -> int:
    return int(_load().or_num_threads())


# ------------------------------------------------------------------ RoPE

def rope_angles(theta: float, rot: int, pos: int):
    c = np.zeros(rot // 2, dtype=np.float32)
    s = np.zeros(rot // 2, dtype=np.float32)
    _load().or_rope_angles(theta, rot, pos, _p(c), _p(s))
    return c, s


def rope_apply(x_bits: np.ndarray, rot: int, theta: float, pos: int) -> np.ndarray:
    """bf16 bits [..., D] -> rotated bf16 bits [..., D]."""
    x = _u16(x_bits)
    D = x.shape[-1]
    y = np.empty_like(x)
    _load().or_rope_apply(_p(x), _p(y), x.size // D, D, rot, theta, pos)
    return y


def rope_append(q, k_new, v_new, pos, layer_type, rot, theta, window, k, v, kev, vev):
    """In place on numpy copies: q [B,Hq,D], k/v [B,Hkv,cap,D], kev/vev [B,Hkv,D]."""
    for a in (q, k, v, kev, vev):
        assert a.dtype == np.uint16 and a.flags.c_contiguous
    k_new, v_new, pos = _u16(k_new), _u16(v_new), _i32(pos)
    B, Hq, D = q.shape
    Hkv, cap = k.shape[1], k.shape[2]
    _load().or_rope_append(_p(q), _p(k_new), _p(v_new), _p(pos), layer_type, B, Hq, Hkv,
                           D, rot, theta, window, cap, _p(k), _p(v), _p(kev), _p(vev))


# ------------------------------------------------------------- attention

def decode_attn(q, k, v, kev, vev, seq_lens, layer_type, window, sinks, scale, gate=None):
    """Returns (out fp64 [B,Hq,D], lse fp64 [B,Hq]).  gate: fp32 [B,Hq] logits
    of the per-head output gate, or None."""
    q, k, v = _u16(q), _u16(k), _u16(v)
    kev = _u16(kev) if kev is not None else None
    vev = _u16(vev) if vev is not None else None
    seq_lens = _i32(seq_lens)
    sinks = _f32(sinks)
    B, Hq, D = q.shape
    Hkv, cap = k.shape[1], k.shape[2]
    out = np.zeros((B, Hq, D), dtype=np.float64)
    lse = np.zeros((B, Hq), dtype=np.float64)
    _load().or_decode_attn(_p(q), _p(k), _p(v), _p(kev), _p(vev), _p(seq_lens), layer_type,
                           B, Hq, Hkv, D, window, cap, _p(sinks), scale, _p(out), _p(lse))
    if gate is not None:
        output_gate(out, gate)
    return out, lse


def output_gate(out, gate):
    """In place: out fp64 [B,Hq,D] times the sigmoid of gate fp32 [B,Hq]."""
    assert out.dtype == np.float64 and out.flags.c_contiguous
    gate = _f32(gate)
    B, Hq, D = out.shape
    assert gate.shape == (B, Hq)
    _load().or_output_gate(_p(out), B, Hq, D, _p(gate))


# ------------------------------------------------------ multi-token decode

def decode_multi(q, k_new, v_new, pos, layer_type, rot, theta, window, k, v, kev, vev, sinks,
                 scale, gate=None):
    """A chunk of T new tokens per sequence (q [B,T,Hq,D], k_new / v_new
    [B,T,Hkv,D], bf16 bits; pos [B] = position of token 0).  Spark export
    page, `SparkStepConfig.cache_len` docstring: a ring holds the window's
    previous entries and the new token is scored with them, so a chunk
    means token t attends to what is cached in its window plus new tokens
    0..t -- the plain definition is T single-token decode steps in order:
    step t appends token t at pos + t (or_rope_append) and attends with
    seq_len pos + t + 1 (or_decode_attn).  The cache (oracle form: k, v
    [B,Hkv,cap,D], side rows kev, vev [B,Hkv,D]) is updated in place and q
    is rotated in place, as the single-token functions do.
    gate: fp32 [B,T,Hq] logits or None.  Returns out fp64 [B,T,Hq,D], lse
    fp64 [B,T,Hq]."""
    assert q.dtype == np.uint16 and q.flags.c_contiguous and q.ndim == 4
    B, T, Hq, D = q.shape
    pos = _i32(pos)
    out = np.zeros((B, T, Hq, D), dtype=np.float64)
    lse = np.zeros((B, T, Hq), dtype=np.float64)
    for t in range(T):
        qt = np.ascontiguousarray(q[:, t])
        rope_append(qt, np.ascontiguousarray(k_new[:, t]), np.ascontiguousarray(v_new[:, t]),
                    pos + t, layer_type, rot, theta, window, k, v, kev, vev)
        q[:, t] = qt
        g = None if gate is None else np.ascontiguousarray(np.asarray(gate)[:, t])
        out[:, t], lse[:, t] = decode_attn(qt, k, v, kev, vev, pos + t + 1, layer_type, window,
                                           sinks, scale, gate=g)
    return out, lse


# ------------------------------------------------------------- FP8 KV

def e4m3_to_f64(code: int) -> float:
    return _load().or_e4m3_to_f64(int(code))


def f32_to_e4m3(x: float) -> int:
    return int(_load().or_f32_to_e4m3(float(x)))


def quant_rows(x_bits):
    """bf16 bits [..., D] -> (codes uint8 [..., D], scales fp32 [...])."""
    x = _u16(x_bits)
    D = x.shape[-1]
    rows = x.size // D
    codes = np.zeros(x.shape, dtype=np.uint8)
    scales = np.zeros(x.shape[:-1], dtype=np.float32)
    _load().or_quant_rows(_p(x), rows, D, _p(codes), _p(scales))
    return codes, scales


def dequant_rows(codes, scales):
    """codes uint8 [..., D], scales fp32 [...] -> fp64 [..., D]."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = _f32(scales)
    D = codes.shape[-1]
    out = np.zeros(codes.shape, dtype=np.float64)
    _load().or_dequant_rows(_p(codes), _p(scales), codes.size // D, D, _p(out))
    return out


def rope_append_fp8(q, k_new, v_new, pos, layer_type, rot, theta, window, kc, vc, ks, vs,
                    kevc, vevc, kevs, vevs):
    """In place on numpy copies: q bf16 [B,Hq,D]; codes kc/vc uint8 [B,Hkv,cap,D],
    scales ks/vs fp32 [B,Hkv,cap]; side rows kevc/vevc uint8 [B,Hkv,D],
    kevs/vevs fp32 [B,Hkv]."""
    assert q.dtype == np.uint16 and q.flags.c_contiguous
    for a in (kc, vc, kevc, vevc):
        assert a.dtype == np.uint8 and a.flags.c_contiguous
    for a in (ks, vs, kevs, vevs):
        assert a.dtype == np.float32 and a.flags.c_contiguous
    k_new, v_new, pos = _u16(k_new), _u16(v_new), _i32(pos)
    B, Hq, D = q.shape
    Hkv, cap = kc.shape[1], kc.shape[2]
    _load().or_rope_append_fp8(_p(q), _p(k_new), _p(v_new), _p(pos), layer_type, B, Hq, Hkv, D,
                               rot, theta, window, cap, _p(kc), _p(vc), _p(ks), _p(vs),
                               _p(kevc), _p(vevc), _p(kevs), _p(vevs))


def decode_attn_f64(q, k, v, kev, vev, seq_lens, layer_type, window, sinks, scale, gate=None):
    """decode_attn over fp64 K/V values [B,Hkv,cap,D] (+ side rows [B,Hkv,D])."""
    q = _u16(q)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    kev = None if kev is None else np.ascontiguousarray(kev, dtype=np.float64)
    vev = None if vev is None else np.ascontiguousarray(vev, dtype=np.float64)
    seq_lens, sinks = _i32(seq_lens), _f32(sinks)
    B, Hq, D = q.shape
    Hkv, cap = k.shape[1], k.shape[2]
    out = np.zeros((B, Hq, D), dtype=np.float64)
    lse = np.zeros((B, Hq), dtype=np.float64)
    _load().or_decode_attn_f64(_p(q), _p(k), _p(v), _p(kev), _p(vev), _p(seq_lens), layer_type,
                               B, Hq, Hkv, D, window, cap, _p(sinks), scale, _p(out), _p(lse))
    if gate is not None:
        output_gate(out, gate)
    return out, lse


def decode_attn_fp8(q, kc, vc, ks, vs, kevc, vevc, kevs, vevs, seq_lens, layer_type, window,
                    sinks, scale, gate=None):
    """Attention over an fp8 cache: every row dequantized (value = e4m3
    code x row scale), then decode_attn_f64."""
    k, v = dequant_rows(kc, ks), dequant_rows(vc, vs)
    kev = None if kevc is None else dequant_rows(kevc, kevs)
    vev = None if vevc is None else dequant_rows(vevc, vevs)
    return decode_attn_f64(q, k, v, kev, vev, seq_lens, layer_type, window, sinks, scale, gate)


def page_gather(pool, block_table):
    """Paged pool bf16 [num_pages, Hkv, page_size, D] + block_table int32
    [B, max_pages] -> contiguous bf16 [B, Hkv, max_pages*page_size, D]."""
    pool, bt = _u16(pool), _i32(block_table)
    num_pages, Hkv, page_size, D = pool.shape
    B, max_pages = bt.shape
    out = np.zeros((B, Hkv, max_pages * page_size, D), dtype=np.uint16)
    _load().or_page_gather(_p(pool), _p(bt), B, Hkv, D, page_size, max_pages, num_pages,
                           _p(out))
    return out


def attn_chunk(qh, kblk, vblk, r0, r1, scale):
    qh, kblk, vblk = _u16(qh), _u16(kblk), _u16(vblk)
    D = qh.shape[-1]
    out = np.zeros(D, dtype=np.float64)
    lse = np.zeros(1, dtype=np.float64)
    _load().or_attn_chunk(_p(qh), _p(kblk), _p(vblk), r0, r1, D, scale, _p(out), _p(lse))
    return out, float(lse[0])


def lse_merge(o_parts, lse_parts, sink=None, gate=None):
    o_parts = np.ascontiguousarray(o_parts, dtype=np.float64)
    lse_parts = np.ascontiguousarray(lse_parts, dtype=np.float64)
    S, D = o_parts.shape
    out = np.zeros(D, dtype=np.float64)
    lse = np.zeros(1, dtype=np.float64)
    sk = None if sink is None else np.array([sink], dtype=np.float32)
    _load().or_lse_merge(_p(o_parts), _p(lse_parts), S, D, _p(sk), _p(out), _p(lse))
    if gate is not None:
        output_gate(out.reshape(1, 1, D), np.array([[gate]], dtype=np.float32))
    return out, float(lse[0])


def sparse_decode_attn(q, kv, indices, topk_length, sinks, scale, dv):
    """q bf16 [T,Hq,Dqk], kv bf16 [N,Dqk], indices int32 [T,topk]."""
    q, kv, indices = _u16(q), _u16(kv), _i32(indices)
    tl = None if topk_length is None else _i32(topk_length)
    sinks = _f32(sinks)
    T, Hq, Dqk = q.shape
    N = kv.shape[0]
    topk = indices.shape[1]
    out = np.zeros((T, Hq, dv), dtype=np.float64)
    lse = np.zeros((T, Hq), dtype=np.float64)
    _load().or_sparse_decode_attn(_p(q), _p(kv), N, _p(indices), topk, _p(tl), T, Hq, Dqk,
                                  dv, _p(sinks), scale, _p(out), _p(lse))
    return out, lse


def sparse_decode_attn_fp8(q, codes, scales, indices, sinks, scale, dv):
    """q bf16 [T,Hq,Dqk], codes uint8 [N,Dqk] (e4m3), scales fp32 [N],
    indices int32 [T,topk]; a row's value is code x scale."""
    q, indices = _u16(q), _i32(indices)
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = _f32(scales)
    sinks = _f32(sinks)
    T, Hq, Dqk = q.shape
    N = codes.shape[0]
    topk = indices.shape[1]
    out = np.zeros((T, Hq, dv), dtype=np.float64)
    lse = np.zeros((T, Hq), dtype=np.float64)
    _load().or_sparse_decode_attn_fp8(_p(q), _p(codes), _p(scales), N, _p(indices), topk, T, Hq,
                                      Dqk, dv, _p(sinks), scale, _p(out), _p(lse))
    return out, lse
