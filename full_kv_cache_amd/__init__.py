"""Python binding of libhda, the hybrid decode-attention library for MI355X.

Argument marshalling only: every step of the path runs in the HIP kernels
behind the C ABI declared in ``include/hda.h``.  torch tensors supply
device memory and the stream; nothing is computed here, and there is no
CPU fallback -- if ``libhda.so`` is missing, every call raises.

Function names match the C entry points.  Tensors must be contiguous, on
the current GPU, with the dtypes the header states (bf16 as
``torch.bfloat16``, fp32, int32).
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from pathlib import Path
from typing import Optional

import torch

SLIDING = 0
FULL = 1
KV_BF16 = 0
KV_FP8_E4M3 = 1

_HERE = Path(__file__).resolve().parent
LIB_PATH = _HERE / "libhda.so"

HDA_OK = 0
_STATUS = {0: "HDA_OK", 1: "HDA_ERR_INVALID_ARGUMENT", 2: "HDA_ERR_UNSUPPORTED",
           3: "HDA_ERR_WORKSPACE", 4: "HDA_ERR_HIP"}


class HdaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


class CacheDesc(ctypes.Structure):
    """Mirror of ``hda_cache_desc``."""
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("rotary_dim", ctypes.c_int32),
        ("capacity", ctypes.c_int64),
        ("rope_theta", ctypes.c_double),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
        ("page_size", ctypes.c_int32),
        ("max_pages", ctypes.c_int32),
        ("num_pages", ctypes.c_int64),
        ("kv_dtype", ctypes.c_int32),
        ("k_scale", ctypes.c_void_p),
        ("v_scale", ctypes.c_void_p),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libhda.so (built by ``python -m full_kv_cache_amd.build``)."""
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m full_kv_cache_amd.build`")
        L = ctypes.CDLL(str(LIB_PATH))
        P, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        D = ctypes.POINTER(CacheDesc)
        L.hda_rope_append.restype = ctypes.c_int
        L.hda_rope_append.argtypes = [P, P, P, P, ctypes.c_int, D, P]
        L.hda_decode_workspace_bytes.restype = sz
        L.hda_decode_workspace_bytes.argtypes = [D, ctypes.c_int, i32, i32]
        L.hda_decode_attn.restype = ctypes.c_int
        L.hda_decode_attn.argtypes = [P, D, P, ctypes.c_int, P, P, ctypes.c_float, P, P, i32, i32,
                                      P, sz, P]
        L.hda_decode_split_plan.restype = ctypes.c_int
        L.hda_decode_split_plan.argtypes = [D, ctypes.c_int, i32, i32, ctypes.POINTER(i32),
                                            ctypes.POINTER(i32)]
        L.hda_decode_attn_partials.restype = ctypes.c_int
        L.hda_decode_attn_partials.argtypes = [P, D, P, ctypes.c_int, ctypes.c_float, i32, i32,
                                               P, P, P]
        L.hda_lse_merge.restype = ctypes.c_int
        L.hda_lse_merge.argtypes = [P, P, i32, i32, i32, i32, P, P, P, P, P]
        L.hda_status_string.restype = ctypes.c_char_p
        L.hda_status_string.argtypes = [ctypes.c_int]
        L.hda_last_error_message.restype = ctypes.c_char_p
        L.hda_last_error_message.argtypes = []
        L.hda_decode_step_workspace_bytes.restype = sz
        L.hda_decode_step_workspace_bytes.argtypes = [D, ctypes.c_int]
        L.hda_decode_step.restype = ctypes.c_int
        L.hda_decode_step.argtypes = [P, P, P, P, ctypes.c_int, D, P, P, ctypes.c_float, P, P, P, sz,
                                      P]
        L.hda_decode_step_noalloc.restype = ctypes.c_int
        L.hda_decode_step_noalloc.argtypes = [P, P, P, P, ctypes.c_int, D, P, P, ctypes.c_float, P, P,
                                              P]
        L.hda_decode_multi.restype = ctypes.c_int
        L.hda_decode_multi.argtypes = [P, P, P, P, i32, ctypes.c_int, D, P, P, ctypes.c_float, P,
                                       P, i32, P, sz, P]
        L.hda_decode_multi_workspace_bytes.restype = ctypes.c_size_t
        L.hda_decode_multi_workspace_bytes.argtypes = [D, ctypes.c_int, i32, i32]
        L.hda_sparse_workspace_bytes.restype = ctypes.c_size_t
        L.hda_sparse_workspace_bytes.argtypes = [i32, i32, i32, i32]
        L.hda_sparse_decode_attn.restype = ctypes.c_int
        L.hda_sparse_decode_attn.argtypes = [P, P, ctypes.c_int64, P, i32, i32, P, i32, i32, i32,
                                             P, ctypes.c_float, P, P, P, ctypes.c_size_t, P]
        L.hda_sparse_decode_attn_fp8.restype = ctypes.c_int
        L.hda_sparse_decode_attn_fp8.argtypes = [P, P, P, ctypes.c_int64, P, i32, i32, i32, i32, i32,
                                                 P, ctypes.c_float, P, P, P, ctypes.c_size_t, P]
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != HDA_OK:
        raise HdaError(status, lib().hda_last_error_message().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


@dataclass
class LayerCache:
    """One layer's KV cache tensors plus the shape facts of hda_cache_desc.

    k, v: bf16 [B, Hkv, capacity, D]; a sliding layer has capacity == window
    (window-1 ring slots, then the evicted-entry row).  Paged (full layers):
    block_table int32 [B, max_pages] and k, v page pools bf16 [num_pages, Hkv,
    page_size, D].  FP8: k, v uint8 e4m3 codes of the same shape, and
    k_scale, v_scale fp32 with one scale per row ([B, Hkv, capacity], paged
    [num_pages, Hkv, page_size]).
    """
    k: torch.Tensor
    v: torch.Tensor
    num_q_heads: int
    window: int
    rotary_dim: int
    rope_theta: float
    block_table: Optional[torch.Tensor] = None
    k_scale: Optional[torch.Tensor] = None
    v_scale: Optional[torch.Tensor] = None

    def _dtype_fields(self):
        if self.k.dtype == torch.bfloat16 and self.v.dtype == torch.bfloat16:
            if self.k_scale is not None or self.v_scale is not None:
                raise ValueError("scales belong to an fp8 (uint8) cache")
            return KV_BF16, None, None
        if self.k.dtype != torch.uint8 or self.v.dtype != torch.uint8:
            raise ValueError("k, v must both be bf16, or both uint8 e4m3 codes")
        rows = self.k.shape[:-1]
        for s in (self.k_scale, self.v_scale):
            if s is None or s.dtype != torch.float32 or not s.is_contiguous() or s.shape != rows:
                raise ValueError(f"an fp8 cache needs contiguous fp32 k_scale and v_scale of "
                                 f"shape {tuple(rows)}")
        return KV_FP8_E4M3, self.k_scale.data_ptr(), self.v_scale.data_ptr()

    def desc(self) -> CacheDesc:
        dt, ks, vs = self._dtype_fields()
        if self.block_table is None:
            B, Hkv, cap, D = self.k.shape
            return CacheDesc(B, self.num_q_heads, Hkv, D, self.window, self.rotary_dim, cap,
                             float(self.rope_theta), self.k.data_ptr(), self.v.data_ptr(),
                             None, 0, 0, 0, dt, ks, vs)
        if self.block_table.dtype != torch.int32 or not self.block_table.is_contiguous():
            raise ValueError("block_table must be a contiguous int32 tensor")
        num_pages, Hkv, page, D = self.k.shape
        B, max_pages = self.block_table.shape
        return CacheDesc(B, self.num_q_heads, Hkv, D, self.window, self.rotary_dim,
                         max_pages * page, float(self.rope_theta), self.k.data_ptr(),
                         self.v.data_ptr(), self.block_table.data_ptr(), page, max_pages,
                         num_pages, dt, ks, vs)


def hda_rope_append(q, k_new, v_new, pos, layer_type: int, cache: LayerCache, stream=None):
    """Rotate q in place, write the rotated new K and the new V into the cache."""
    d = cache.desc()
    _check(lib().hda_rope_append(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(pos), int(layer_type),
                                 ctypes.byref(d), _stream(stream)))


def hda_decode_workspace_bytes(cache: LayerCache, layer_type: int, max_seq_len: int,
                               chunk_keys: int = 0) -> int:
    d = cache.desc()
    return int(lib().hda_decode_workspace_bytes(ctypes.byref(d), int(layer_type),
                                                int(max_seq_len), int(chunk_keys)))


def validate_sinks(sinks: Optional[torch.Tensor], q: torch.Tensor) -> None:
    """The sink contract of the flashmla_sparse page (`_validate_sinks`,
    `_sinks_for_query`): fp32, shape (num_heads,), on q's device."""
    if sinks is None:
        return
    if sinks.dtype != torch.float32:
        raise ValueError(f"sinks must have dtype torch.float32, got {sinks.dtype}")
    heads = q.shape[1]
    if sinks.ndim != 1 or sinks.shape[0] != heads:
        raise ValueError(f"sinks must have shape ({heads},), got {tuple(sinks.shape)}")
    if sinks.device != q.device:
        raise ValueError(f"sinks and q must be on the same device, got {sinks.device} and {q.device}")


def validate_gate(gate: Optional[torch.Tensor], out: torch.Tensor) -> None:
    """Per-head output-gate logits (Spark export page, `_Layer.forward`: one
    g_proj value per query head): fp32, shape (batch, num_heads), on out's
    device, contiguous."""
    if gate is None:
        return
    if gate.dtype != torch.float32:
        raise ValueError(f"gate must have dtype torch.float32, got {gate.dtype}")
    want = tuple(out.shape[:2])
    if tuple(gate.shape) != want:
        raise ValueError(f"gate must have shape {want}, got {tuple(gate.shape)}")
    if gate.device != out.device:
        raise ValueError(f"gate and out must be on the same device, got {gate.device} and {out.device}")
    if not gate.is_contiguous():
        raise ValueError("gate must be contiguous")


def hda_decode_attn(q, cache: LayerCache, seq_lens, layer_type: int, sinks, scale: float, out,
                    lse=None, max_seq_len: int = 0, chunk_keys: int = 0, workspace=None,
                    stream=None, gate=None):
    """Decode attention of one layer (after hda_rope_append); gate: optional
    fp32 [B, Hq] output-gate logits."""
    validate_sinks(sinks, q)
    validate_gate(gate, out)
    d = cache.desc()
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().hda_decode_attn(_ptr(q), ctypes.byref(d), _ptr(seq_lens), int(layer_type),
                                 _ptr(sinks), _ptr(gate), float(scale), _ptr(out), _ptr(lse),
                                 int(max_seq_len), int(chunk_keys), _ptr(workspace), wbytes,
                                 _stream(stream)))


def hda_decode_split_plan(cache: LayerCache, layer_type: int, max_seq_len: int,
                          chunk_keys: int = 0) -> tuple[int, int]:
    """(keys per chunk, chunks per (sequence, KV head)) that hda_decode_attn uses."""
    d = cache.desc()
    c, n = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().hda_decode_split_plan(ctypes.byref(d), int(layer_type), int(max_seq_len),
                                       int(chunk_keys), ctypes.byref(c), ctypes.byref(n)))
    return c.value, n.value


def hda_decode_attn_partials(q, cache: LayerCache, seq_lens, layer_type: int, scale: float,
                             max_seq_len: int, chunk_keys: int, part_o, part_lse, stream=None):
    """Split-K stage alone: part_o fp32 [B,Hq,nsplit,D], part_lse fp32 [B,Hq,nsplit]."""
    d = cache.desc()
    _check(lib().hda_decode_attn_partials(_ptr(q), ctypes.byref(d), _ptr(seq_lens),
                                          int(layer_type), float(scale), int(max_seq_len),
                                          int(chunk_keys), _ptr(part_o), _ptr(part_lse),
                                          _stream(stream)))


def hda_lse_merge(part_o, part_lse, sinks, out, lse=None, stream=None, gate=None):
    """Merge partials [B,H,nsplit,D] / [B,H,nsplit] into out bf16 [B,H,D] (+ sink, gate)."""
    B, H, S, D = part_o.shape
    if sinks is not None:
        validate_sinks(sinks, out)
    validate_gate(gate, out)
    _check(lib().hda_lse_merge(_ptr(part_o), _ptr(part_lse), int(B), int(H), int(S), int(D),
                               _ptr(sinks), _ptr(gate), _ptr(out), _ptr(lse), _stream(stream)))


def hda_decode_step_workspace_bytes(cache: LayerCache, layer_type: int) -> int:
    d = cache.desc()
    return int(lib().hda_decode_step_workspace_bytes(ctypes.byref(d), int(layer_type)))


def hda_decode_step(q, k_new, v_new, pos, layer_type: int, cache: LayerCache, sinks, scale: float,
                    out, lse=None, workspace=None, stream=None, gate=None):
    """RoPE + append + attention of one layer in one launch (q is not modified).
    The workspace must be zero-filled before its first use; gate: optional
    fp32 [B, Hq] output-gate logits."""
    validate_sinks(sinks, q)
    validate_gate(gate, out)
    d = cache.desc()
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().hda_decode_step(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(pos), int(layer_type),
                                 ctypes.byref(d), _ptr(sinks), _ptr(gate), float(scale), _ptr(out),
                                 _ptr(lse),
                                 _ptr(workspace), wbytes, _stream(stream)))


def hda_decode_step_noalloc(q, k_new, v_new, pos, layer_type: int, cache: LayerCache, sinks,
                            scale: float, out, lse=None, stream=None, gate=None):
    """hda_decode_step with the library's static per-device scratch as its
    workspace (nothing allocated by the call); calls on one GPU must not
    overlap."""
    validate_sinks(sinks, q)
    validate_gate(gate, out)
    d = cache.desc()
    _check(lib().hda_decode_step_noalloc(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(pos),
                                         int(layer_type), ctypes.byref(d), _ptr(sinks), _ptr(gate),
                                         float(scale), _ptr(out), _ptr(lse), _stream(stream)))


def hda_decode_multi_workspace_bytes(cache: LayerCache, layer_type: int, tokens: int,
                                     max_seq_len: int) -> int:
    d = cache.desc()
    return int(lib().hda_decode_multi_workspace_bytes(ctypes.byref(d), int(layer_type),
                                                      int(tokens), int(max_seq_len)))


def hda_decode_multi(q, k_new, v_new, pos, layer_type: int, cache: LayerCache, sinks,
                     scale: float, out, lse=None, stream=None, gate=None, max_seq_len=None,
                     workspace=None):
    """Decode of a chunk of T (<= 512) new tokens per sequence: q [B, T, Hq, D]
    is rotated in place (as hda_rope_append does); k_new and v_new
    [B, T, Hkv, D] are only read; out [B, T, Hq, D], lse [B, T, Hq]; gate:
    optional fp32 [B, T, Hq] logits.  max_seq_len: host bound on pos + T
    (default: the cache capacity); workspace: hda_decode_multi_workspace_bytes()
    bytes of device memory (it holds the rotated new K)."""
    if q.dim() != 4:
        raise ValueError("q must be [B, T, Hq, D]")
    validate_sinks(sinks, q[:, 0])
    if gate is not None:
        validate_gate(gate.reshape(-1, gate.shape[-1]), out.reshape(-1, *out.shape[2:]))
    d = cache.desc()
    msl = int(d.capacity if max_seq_len is None else max_seq_len)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().hda_decode_multi(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(pos), int(q.shape[1]),
                                  int(layer_type), ctypes.byref(d), _ptr(sinks), _ptr(gate),
                                  float(scale), _ptr(out), _ptr(lse), msl, _ptr(workspace),
                                  wbytes, _stream(stream)))


def hda_sparse_workspace_bytes(tokens: int, num_q_heads: int, topk: int, dv: int = 512) -> int:
    return int(lib().hda_sparse_workspace_bytes(int(tokens), int(num_q_heads), int(topk), int(dv)))


def hda_sparse_decode_attn(q, kv, indices, topk_length, sinks, scale: float, out, lse=None,
                           workspace=None, stream=None):
    """Sparse top-k decode over one latent KV head shared by all query heads.

    q bf16 [T, Hq, Dqk]; kv bf16 [N, Dqk]; indices int32 [T, topk];
    topk_length int32 [T] or None; sinks fp32 [Hq] or None; out bf16
    [T, Hq, Dv] (Dv = out.shape[-1], the leading dims of each row)."""
    validate_sinks(sinks, q)
    T, H, dqk = q.shape
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().hda_sparse_decode_attn(_ptr(q), _ptr(kv), int(kv.shape[0]), _ptr(indices), int(T),
                                        int(indices.shape[1]), _ptr(topk_length), int(H), int(dqk),
                                        int(out.shape[-1]), _ptr(sinks), float(scale), _ptr(out),
                                        _ptr(lse), _ptr(workspace), wbytes, _stream(stream)))


def hda_sparse_decode_attn_fp8(q, kv_codes, kv_scales, indices, sinks, scale: float, out, lse=None,
                               workspace=None, stream=None):
    """Sparse top-k decode over an fp8 latent pool: kv_codes uint8 [N, Dqk]
    (e4m3), kv_scales fp32 [N] (a row's value is code x scale); q, indices,
    sinks, out, lse and workspace as hda_sparse_decode_attn."""
    validate_sinks(sinks, q)
    T, H, dqk = q.shape
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().hda_sparse_decode_attn_fp8(_ptr(q), _ptr(kv_codes), _ptr(kv_scales),
                                            int(kv_codes.shape[0]), _ptr(indices), int(T),
                                            int(indices.shape[1]), int(H), int(dqk), int(out.shape[-1]),
                                            _ptr(sinks), float(scale), _ptr(out), _ptr(lse),
                                            _ptr(workspace), wbytes, _stream(stream)))
