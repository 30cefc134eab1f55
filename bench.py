#!/usr/bin/env python3
"""Decode-attention throughput of the hybrid model on one MI355X.

One step is one decode step of the attention path for a whole batch: for
each of the 28 layers (21 sliding with a 512-token window held as a
512-row block -- 511 ring slots plus the evicted-entry row -- and 7 full;
layer i is full when i % 4 == 3)

    hda_rope_append  -- rotate q in place, write the rotated new K and V
                        into the ring slot (sliding) or row pos (full);
    hda_decode_attn  -- GQA attention over the layer's keys with a per-head
                        sink: balanced streaming kernel plus the LSE merge
    (--path fused: hda_decode_step, the same step in one call -- one launch
    for a sliding layer, the streaming kernel in its step form plus the
    merge, which scores and appends the new token, for a full layer; --path
    auto, the default: the faster of the two per layer type, measured on
    MI355X -- hda_decode_step for both).

Each timed step re-appends at the same positions; the rows read and the
work done are those of one decode step either way.

Every layer has its own cache, so a step streams the whole resident KV
(about 5.2 GB at the default shape), far more than the 256 MB last-level
cache: nothing is served from cache between steps.  Inputs are synthetic
(seeded, unit-normal bf16), already resident in HBM when timing starts.

Reported: KV GB/s (attended K and V bytes per step / step time), its
fraction of the 8 TB/s HBM peak, decode tokens/s (batch / step time), a
roofline entry for the dominant kernel and the CPU oracle's rate on a
bounded sample of the same workload; also the same step with the per-head
output gate (Spark export page, `_Layer.forward`) applied in every
attention epilogue (gated_ms_per_step), and the same step with every full
layer's cache held in a shuffled pool of 64-row pages read through a block
table (flashmla_sparse page, `_fp8_flash_mla_kernel`; paged_ms_per_step and
the paged full-layer kernel in "paged"), and the same step on an FP8 KV
cache -- e4m3 codes with one fp32 scale per row, quantized on append, the
reading of that page's fp8 call -- in "fp8"; and chunks of 4 new tokens
per sequence through hda_decode_multi on every layer (Spark export page,
`SparkStepConfig.cache_len` docstring: each token attends to its own
window) in "multi"; chunked prefill of 256 tokens into the first 8
sequences' caches on every layer (the prefill kernel: both products on the
matrix cores) in "prefill"; the batch-1 28-layer step at context 4096 in
"step28" and the batch-16 step at context 32768 in "long" (graph and eager,
with their layer kernels' rooflines).  Step times are the median of 5
windows of the timed steps; the line also records the device, ROCm version,
clocks and host CPU model.

    python bench.py [--steps K] [--warmup W] [--config throughput|step28|long|tiny]
                    [--path auto|fused|separate]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "decode-attn KV GB/s (% HBM peak) + tokens/s, batch 64 at 4k context"

CONFIGS = {
    # name: (batch, seq_len spec, lmax, n_layers, description)
    "throughput": dict(batch=64, lo=512, hi=4096, lmax=4096, layers=28,
                       desc="batch 64, context lengths uniform in [512, 4096], 28 layers "
                            "(21 sliding window 512 + 7 full), 8 q / 2 KV heads, head_dim 256, "
                            "bf16, per-head sinks"),
    "step28": dict(batch=1, lo=4096, hi=4096, lmax=4096, layers=28,
                   desc="batch 1 at context 4096, 28 layers (21 sliding + 7 full)"),
    "long": dict(batch=16, lo=32768, hi=32768, lmax=32768, layers=28,
                 desc="batch 16 at context 32768, 28 layers (21 sliding + 7 full)"),
    "tiny": dict(batch=1, lo=1024, hi=1024, lmax=1024, layers=2,
                 desc="batch 1 at position 1023, one sliding and one full layer"),
}


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="throughput", choices=sorted(CONFIGS))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead of a HIP graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sparse", action="store_true", help="skip the sparse top-k measurement")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum oracle time for the CPU baseline sample")
    ap.add_argument("--chunk-keys", type=int, default=0,
                    help="split size for full layers on the separate path (0: default)")
    ap.add_argument("--path", default="auto", choices=["auto", "fused", "separate"],
                    help="one launch per layer (hda_decode_step) or rope_append + decode_attn")
    ap.add_argument("--page-size", type=int, default=64,
                    help="rows per page of the paged full-layer measurement (0: skip it)")
    ap.add_argument("--no-fp8", action="store_true", help="skip the fp8-cache measurement")
    ap.add_argument("--multi-tokens", type=int, default=4,
                    help="tokens per chunk of the chunk-decode measurement (0: skip it)")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip the batch-1 and 16 x 32k step measurements")
    ap.add_argument("--prefill-tokens", type=int, default=256,
                    help="tokens per chunk of the chunked-prefill measurement (0: skip it)")
    ap.add_argument("--prefill-batch", type=int, default=8,
                    help="sequences of the chunked-prefill measurement")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MB",
                    help="only run a plain device copy of this many MB (PMC byte calibration)")
    return ap.parse_args()


def layer_types(n):
    import workloads
    return workloads.layer_pattern(n) if n != 2 else [workloads.SLIDING, workloads.FULL]


class Workload:
    """All layers' tensors for one configuration, resident on the GPU."""

    def __init__(self, cfg: dict, seed: int, dev="cuda"):
        import torch
        import workloads
        import full_kv_cache_amd as hda

        self.cfg = cfg
        B = cfg["batch"]
        self.shape = workloads.HybridShape(batch=B, lmax=cfg["lmax"])
        g = workloads.generator(seed, dev)
        self.seq_lens = workloads.uniform_seq_lens(g, B, cfg["lo"], cfg["hi"], dev)
        self.pos = (self.seq_lens - 1).contiguous()
        self.max_seq_len = int(self.seq_lens.max().item())
        self.types = layer_types(cfg["layers"])
        self.layers = []
        s = self.shape
        for lt in self.types:
            t = workloads.layer_inputs(g, s, lt, dev)
            cache = hda.LayerCache(t["k"], t["v"], s.num_q_heads, s.window, s.rot(lt), s.theta(lt))
            self.layers.append(dict(
                lt=lt, q=t["q"], k_new=t["k_new"], v_new=t["v_new"], cache=cache, raw=t,
                sinks=workloads.sinks(g, s.num_q_heads, dev),
                out=torch.empty(B, s.num_q_heads, s.head_dim, dtype=torch.bfloat16, device=dev),
                lse=torch.empty(B, s.num_q_heads, dtype=torch.float32, device=dev)))
        # output-gate logits from a generator of their own (the draws above
        # stay what they were)
        gg = workloads.generator(seed + 2, dev)
        for L in self.layers:
            L["gate"] = workloads.gate_logits(gg, B, s.num_q_heads, dev)
        self.scale = 1.0 / s.head_dim ** 0.5
        ws = max(max(hda.hda_decode_workspace_bytes(L["cache"], L["lt"], self.max_seq_len, 0),
                     hda.hda_decode_step_workspace_bytes(L["cache"], L["lt"])) for L in self.layers)
        self.workspace = torch.zeros(max(ws, 256), dtype=torch.uint8, device=dev)  # counters start at 0
        sl = self.seq_lens.cpu().long()
        self.kv_row_bytes = 2 * s.num_kv_heads * s.head_dim * 2  # K and V, all KV heads, bf16
        self.rows = {lt: int((sl.clamp(max=s.window) if lt == workloads.SLIDING else sl).sum())
                     for lt in (workloads.SLIDING, workloads.FULL)}
        self.kv_bytes = sum(self.rows[lt] for lt in self.types) * self.kv_row_bytes

    def make_paged(self, page_size, seed):
        """Give every full layer a paged copy of its cache: the blocks cut
        into page_size-row pages, scattered over a pool in a random order,
        and a block table [B, max_pages] naming them."""
        import torch
        import workloads
        import full_kv_cache_amd as hda
        s, B = self.shape, self.cfg["batch"]
        cap = s.capacity(workloads.FULL)
        assert cap % page_size == 0, "capacity must be a whole number of pages"
        mp = cap // page_size
        g = torch.Generator().manual_seed(seed + 3)
        for L in self.layers:
            if L["lt"] != workloads.FULL:
                continue
            perm = torch.randperm(B * mp, generator=g).to(L["raw"]["k"].device)
            pools = []
            for blk in (L["cache"].k, L["cache"].v):
                pages = blk.view(B, s.num_kv_heads, mp, page_size, s.head_dim).permute(0, 2, 1, 3, 4)
                pool = torch.empty((B * mp, s.num_kv_heads, page_size, s.head_dim),
                                   dtype=blk.dtype, device=blk.device)
                pool[perm] = pages.reshape(B * mp, s.num_kv_heads, page_size, s.head_dim)
                pools.append(pool)
            table = perm.view(B, mp).to(torch.int32).contiguous()
            L["pcache"] = hda.LayerCache(pools[0], pools[1], s.num_q_heads, s.window,
                                         s.rot(workloads.FULL), s.theta(workloads.FULL),
                                         block_table=table)

    def make_fp8(self, seed):
        """Give every layer an fp8 cache of the same shape: seeded random
        e4m3 codes (never NaN) and per-row scales in [1, 2) / 448."""
        import torch
        import workloads
        import full_kv_cache_amd as hda
        s = self.shape
        g = workloads.generator(seed + 4, self.seq_lens.device)
        for L in self.layers:
            c = L["cache"]
            shp = tuple(c.k.shape)
            L["fcache"] = hda.LayerCache(
                workloads.fp8_codes(g, shp, c.k.device), workloads.fp8_codes(g, shp, c.k.device),
                s.num_q_heads, s.window, c.rotary_dim, c.rope_theta,
                k_scale=workloads.fp8_scales(g, shp[:-1], c.k.device),
                v_scale=workloads.fp8_scales(g, shp[:-1], c.k.device))
        self.fp8_row_bytes = 2 * s.num_kv_heads * (s.head_dim + 4)  # K and V codes + scales
        need = max(hda.hda_decode_workspace_bytes(L["fcache"], L["lt"], self.max_seq_len, 0)
                   for L in self.layers)
        if need > self.workspace.numel():
            self.workspace = torch.zeros(need, dtype=torch.uint8, device=self.workspace.device)

    def make_multi(self, T, seed):
        """Chunk inputs for every layer: q [B,T,Hq,D], k_new / v_new
        [B,T,Hkv,D], out [B,T,Hq,D]; token 0 at seq_len - T, so the last
        token of a chunk attends to as many keys as the one-token step."""
        import torch
        import workloads
        s, B = self.shape, self.cfg["batch"]
        g = workloads.generator(seed + 5, self.seq_lens.device)
        self.multi_T = T
        self.multi_pos = (self.seq_lens - T).clamp(min=0).to(torch.int32).contiguous()
        for L in self.layers:
            L["mq"] = workloads.randn_bf16(g, (B, T, s.num_q_heads, s.head_dim), self.seq_lens.device)
            L["mk"] = workloads.randn_bf16(g, (B, T, s.num_kv_heads, s.head_dim), self.seq_lens.device)
            L["mv"] = workloads.randn_bf16(g, (B, T, s.num_kv_heads, s.head_dim), self.seq_lens.device)
            L["mout"] = torch.empty(B, T, s.num_q_heads, s.head_dim, dtype=torch.bfloat16,
                                    device=self.seq_lens.device)
        import full_kv_cache_amd as hda
        need = max(hda.hda_decode_multi_workspace_bytes(L["cache"], L["lt"], T, self.max_seq_len)
                   for L in self.layers)
        self.multi_ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=self.seq_lens.device)
        old = self.multi_pos.cpu().long()
        self.multi_rows = {lt: int((old.clamp(max=s.window - 1) if lt == workloads.SLIDING else old).sum()
                                   + B * T) for lt in (workloads.SLIDING, workloads.FULL)}

    def make_prefill(self, B, T, seed):
        """Prefill chunks: the first B sequences of the batch, T new tokens
        each ending at the sequence's length (token 0 at seq_len - T), on
        every layer's cache (its first B blocks: a view, so the chunk
        appends where those sequences' rows are)."""
        import torch
        import workloads
        import full_kv_cache_amd as hda
        s = self.shape
        dev = self.seq_lens.device
        g = workloads.generator(seed + 6, dev)
        self.pf_B, self.pf_T = B, T
        self.pf_pos = (self.seq_lens[:B] - T).clamp(min=0).to(torch.int32).contiguous()
        for L in self.layers:
            L["pq"] = workloads.randn_bf16(g, (B, T, s.num_q_heads, s.head_dim), dev)
            L["pk"] = workloads.randn_bf16(g, (B, T, s.num_kv_heads, s.head_dim), dev)
            L["pv"] = workloads.randn_bf16(g, (B, T, s.num_kv_heads, s.head_dim), dev)
            L["pout"] = torch.empty(B, T, s.num_q_heads, s.head_dim, dtype=torch.bfloat16, device=dev)
            c = L["cache"]
            L["pcache_b"] = hda.LayerCache(c.k[:B], c.v[:B], s.num_q_heads, s.window, c.rotary_dim,
                                           c.rope_theta)
        need = max(hda.hda_decode_multi_workspace_bytes(L["pcache_b"], L["lt"], T, self.max_seq_len)
                   for L in self.layers)
        self.pf_ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=dev)
        old = self.pf_pos.cpu().long()
        # attended keys: token t sees its cached window entries plus tokens 0..t
        G = s.num_q_heads // s.num_kv_heads
        keys = {}
        for lt in (workloads.SLIDING, workloads.FULL):
            n = 0
            for p0 in old.tolist():
                for t in range(T):
                    cached = min(p0, s.window - 1 - t) if lt == workloads.SLIDING else p0
                    n += max(cached, 0) + t + 1
            keys[lt] = n
        self.pf_flops = sum(keys[L["lt"]] for L in self.layers) * s.num_kv_heads * G * s.head_dim * 4
        self.pf_rows = sum((old.clamp(max=s.window - 1) if L["lt"] == workloads.SLIDING else old).sum().item()
                           + B * T for L in self.layers)

    def prefill_call(self, L):
        import full_kv_cache_amd as hda
        hda.hda_decode_multi(L["pq"], L["pk"], L["pv"], self.pf_pos, L["lt"], L["pcache_b"], L["sinks"],
                             self.scale, L["pout"], max_seq_len=self.max_seq_len, workspace=self.pf_ws)

    def multi_call(self, L):
        import full_kv_cache_amd as hda
        hda.hda_decode_multi(L["mq"], L["mk"], L["mv"], self.multi_pos, L["lt"], L["cache"],
                             L["sinks"], self.scale, L["mout"], max_seq_len=self.max_seq_len,
                             workspace=self.multi_ws)

    def fp8_call(self, L):
        """The layer's step on its fp8 cache, as path auto: one launch for a
        sliding layer, append + attention for a full one."""
        import full_kv_cache_amd as hda
        import workloads
        if L["lt"] == workloads.SLIDING:
            hda.hda_decode_step(L["q"], L["k_new"], L["v_new"], self.pos, L["lt"], L["fcache"],
                                L["sinks"], self.scale, L["out"], L["lse"], self.workspace)
            return
        hda.hda_rope_append(L["q"], L["k_new"], L["v_new"], self.pos, L["lt"], L["fcache"])
        hda.hda_decode_attn(L["q"], L["fcache"], self.seq_lens, L["lt"], L["sinks"], self.scale,
                            L["out"], L["lse"], self.max_seq_len, 0, self.workspace)

    def layer_call(self, L, path="auto", chunk_keys=0, gate=False, paged=False):
        import full_kv_cache_amd as hda
        g = L["gate"] if gate else None
        if paged and "pcache" in L and layer_path(path, L["lt"]) == "fused":
            hda.hda_decode_step(L["q"], L["k_new"], L["v_new"], self.pos, L["lt"], L["pcache"],
                                L["sinks"], self.scale, L["out"], L["lse"], self.workspace, gate=g)
            return
        if paged and "pcache" in L:
            hda.hda_rope_append(L["q"], L["k_new"], L["v_new"], self.pos, L["lt"], L["pcache"])
            hda.hda_decode_attn(L["q"], L["pcache"], self.seq_lens, L["lt"], L["sinks"],
                                self.scale, L["out"], L["lse"], self.max_seq_len, 0,
                                self.workspace, gate=g)
            return
        if layer_path(path, L["lt"]) == "fused":
            hda.hda_decode_step(L["q"], L["k_new"], L["v_new"], self.pos, L["lt"], L["cache"],
                                L["sinks"], self.scale, L["out"], L["lse"], self.workspace, gate=g)
        else:
            hda.hda_rope_append(L["q"], L["k_new"], L["v_new"], self.pos, L["lt"], L["cache"])
            hda.hda_decode_attn(L["q"], L["cache"], self.seq_lens, L["lt"], L["sinks"], self.scale,
                                L["out"], L["lse"], self.max_seq_len, chunk_keys, self.workspace,
                                gate=g)

    def step(self, path="auto", chunk_keys=0, gate=False, paged=False):
        for L in self.layers:
            self.layer_call(L, path, chunk_keys, gate, paged)


def time_graph(fn, steps, warmup, use_graph=True, windows=5):
    """Milliseconds per call of fn: `steps` runs split into up to `windows`
    consecutive windows with HIP events on the stream at every boundary
    (no synchronisation between windows), the median window's per-call
    time.  Also returns the host wall clock per call over all steps and the
    per-window times."""
    import torch
    if use_graph:
        g = torch.cuda.CUDAGraph()
        fn()  # make sure every lazy init happened outside capture
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            fn()
        run = g.replay
    else:
        run = fn
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    nw = max(1, min(windows, steps))
    sizes = [steps // nw + (1 if i < steps % nw else 0) for i in range(nw)]
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(nw + 1)]
    wall = time.perf_counter()
    ev[0].record()
    for i, n in enumerate(sizes):
        for _ in range(n):
            run()
        ev[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall
    per = sorted(ev[i].elapsed_time(ev[i + 1]) / n for i, n in enumerate(sizes))
    median = per[len(per) // 2] if len(per) % 2 else 0.5 * (per[len(per) // 2 - 1] + per[len(per) // 2])
    time_graph.last_windows = [round(x, 4) for x in per]
    time_graph.last_mean = ev[0].elapsed_time(ev[-1]) / steps
    return median, wall * 1e3 / steps


def layer_path(path, lt):
    """The path a layer call takes: auto = hda_decode_step on both layer
    types (measured faster than hda_rope_append + hda_decode_attn on each:
    sliding 19.3 vs ~25 us, full 61.4 vs 62.7 us per layer at batch 64)."""
    if path == "auto":
        return "fused"
    return path


# Kernels a layer call runs on each path at G = 4 (the window kernels serve
# every sliding layer: keys <= 1024; full layers at these shapes take the
# stream).
KERNELS = {
    ("separate", "sliding"): "decode_pair_kernel<2, false>",
    ("separate", "full"): "decode_stream_kernel<4, false, 0> + stream_merge_kernel<false>",
    ("fused", "sliding"): "decode_window_step_kernel<2, 256, false, false, 8>",
    ("fused", "full"): "decode_stream_kernel<4, false, 64> + stream_merge_kernel<true>",
}


def kernel_name(path, name, batch):
    """The kernel names of a layer call.  The one-launch sliding step splits
    a (sequence, KV head) pair by heads when there are at least 128 pairs
    (two workgroups, two heads each) and by keys below that (four heads,
    last-arriver merge): the library's window_step_plan at G = 4, window
    512, two KV heads."""
    if (path, name) == ("fused", "sliding") and batch * 2 < 128:
        return "decode_window_step_kernel<4, 256, false, true, 8>"
    return KERNELS[(path, name)]


# Sources whose change invalidates a committed traffic measurement.
TRAFFIC_SOURCES = ("decode_attn.hip", "decode_wave.h", "decode_step.hip", "hda_device.h",
                   "hda_kernels.h", "hda_api.cpp", "rope_append.hip", "sparse_attn.hip",
                   "decode_multi.hip")


def layer_kernel(wl: Workload, lt: int, steps, warmup, path="auto", chunk_keys=0, paged=False):
    """Time one layer type's attention calls (exactly as the step makes them:
    on the separate path hda_decode_attn without the RoPE/append launch, on
    the fused path the whole hda_decode_step) captured in one graph, HIP
    events on the launch stream around the replays; average per call.  Algorithmic bytes per
    call: every attended K and V row once (per sequence min(seq_len, window)
    rows for a sliding layer, seq_len rows for a full one, of 2 KV heads x
    256 dims x 2 bytes, for K and for V)."""
    import full_kv_cache_amd as hda
    import workloads
    Ls = [L for L in wl.layers if L["lt"] == lt]
    if not Ls or (paged and "pcache" not in Ls[0]):
        return None
    path = "separate" if paged else layer_path(path, lt)
    key = "pcache" if paged else "cache"

    def fn():
        for L in Ls:
            if path == "fused":
                wl.layer_call(L, "fused")
            else:
                hda.hda_decode_attn(L["q"], L[key], wl.seq_lens, lt, L["sinks"], wl.scale,
                                    L["out"], L["lse"], wl.max_seq_len, chunk_keys, wl.workspace)

    ms, _ = time_graph(fn, steps, warmup)
    per_call_s = ms / len(Ls) / 1e3
    algo = wl.rows[lt] * wl.kv_row_bytes
    achieved = algo / per_call_s / 1e9
    name = "sliding" if lt == workloads.SLIDING else "full"
    kname = kernel_name(path, name, wl.cfg["batch"])
    if paged:
        p = Ls[0]["pcache"].desc()
        return {
            "kernel": f"{kname} (full-layer hda_decode_attn, paged)",
            "page_size": p.page_size, "pool_pages": p.num_pages,
            "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "algorithmic_bytes_per_launch": algo,
            "avg_launch_us": round(per_call_s * 1e6, 2), "launches_timed": steps * len(Ls),
            "launches_per_call": kname.count(" + ") + 1,
        }
    return {
        "kernel": f"{kname} ({name}-layer hda_decode_attn)" if path == "separate"
                  else f"{kname} ({name}-layer hda_decode_step)",
        "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4),
        "traffic": measured_traffic(kname, wl.cfg["batch"]),
        "algorithmic_bytes_per_launch": algo, "avg_launch_us": round(per_call_s * 1e6, 2),
        "launches_timed": steps * len(Ls),
        # avg_launch_us is per call: per launch when the call is one launch
        "launches_per_call": kname.count(" + ") + 1,
    }


def sources_digest():
    import hashlib
    h = hashlib.sha256()
    for src in TRAFFIC_SOURCES:
        h.update(open(os.path.join(ROOT, "full_kv_cache_amd", "csrc", src), "rb").read())
    return h.hexdigest()


def measured_traffic(kernel, batch):
    """HBM bytes per launch from the committed PMC summary
    (profiles/traffic_decode_b64_u512-4096.txt: FETCH_SIZE x the
    copy-calibrated factor + WRITE_SIZE, per launch of the kernel), or None
    when there is none for this kernel, or it was taken on other sources."""
    f = os.path.join(ROOT, "profiles", "traffic_decode_b64_u512-4096.txt")
    if batch != 64 or not os.path.exists(f):
        return None
    digest, table = None, {}
    for line in open(f):
        line = line.strip()
        if line.startswith("source_sha256:"):
            digest = line.split(":", 1)[1].strip()
        elif line.startswith("|") and "bytes" not in line and "---" not in line:
            cells = [c.strip() for c in line.strip("|").split("|")]
            if len(cells) >= 5:
                try:
                    table[cells[0]] = int(cells[4].replace(",", ""))
                except ValueError:
                    pass
    if digest != sources_digest():
        return None
    return table.get(kernel)


def sparse_kernel(steps, warmup, seed, pools=8, fp8=False):
    """The sparse top-k decode with sinks at its page shape (32 tokens, 64
    query heads over one 576-dim latent head, value = leading 512 dims,
    pool of 32768 rows, top-2048 indices per token): `pools` distinct pools
    (8 x 37.7 MB bf16, more than the 256 MB last-level cache) are cycled
    through one graph so that rows come from HBM, HIP events on the launch
    stream.  Gathered bytes per call = tokens x topk x row bytes (1152 bf16;
    fp8: 576 codes + a 4-byte scale); flops = tokens x heads x topk x 2
    (576 + 512).  fp8: the pools hold e4m3 codes with per-row scales
    (hda_sparse_decode_attn_fp8)."""
    import torch
    import workloads
    import full_kv_cache_amd as hda
    s = workloads.SparseShape()
    g = workloads.generator(seed + 1, "cuda")
    ins = [workloads.sparse_inputs(g, s, "cuda") for _ in range(pools)]
    if fp8:
        g8 = workloads.generator(seed + 7, "cuda")
        for t in ins:
            t["codes"] = workloads.fp8_codes(g8, (s.pool, s.dqk), "cuda")
            t["scales"] = workloads.fp8_scales(g8, (s.pool,), "cuda")
            del t["kv"]
    outs = [torch.empty(s.tokens, s.num_q_heads, s.dv, dtype=torch.bfloat16, device="cuda")
            for _ in range(pools)]
    lses = [torch.empty(s.tokens, s.num_q_heads, dtype=torch.float32, device="cuda")
            for _ in range(pools)]
    nbytes = hda.hda_sparse_workspace_bytes(s.tokens, s.num_q_heads, s.topk, s.dv)
    ws = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device="cuda")
    scale = 1.0 / s.dqk ** 0.5

    def fn():
        for i in range(pools):
            if fp8:
                hda.hda_sparse_decode_attn_fp8(ins[i]["q"], ins[i]["codes"], ins[i]["scales"],
                                               ins[i]["indices"], ins[i]["sinks"], scale, outs[i],
                                               lses[i], ws)
            else:
                hda.hda_sparse_decode_attn(ins[i]["q"], ins[i]["kv"], ins[i]["indices"], None,
                                           ins[i]["sinks"], scale, outs[i], lses[i], ws)

    ms, _ = time_graph(fn, steps, warmup)
    per_call_s = ms / pools / 1e3
    row_bytes = s.dqk + 4 if fp8 else s.dqk * 2
    gathered = s.tokens * s.topk * row_bytes
    flops = s.tokens * s.num_q_heads * s.topk * 2 * (s.dqk + s.dv)
    gbs = gathered / per_call_s / 1e9
    # up to 64 heads take the shared-tile kernel, bf16 or fp8 pool (the
    # library's sparse routing)
    kname = ("sparse_tile_kernel<false, true> + sparse_merge_kernel" if fp8
             else "sparse_tile_kernel<false, false> + sparse_merge_kernel")
    return {
        "kernel": f"{kname} (hda_sparse_decode_attn{'_fp8' if fp8 else ''})",
        "workload": f"{s.tokens} tokens x {s.num_q_heads} heads, dqk {s.dqk} / dv {s.dv}, pool "
                    f"{s.pool} rows{' (e4m3 codes + row scales)' if fp8 else ''}, top-{s.topk}, "
                    f"per-head sinks, {pools} pools cycled",
        "us_per_call": round(per_call_s * 1e6, 2), "gather_GBs": round(gbs, 1),
        "tflops": round(flops / per_call_s / 1e12, 1),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(kname, 64),
                     "algorithmic_bytes_per_launch": gathered},
        "mfma_bf16_frac": round(flops / per_call_s / 2.5e15, 4),
    }


def device_info():
    """Device name, architecture, ROCm/HIP version, the current clock
    levels the driver exposes in sysfs, and the host CPU model."""
    import glob
    import torch
    p = torch.cuda.get_device_properties(0)
    info = {"device": torch.cuda.get_device_name(0), "arch": getattr(p, "gcnArchName", None),
            "compute_units": p.multi_processor_count,
            "hbm_GiB": round(p.total_memory / 2 ** 30, 1), "hip": torch.version.hip,
            "torch": torch.__version__, "cpu_model": cpu_model()}
    try:
        info["rocm"] = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        info["rocm"] = None
    clocks = {}
    for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
        for name in ("product_name", "pp_dpm_sclk", "pp_dpm_mclk"):
            try:
                text = open(os.path.join(dev, name)).read()
            except OSError:
                continue
            if name == "product_name":
                clocks.setdefault("product_name", text.strip())
            else:  # the level the driver marks as current
                cur = [ln.split(":", 1)[-1].strip(" *") for ln in text.splitlines() if ln.endswith("*")]
                if cur:
                    clocks.setdefault(name[-4:], cur[0])
        if clocks:
            break
    info["clocks"] = clocks or None
    return info


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def other_config(name, args):
    """Step time of another configuration on its own workload: graph and
    eager timing of the whole 28-layer step, KV GB/s and tokens/s, and the
    full-layer kernel's roofline entry."""
    import torch
    import workloads
    cfg = CONFIGS[name]
    print(f"# timing {name}: {cfg['desc']}", file=sys.stderr, flush=True)
    wl = Workload(cfg, args.seed)
    torch.cuda.synchronize()
    step = lambda: wl.step(args.path, args.chunk_keys)
    ms, _ = time_graph(step, args.steps, args.warmup)
    win = time_graph.last_windows
    eager, _ = time_graph(step, max(5, args.steps // 5), 2, use_graph=False)
    gbs = wl.kv_bytes / (ms / 1e3) / 1e9
    sl = wl.seq_lens.cpu()
    rec = {"workload": f"{name}: {cfg['desc']}", "batch": cfg["batch"],
           "seq_len_min": int(sl.min()), "seq_len_max": int(sl.max()),
           "ms_per_step": round(ms, 4), "window_ms_per_step": win,
           "eager_ms_per_step": round(eager, 4), "tokens_per_s": round(cfg["batch"] / (ms / 1e3), 1),
           "kv_bytes_per_step": wl.kv_bytes, "GB/s": round(gbs, 1),
           "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
           "layer_kernels": {
               "sliding": layer_kernel(wl, workloads.SLIDING, args.steps, args.warmup, args.path,
                                       args.chunk_keys),
               "full": layer_kernel(wl, workloads.FULL, args.steps, args.warmup, args.path,
                                    args.chunk_keys)}}
    del wl
    torch.cuda.empty_cache()
    return rec


def cpu_baseline(wl: Workload, min_seconds: float):
    """The oracle on host copies of the same workload: whole 28-layer steps
    over the batch (append + attention per layer), repeated until at least
    min_seconds have passed (at most 50 steps)."""
    import numpy as np
    import oracle
    import workloads
    s = wl.shape
    host = []
    W = s.window
    for L in wl.layers:
        h = {k: workloads.bits(v).copy() for k, v in L["raw"].items()}
        h["q"] = workloads.bits(L["q"]).copy()
        if L["lt"] == workloads.SLIDING:  # the oracle keeps ring and side row apart
            for a in ("k", "v"):
                blk = h[a]
                h[a] = np.ascontiguousarray(blk[:, :, :W - 1])
                h[a + "ev"] = np.ascontiguousarray(blk[:, :, W - 1])
        else:
            h["kev"] = h["vev"] = np.zeros((s.batch, s.num_kv_heads, s.head_dim), np.uint16)
        host.append((L["lt"], h, L["sinks"].cpu().numpy()))
    pos = wl.pos.cpu().numpy()
    seq = wl.seq_lens.cpu().numpy()
    steps = 0
    t0 = time.perf_counter()
    while True:
        for lt, h, sk in host:
            oracle.rope_append(h["q"], h["k_new"], h["v_new"], pos, lt, s.rot(lt), s.theta(lt),
                               s.window, h["k"], h["v"], h["kev"], h["vev"])
            oracle.decode_attn(h["q"], h["k"], h["v"], h["kev"], h["vev"], seq, lt, s.window, sk,
                               wl.scale)
        steps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds or steps >= 50:
            break
    return {
        "value": round(wl.kv_bytes * steps / el / 1e9, 3), "unit": "GB/s",
        "tokens_per_s": round(s.batch * steps / el, 2),
        "cores": oracle.num_threads(), "kind": "oracle", "cpu_model": cpu_model(),
        "sample": f"{steps} whole step(s) of the same workload ({s.batch} sequences x "
                  f"{len(wl.layers)} layers, append + attention) in {el:.1f} s, fp64 C oracle",
    }


def copy_calibration(mb: int):
    """A plain device copy of a known size, for scaling PMC byte counters."""
    import torch
    n = mb * (1 << 20)
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 5}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the decode path is "
              "measured as one GPU's share at its full shape.", file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    import full_kv_cache_amd as hda
    hda.lib()  # fail loudly if the library is missing

    cfg = CONFIGS[args.config]
    print(f"# building workload {args.config}: {cfg['desc']}", file=sys.stderr, flush=True)
    wl = Workload(cfg, args.seed)
    torch.cuda.synchronize()
    step = lambda: wl.step(args.path, args.chunk_keys)
    for _ in range(2):
        step()
    torch.cuda.synchronize()

    print("# timing step", file=sys.stderr, flush=True)
    ms, wall_ms = time_graph(step, args.steps, args.warmup, use_graph=not args.no_graph)
    windows, mean_ms = time_graph.last_windows, time_graph.last_mean
    eager_ms = None
    if not args.no_graph:
        eager_ms, _ = time_graph(step, max(3, args.steps // 5), 2, use_graph=False)
    # the same step with the per-head output gate applied in every epilogue
    gated_ms, _ = time_graph(lambda: wl.step(args.path, args.chunk_keys, gate=True), args.steps,
                             args.warmup, use_graph=not args.no_graph)
    print("# timing the layer kernels", file=sys.stderr, flush=True)
    import workloads
    k_slide = layer_kernel(wl, workloads.SLIDING, args.steps, args.warmup, args.path, args.chunk_keys)
    k_full = layer_kernel(wl, workloads.FULL, args.steps, args.warmup, args.path, args.chunk_keys)
    paged_ms, k_paged = None, None
    if args.page_size and wl.shape.capacity(workloads.FULL) % args.page_size == 0:
        print(f"# timing the step with paged full layers ({args.page_size}-row pages)",
              file=sys.stderr, flush=True)
        wl.make_paged(args.page_size, args.seed)
        torch.cuda.synchronize()
        paged_ms, _ = time_graph(lambda: wl.step(args.path, args.chunk_keys, paged=True),
                                 args.steps, args.warmup, use_graph=not args.no_graph)
        k_paged = layer_kernel(wl, workloads.FULL, args.steps, args.warmup, paged=True)
    # the dominant kernel: the layer type with the most attention time per step
    n_s = sum(1 for L in wl.layers if L["lt"] == workloads.SLIDING)
    n_f = len(wl.layers) - n_s
    # The roofline names one kernel, so a call that is one launch is
    # preferred: the full layer's call is the streaming kernel plus its merge
    # (at the default shape the one-launch sliding step is also the larger
    # single-kernel share: 21 x 19.3 us against 7 x 52.7 us of streaming
    # kernel in the kernel trace).
    cands = [(k["launches_per_call"] == 1, k["avg_launch_us"] * n, k)
             for k, n in ((k_slide, n_s), (k_full, n_f)) if k]
    roof = max(cands, key=lambda c: c[:2])[2] if cands else None
    fp8 = None
    if not args.no_fp8:
        print("# timing the step on an fp8 cache", file=sys.stderr, flush=True)
        wl.make_fp8(args.seed)
        torch.cuda.synchronize()

        def fp8_step():
            for L in wl.layers:
                wl.fp8_call(L)
        fp8_ms, _ = time_graph(fp8_step, args.steps, args.warmup, use_graph=not args.no_graph)
        fp8 = {"ms_per_step": round(fp8_ms, 4),
               "tokens_per_s": round(cfg["batch"] / (fp8_ms / 1e3), 1),
               "kv_bytes_per_step": sum(wl.rows[L["lt"]] for L in wl.layers) * wl.fp8_row_bytes,
               "path": "hda_decode_step (one launch) for sliding layers, hda_rope_append + "
                       "hda_decode_attn (streaming kernel + merge) for full layers"}
        fp8["GB/s"] = round(fp8["kv_bytes_per_step"] / (fp8_ms / 1e3) / 1e9, 1)
        for lt, name in ((workloads.SLIDING, "sliding"), (workloads.FULL, "full")):
            Ls = [L for L in wl.layers if L["lt"] == lt]
            if not Ls:
                continue

            def attn(Ls=Ls, lt=lt):  # sliding: the whole one-launch step; full: attention
                for L in Ls:
                    if lt == workloads.SLIDING:
                        wl.fp8_call(L)
                        continue
                    hda.hda_decode_attn(L["q"], L["fcache"], wl.seq_lens, lt, L["sinks"], wl.scale,
                                        L["out"], L["lse"], wl.max_seq_len, 0, wl.workspace)
            ms_l, _ = time_graph(attn, args.steps, args.warmup)
            us = ms_l / len(Ls) * 1e3
            byts = wl.rows[lt] * wl.fp8_row_bytes
            fp8[f"{name}_attn_us"] = round(us, 2)
            fp8[f"{name}_attn_GB/s"] = round(byts / (us / 1e6) / 1e9, 1)
    multi = None
    if args.multi_tokens:
        T = args.multi_tokens
        print(f"# timing chunk decode, {T} tokens per sequence", file=sys.stderr, flush=True)
        wl.make_multi(T, args.seed)
        torch.cuda.synchronize()

        def multi_step():
            for L in wl.layers:
                wl.multi_call(L)
        m_ms, _ = time_graph(multi_step, args.steps, args.warmup, use_graph=not args.no_graph)
        m_bytes = sum(wl.multi_rows[L["lt"]] for L in wl.layers) * wl.kv_row_bytes
        multi = {"tokens_per_chunk": T, "ms_per_step": round(m_ms, 4),
                 "tokens_per_s": round(cfg["batch"] * T / (m_ms / 1e3), 1),
                 "kv_bytes_per_step": m_bytes, "GB/s": round(m_bytes / (m_ms / 1e3) / 1e9, 1),
                 "path": "hda_decode_multi on every layer (RoPE; attention split over "
                         "workgroups (2 per pair at this batch, one per pair for one-token "
                         "chunks on sliding layers, which then append); merge, whose launch "
                         "also writes the append)"}
    prefill = None
    if args.prefill_tokens:
        B, T = args.prefill_batch, args.prefill_tokens
        print(f"# timing chunked prefill, {B} sequences x {T} tokens", file=sys.stderr, flush=True)
        wl.make_prefill(B, T, args.seed)
        torch.cuda.synchronize()

        def prefill_step():
            for L in wl.layers:
                wl.prefill_call(L)
        p_ms, _ = time_graph(prefill_step, args.steps, args.warmup, use_graph=not args.no_graph)
        prefill = {"batch": B, "tokens_per_chunk": T, "ms_per_step": round(p_ms, 4),
                   "tokens_per_s": round(B * T / (p_ms / 1e3), 1),
                   "attn_tflops": round(wl.pf_flops / (p_ms / 1e3) / 1e12, 1),
                   "mfma_bf16_frac": round(wl.pf_flops / (p_ms / 1e3) / 2.5e15, 4),
                   "kv_GB/s": round(wl.pf_rows * wl.kv_row_bytes / (p_ms / 1e3) / 1e9, 1),
                   "path": "hda_decode_multi on every layer (RoPE, prefill_chunk_kernel: both "
                           "products on MFMA, merge of the key split with the append: 3 "
                           "launches)"}
    sparse = None
    if not args.no_sparse:
        print("# timing sparse top-k decode", file=sys.stderr, flush=True)
        sparse = sparse_kernel(args.steps, args.warmup, args.seed)
        sparse["fp8"] = sparse_kernel(args.steps, args.warmup, args.seed, fp8=True)
    others = {}
    if args.config == "throughput" and not args.no_other_configs:
        for name in ("step28", "long"):
            others[name] = other_config(name, args)
    cpu = None
    if not args.no_cpu_baseline:
        print("# cpu baseline (oracle)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl, args.cpu_seconds)

    gbs = wl.kv_bytes / (ms / 1e3) / 1e9
    sl = wl.seq_lens.cpu()
    rec = {
        "metric": METRIC, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded unit-normal bf16 q/K/V, N(0,1) fp32 sinks)",
        "config": {"workload": f"{args.config}: {cfg['desc']}", "batch": cfg["batch"],
                   "layers": cfg["layers"], "seq_len_min": int(sl.min()),
                   "seq_len_max": int(sl.max()), "seq_len_mean": round(float(sl.float().mean()), 1),
                   "graph": not args.no_graph, "path": args.path, "chunk_keys": args.chunk_keys},
        "tokens_per_s": round(cfg["batch"] / (ms / 1e3), 1),
        "timing": f"median of {len(windows)} windows of the {args.steps} timed steps (HIP events "
                  "on the stream at each window boundary)",
        "window_ms_per_step": windows, "mean_ms_per_step": round(mean_ms, 4),
        "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "kv_bytes_per_step": wl.kv_bytes,
        "eager_ms_per_step": None if eager_ms is None else round(eager_ms, 4),
        "gated_ms_per_step": round(gated_ms, 4),
        "paged_ms_per_step": None if paged_ms is None else round(paged_ms, 4),
        "host_wall_ms_per_step": round(wall_ms, 4),
        "roofline": roof, "layer_kernels": {"sliding": k_slide, "full": k_full},
        "cpu_baseline": cpu, "sparse": sparse, "paged": k_paged, "fp8": fp8, "multi": multi,
        "prefill": prefill, "step28": others.get("step28"), "long": others.get("long"),
        "device": device_info(),
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
