"""Register and scratch budget of the default-path kernels (CPU only: the
compiler's resource-usage report, no GPU).

A kernel whose per-lane arrays leave registers for scratch memory still
computes the right result but streams far slower (a value-initialised
vector in shared code once pushed the sliding-layer step from 20 to 48 us).
Every kernel on a default path -- the one-launch window step, the
streaming kernel (plain and in its step form) and the window kernels, bf16
and fp8, the chunk-decode and chunked-prefill kernels, the sparse decode (bf16 and fp8 pools),
the merges and the appends -- and the
one-launch step for sliding windows past one workgroup must use no scratch
and spill nothing.
"""
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from full_kv_cache_amd import build as hb

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "full_kv_cache_amd", "csrc")

# mangled-name fragments of the kernels that must stay in registers
DEFAULT_PATH = {
    "decode_step.hip": ["decode_window_step_kernelILi2ELi256ELb0E", "decode_window_step_kernelILi2ELi256ELb1E",
                        "decode_window_step_kernelILi2ELi64ELb0E", "decode_step_kernelILi4ELi256E"],
    "decode_attn.hip": ["decode_stream_kernelILi4ELb0E", "decode_stream_kernelILi4ELb1E",
                        "decode_pair_kernelILi2ELb0E", "decode_pair_kernelILi2ELb1E",
                        "stream_merge_kernel", "lse_merge_kernel"],
    "decode_multi.hip": ["decode_multi_kernelILi4ELi1E", "decode_multi_kernelILi4ELi2E",
                         "decode_multi_kernelILi4ELi3E", "decode_multi_kernelILi4ELi4E",
                         "prefill_chunk_kernel", "multi_merge_kernel", "rope_multi_kernel",
                         "append_multi_kernel"],
    "rope_append.hip": ["rope_append_kernel", "rope_append_fp8_kernel"],
    "sparse_attn.hip": ["sparse_decode_kernelILb0ELb0E", "sparse_decode_kernelILb0ELb1E",
                        "sparse_decode_kernelILb1ELb0E", "sparse_decode_kernelILb1ELb1E",
                        "sparse_merge_kernel", "sparse_tile_kernelILb0E", "sparse_tile_kernelILb1E"],
    "noalloc.hip": ["zero_fill_kernel"],
}


def _report(src):
    cmd = [hb.HIPCC, *hb.compile_flags(), "--cuda-device-only", "-c", "-x", "hip",
           "-Rpass-analysis=kernel-resource-usage", "-o", os.devnull, os.path.join(CSRC, src)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    usage, name = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            usage[name] = {}
            continue
        m = re.search(r"remark:\s+(ScratchSize \[bytes/lane\]|VGPRs Spill|VGPRs): (\d+)", line)
        if m and name:
            usage[name][m.group(1)] = int(m.group(2))
    return src, usage


@pytest.mark.skipif(shutil.which(hb.HIPCC) is None and not os.path.exists(hb.HIPCC),
                    reason="hipcc not available")
def test_default_path_kernels_use_no_scratch():
    with ThreadPoolExecutor(max_workers=4) as ex:
        reports = dict(ex.map(_report, DEFAULT_PATH))
    for src, wanted in DEFAULT_PATH.items():
        usage = reports[src]
        for frag in wanted:
            hits = [n for n in usage if frag in n]
            assert hits, f"{frag} not found in {src}"
            for n in hits:
                u = usage[n]
                assert u.get("ScratchSize [bytes/lane]", 0) == 0, (n, u)
                assert u.get("VGPRs Spill", 0) == 0, (n, u)
