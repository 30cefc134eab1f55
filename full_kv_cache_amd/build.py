"""Build libhda.so (the C-ABI library) for gfx950 with hipcc, in-tree.

    python -m full_kv_cache_amd.build

Compiles every HIP source under ``csrc/`` and the host API into one shared
library next to this file.  Packed-fp32 instructions are disabled for the
device code (``-packed-fp32-ops``); the host pass warns that it does not
know the feature, which is harmless.  Type-based alias analysis is off
(``-fno-strict-aliasing``): KV rows are loaded through one vector type and
stored through another, and a store must never pass a load of the same row.
"""
from __future__ import annotations

import os
import subprocess
import sys
from pathlib import Path

HERE = Path(__file__).resolve().parent
CSRC = HERE / "csrc"
LIB = HERE / "libhda.so"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["hda_api.cpp", "rope_append.hip", "decode_attn.hip", "decode_step.hip", "sparse_attn.hip",
           "decode_multi.hip", "noalloc.hip"]


def compile_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wextra",
        "-Wno-unused-parameter", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # the kernels read KV rows as one vector type and write them as another:
        # ordering between the two must come from the addresses, not the types
        "-fno-strict-aliasing",
        "-I", str(HERE.parent / "include"),
    ]


def build(verbose: bool = False) -> Path:
    """Compile all sources (always) and link libhda.so atomically."""
    objs = []
    build_dir = HERE / "_build"
    build_dir.mkdir(exist_ok=True)
    procs = []
    for src in SOURCES:
        path = CSRC / src
        if not path.exists():
            raise FileNotFoundError(f"library source {path} is missing")
        obj = build_dir / (src + ".o")
        cmd = [HIPCC, *compile_flags(), "-c", "-x", "hip", str(path), "-o", str(obj)]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs.append(obj)
    failed = []
    for src, pr in procs:
        out, _ = pr.communicate()
        text = out.decode(errors="replace")
        text = "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l)
        if text.strip() and (verbose or pr.returncode):
            print(text, file=sys.stderr)
        if pr.returncode:
            failed.append(src)
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    tmp = LIB.with_suffix(".so.tmp%d" % os.getpid())
    link = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", str(tmp), *map(str, objs)]
    subprocess.check_call(link)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
