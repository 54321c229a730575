"""Build libkvarn.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m kv_cache_quantization_kvarn_amd.build   (or import and call build())
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkvarn.so")
SOURCES = ["kvarn_api.hip", "kvarn_quantize.hip", "kvarn_decode.hip", "kvarn_fp16_decode.hip",
           "kvarn_prefill.hip", "kvarn_headdim.hip"]

# Packed fp32 VALU instructions are disabled for device code; the host pass
# ignores the feature (and says so).
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed (%d): %s\n%s" % (res.returncode, " ".join(cmd), err))
    return err


def build(verbose: bool = False) -> str:
    """Compile every source to an object (in parallel), then link libkvarn.so."""
    import concurrent.futures
    import tempfile
    with tempfile.TemporaryDirectory(prefix="kvarn_build_") as tmpdir:
        jobs = []
        for src in SOURCES:
            obj = os.path.join(tmpdir, src.replace(".hip", ".o"))
            jobs.append((obj, [hipcc()] + FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]))
        with concurrent.futures.ThreadPoolExecutor(max_workers=len(jobs)) as pool:
            msgs = list(pool.map(_run, [cmd for _, cmd in jobs]))
        tmp = LIB + ".tmp"
        msgs.append(_run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + [o for o, _ in jobs]))
    if verbose and any(m.strip() for m in msgs):
        print("\n".join(m for m in msgs if m.strip()), file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
