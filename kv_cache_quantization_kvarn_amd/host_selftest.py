"""Build and run the host self-test of the C ABI's validation and planning (csrc/host_selftest.cpp).

The self-test includes csrc/kvarn_host.h, the same header libkvarn.so is built from, and is compiled
with g++ under AddressSanitizer and UndefinedBehaviorSanitizer without recovery, so an overflow, an
out-of-bounds access or a failed check ends it with a non-zero status.  It needs no GPU.

    python -m kv_cache_quantization_kvarn_amd.host_selftest
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "csrc", "host_selftest.cpp")
HEADERS = [os.path.join(HERE, "csrc", "kvarn_host.h"), os.path.join(HERE, "..", "include", "kvarn.h")]
EXE = os.path.join(HERE, "_build", "host_selftest")
SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
CXXFLAGS = ["-std=c++17", "-O1", "-g", "-Wall", "-Wextra", "-Werror"]
ENV = {"ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0:halt_on_error=1",
       "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"}


def build() -> str:
    os.makedirs(os.path.dirname(EXE), exist_ok=True)
    tmp = EXE + ".tmp"
    cmd = ["g++"] + CXXFLAGS + SANITIZE + ["-o", tmp, SRC]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("g++ failed (%d): %s\n%s" % (res.returncode, " ".join(cmd), res.stdout + res.stderr))
    os.replace(tmp, EXE)
    return EXE


def _stale() -> bool:
    if not os.path.exists(EXE):
        return True
    t = os.path.getmtime(EXE)
    return any(os.path.getmtime(p) > t for p in [SRC] + HEADERS)


def run(timeout: float = 600) -> subprocess.CompletedProcess:
    """Run the self-test (building it first if it is missing or older than its sources)."""
    if _stale():
        build()
    env = dict(os.environ)
    env.update(ENV)
    return subprocess.run([EXE], capture_output=True, text=True, timeout=timeout, env=env)


if __name__ == "__main__":
    r = run()
    print(r.stdout + r.stderr)
    raise SystemExit(r.returncode)
