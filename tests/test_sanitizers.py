"""Sanitizer runs on the CPU: the host validation and planning of the C ABI, and the C++ oracle.

* csrc/kvarn_host.h (the code libkvarn.so validates and plans with) in a self-test built with g++
  under AddressSanitizer + UndefinedBehaviorSanitizer: extreme sizes, NULL and misaligned pointers,
  every format; the documented status for chosen cases and, for every call that would launch, sizes
  and a split plan the kernels accept.
* oracle/kvarn_oracle.cpp with its self-test under AddressSanitizer + UndefinedBehaviorSanitizer and,
  for the threaded driver, ThreadSanitizer.
Any sanitizer report ends the run with a non-zero status.
"""
import ctypes

import pytest

from kv_cache_quantization_kvarn_amd import host_selftest
from kv_cache_quantization_kvarn_amd import kvarn as K
from oracle import kvarn_oracle_cpp as C


def _ok(r, tag):
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "0 failed" in out and "ERROR" not in out and "WARNING: ThreadSanitizer" not in out, out[-4000:]
    assert tag in out


def test_host_validation_under_asan_ubsan():
    _ok(host_selftest.run(), "host self-test")


@pytest.mark.parametrize("kind", ["asan", "tsan"])
def test_oracle_under_sanitizers(kind):
    _ok(C.run_selftest(kind), "oracle self-test")


def test_workspace_query_refuses_sizes_decode_refuses():
    lib = K.library()
    cfg = K.kvarn_config_parse("kvarn_k4v2_g128")
    q = lib.kvarn_decode_workspace_bytes
    assert q(ctypes.byref(cfg), 64, 16, 2, 32) > 0
    for batch, nq, hkv, mb in ((65536, 8, 8, 32), (1, 8, 65536 * 8 // 8 + 1, 32), (1, 8, 8, 1 << 24),
                               (2 ** 31 - 1, 2 ** 31 - 1, 2 ** 31 - 1, 2 ** 31 - 1), (0, 8, 8, 32), (4, 0, 8, 32)):
        assert q(ctypes.byref(cfg), batch, nq, hkv, mb) == 0, (batch, nq, hkv, mb)
