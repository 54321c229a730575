"""Python access to the C++ oracle (oracle/kvarn_oracle.cpp): build and ctypes calls.

TEST INFRASTRUCTURE ONLY, like the Python oracle next to it: only the tests, the package smoke check
and the CPU-baseline leg of the benchmark may load it.  The C++ oracle computes what the Python
oracle computes (the same readings, restated in the .cpp header), in double precision with threads,
so that parity can cover whole workloads: every tile of a layer, every (sequence, query head) of a
decode step.

The library is built with g++ (not hipcc), without fused multiply-add contraction, so that fp32 and
fp64 operations round exactly as written.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kvarn_oracle.cpp")
LIB_PATH = os.path.join(HERE, "libkvarn_oracle.so")
CXXFLAGS = ["-std=c++17", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-Wall", "-Wextra",
            "-pthread"]


def build(verbose: bool = False) -> str:
    """Compile the C++ oracle into oracle/libkvarn_oracle.so."""
    tmp = LIB_PATH + ".tmp"
    cmd = ["g++"] + CXXFLAGS + ["-o", tmp, SRC]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("g++ failed (%d): %s\n%s" % (res.returncode, " ".join(cmd), res.stdout + res.stderr))
    if verbose and (res.stdout + res.stderr).strip():
        print(res.stdout + res.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


# Sanitizer builds of the oracle with its self-test driver (kvarn_oracle_selftest.cpp): AddressSanitizer
# with UndefinedBehaviorSanitizer, and ThreadSanitizer for the threaded driver.
SELFTEST_SRC = os.path.join(HERE, "kvarn_oracle_selftest.cpp")
SELFTEST_FLAGS = {"asan": ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"],
                  "tsan": ["-fsanitize=thread"]}
SELFTEST_ENV = {"ASAN_OPTIONS": "detect_leaks=1:halt_on_error=1", "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1",
                "TSAN_OPTIONS": "halt_on_error=1"}


def selftest_path(kind: str) -> str:
    return os.path.join(HERE, "_build", "oracle_selftest_" + kind)


def build_selftest(kind: str) -> str:
    """Compile the oracle and its self-test under one sanitizer kind ("asan" or "tsan")."""
    exe = selftest_path(kind)
    os.makedirs(os.path.dirname(exe), exist_ok=True)
    cmd = (["g++", "-std=c++17", "-O1", "-g", "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra", "-Werror",
            "-pthread"] + SELFTEST_FLAGS[kind] + ["-o", exe + ".tmp", SRC, SELFTEST_SRC])
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("g++ failed (%d): %s\n%s" % (res.returncode, " ".join(cmd), res.stdout + res.stderr))
    os.replace(exe + ".tmp", exe)
    return exe


def run_selftest(kind: str, timeout: float = 600) -> subprocess.CompletedProcess:
    """Run one sanitizer build of the self-test, building it first if it is missing or older than its sources."""
    exe = selftest_path(kind)
    if not os.path.exists(exe) or max(os.path.getmtime(SRC), os.path.getmtime(SELFTEST_SRC)) > os.path.getmtime(exe):
        build_selftest(kind)
    env = dict(os.environ)
    env.update(SELFTEST_ENV)
    return subprocess.run([exe], capture_output=True, text=True, timeout=timeout, env=env)


_lib = None


def default_threads() -> int:
    """Worker threads: the cores this process may run on, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("the C++ oracle is not built (%s); run oracle.kvarn_oracle_cpp.build()" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        P, I, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_double
        sig = {
            "kvo_page_bytes": (ctypes.c_long, [I, I, I, I]),
            "kvo_half_to_double": (D, [ctypes.c_uint16]),
            "kvo_double_to_half": (ctypes.c_uint16, [D]),
            "kvo_rotate": (I, [P, I, I, I, P]),
            "kvo_normalize": (I, [P, I, I, I, D, P, P]),
            "kvo_quantize_blocks": (ctypes.c_long, [P, P, I, I, I, P, P, P, I, I, I, I, I, I]),
            "kvo_dequantize_page": (I, [P, I, I, I, I, I, P]),
            "kvo_decode": (I, [P, P, P, I, P, I, P, P, P, I, I, I, I, I, I, I, D, P, I, I, I, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _p(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def page_bytes(bits: int, group: int = 128, head_dim: int = 128, is_v: bool = False) -> int:
    return int(lib().kvo_page_bytes(head_dim, bits, group, int(bool(is_v))))


def format_of_pools(k_pool: np.ndarray, v_pool: np.ndarray, head_dim: int = 128):
    """(key bits, value bits, group) whose page sizes match the pools' last dimension."""
    for group in (128, 64):
        for kb in (4, 8):
            for vb in (2, 4):
                if (page_bytes(kb, group, head_dim, False) == k_pool.shape[-1]
                        and page_bytes(vb, group, head_dim, True) == v_pool.shape[-1]):
                    return kb, vb, group
    raise ValueError("pools of %d / %d bytes per page match no format at head_dim %d"
                     % (k_pool.shape[-1], v_pool.shape[-1], head_dim))


def half_to_double(bits: np.ndarray) -> np.ndarray:
    f = lib().kvo_half_to_double
    return np.array([f(int(b)) for b in np.asarray(bits, dtype=np.uint16).ravel()]).reshape(np.shape(bits))


def double_to_half(x: np.ndarray) -> np.ndarray:
    f = lib().kvo_double_to_half
    return np.array([f(float(v)) for v in np.asarray(x, dtype=np.float64).ravel()],
                    dtype=np.uint16).reshape(np.shape(x))


def rotate(x: np.ndarray, fwht: bool = False) -> np.ndarray:
    x = _c(x, np.float64)
    rows, d = x.reshape(-1, x.shape[-1]).shape
    out = np.empty_like(x)
    assert lib().kvo_rotate(_p(x), rows, d, int(fwht), _p(out)) == 0
    return out


def normalize(r: np.ndarray, iters: int = 4, eps: float = 1e-6):
    r = _c(r, np.float64)
    rho, gam = np.empty(r.shape[0]), np.empty(r.shape[1])
    assert lib().kvo_normalize(_p(r), r.shape[0], r.shape[1], iters, eps, _p(rho), _p(gam)) == 0
    return rho, gam


def quantize_blocks(k16: np.ndarray, v16: np.ndarray, dst_pages, k_pool: np.ndarray, v_pool: np.ndarray,
                    fwht: bool = True, threads: int = 0) -> int:
    """k16, v16 fp16 [n_blocks*128, Hkv, D]; pools uint8 [num_pages, Hkv, page bytes], written in place (the
    page sizes give the format).  Returns the number of blocks whose page id is out of range (skipped)."""
    threads = threads or default_threads()
    n_tok, hkv, d = k16.shape
    kb, vb, group = format_of_pools(k_pool, v_pool, d)
    k = _c(k16, np.float16).view(np.uint16)
    v = _c(v16, np.float16).view(np.uint16)
    pages = _c(dst_pages, np.int32)
    assert k_pool.flags.c_contiguous and v_pool.flags.c_contiguous and k_pool.dtype == np.uint8
    bad = lib().kvo_quantize_blocks(_p(k), _p(v), n_tok // 128, hkv, d, _p(pages), _p(k_pool), _p(v_pool),
                                    k_pool.shape[0], kb, vb, group, int(fwht), threads)
    assert bad >= 0
    return int(bad)


def quantize_tile_page(x16: np.ndarray, is_v: bool, bits: int, group: int = 128, fwht: bool = False) -> bytes:
    """Page bytes of one fp16 tile [128, D]."""
    d = x16.shape[-1]
    x = _c(x16, np.float16).reshape(128, 1, d)
    kb, vb = (4, bits) if is_v else (bits, 2)
    kp = np.zeros((1, 1, page_bytes(kb, group, d, False)), np.uint8)
    vp = np.zeros((1, 1, page_bytes(vb, group, d, True)), np.uint8)
    assert lib().kvo_quantize_blocks(_p(x.view(np.uint16)), _p(x.view(np.uint16)), 1, 1, d,
                                     _p(np.zeros(1, np.int32)), _p(kp), _p(vp), 1, kb, vb, group, int(fwht), 1) == 0
    return (vp if is_v else kp)[0, 0].tobytes()


def dequantize_page(page, is_v: bool, bits: int, group: int = 128, head_dim: int = 128,
                    fwht: bool = True) -> np.ndarray:
    buf = np.frombuffer(bytes(page), dtype=np.uint8)
    assert buf.size == page_bytes(bits, group, head_dim, is_v)
    out = np.empty((128, head_dim))
    assert lib().kvo_dequantize_page(_p(buf), int(bool(is_v)), head_dim, bits, group, int(fwht), _p(out)) == 0
    return out


def decode(q16: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray, block_table: np.ndarray, seq_lens,
           num_kv_heads: int, softmax_scale: float = 0.0, k_tail=None, v_tail=None, pairs=None,
           fwht: bool = True, threads: int = 0) -> np.ndarray:
    """Decode attention -> fp64 [B, Hq, D]; rows outside ``pairs`` (a list of (sequence, query head)) are NaN.
    With fp16 tails k_tail, v_tail [B, 128, Hkv, D], the seq_lens % 128 tail rows follow the packed blocks."""
    threads = threads or default_threads()
    bsz, hq, d = q16.shape
    kb, vb, group = format_of_pools(k_pool, v_pool, d)
    q = _c(q16, np.float16).view(np.uint16)
    bt = _c(block_table, np.int32)
    if bt.ndim != 2 or bt.shape[1] == 0:
        bt = np.zeros((bsz, 1), np.int32) - 1
    sl = _c(seq_lens, np.int32)
    kt = None if k_tail is None else _c(k_tail, np.float16).view(np.uint16)
    vt = None if v_tail is None else _c(v_tail, np.float16).view(np.uint16)
    pr = None if pairs is None else _c(np.asarray(pairs, dtype=np.int32).reshape(-1, 2), np.int32)
    out = np.full((bsz, hq, d), np.nan)
    assert k_pool.flags.c_contiguous and v_pool.flags.c_contiguous
    rc = lib().kvo_decode(_p(q), _p(k_pool), _p(v_pool), k_pool.shape[0], _p(bt), bt.shape[1], _p(sl), _p(kt),
                          _p(vt), bsz, hq, num_kv_heads, d, kb, vb, group, float(softmax_scale), _p(pr),
                          0 if pr is None else pr.shape[0], int(fwht), threads, _p(out))
    assert rc == 0
    return out
