"""ctypes binding of libkvarn.so: argument marshalling only.

Every function mirrors the C entry point of the same name in include/kvarn.h.
Tensors are torch tensors on the GPU; the binding passes their data pointers
and the current HIP stream, checks the returned status and raises
``KvarnError`` on failure.  All computation happens in the HIP kernels; there
is no fallback: if the library is missing, importing this module fails.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvarn.so")


class KvarnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("libkvarn status %d: %s" % (status, message))
        self.status = status


class kvarn_config(ctypes.Structure):
    _fields_ = [("head_dim", ctypes.c_int32), ("block_tokens", ctypes.c_int32), ("k_bits", ctypes.c_int32),
                ("v_bits", ctypes.c_int32), ("group_size", ctypes.c_int32), ("norm_iters", ctypes.c_int32),
                ("eps", ctypes.c_float)]


EXPORTS = ("kvarn_config_parse", "kvarn_page_bytes", "kvarn_quantize_blocks", "kvarn_dequantize_blocks",
           "kvarn_decode_workspace_bytes", "kvarn_decode_attention", "kvarn_decode_attention_tail",
           "kvarn_fp16_page_bytes",
           "kvarn_fp16_decode_attention", "kvarn_prefill_attention", "kvarn_read_flags", "kvarn_status_string",
           "kvarn_last_error")

KVARN_OK, KVARN_ERR_NULL, KVARN_ERR_SHAPE, KVARN_ERR_UNSUPPORTED, KVARN_ERR_WORKSPACE, KVARN_ERR_LAUNCH = 0, -1, -2, -3, -4, -5
FLAG_BAD_PAGE, FLAG_BAD_SEQLEN = 1, 2


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError("libkvarn.so is not built (%s); run kv_cache_quantization_kvarn_amd.build" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, SZ, F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
    CFG = ctypes.POINTER(kvarn_config)
    sig = {
        "kvarn_config_parse": (I32, [ctypes.c_char_p, CFG]),
        "kvarn_page_bytes": (SZ, [CFG, ctypes.c_int]),
        "kvarn_quantize_blocks": (I32, [CFG, P, P, I32, I32, P, P, P, I32, P, P]),
        "kvarn_dequantize_blocks": (I32, [CFG, P, P, I32, P, I32, I32, P, P, P, P]),
        "kvarn_decode_workspace_bytes": (SZ, [CFG, I32, I32, I32, I32]),
        "kvarn_decode_attention": (I32, [CFG, P, P, P, I32, P, I32, P, I32, I32, I32, F32, P, P, SZ, P, P]),
        "kvarn_decode_attention_tail": (I32, [CFG, P, P, P, I32, P, I32, P, P, P, I32, I32, I32, F32, P, P, SZ, P, P]),
        "kvarn_fp16_page_bytes": (SZ, [CFG]),
        "kvarn_fp16_decode_attention": (I32, [CFG, P, P, P, I32, P, I32, P, I32, I32, I32, F32, P, P, SZ, P, P]),
        "kvarn_prefill_attention": (I32, [CFG, P, I32, P, P, I32, P, I32, P, P, P, I32, P, P, I32, I32, I32, F32, P,
                                          P, P]),
        "kvarn_read_flags": (I32, [P, P, P]),
        "kvarn_status_string": (ctypes.c_char_p, [I32]),
        "kvarn_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def library() -> ctypes.CDLL:
    return _lib


def _check(status: int) -> None:
    if status != KVARN_OK:
        raise KvarnError(status, _lib.kvarn_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def kvarn_config_parse(name: str = "kvarn_k4v2_g128") -> kvarn_config:
    cfg = kvarn_config()
    _check(_lib.kvarn_config_parse(name.encode(), ctypes.byref(cfg)))
    return cfg


def kvarn_page_bytes(cfg: kvarn_config, is_v: bool) -> int:
    return int(_lib.kvarn_page_bytes(ctypes.byref(cfg), int(bool(is_v))))


def kvarn_quantize_blocks(cfg, k: torch.Tensor, v: torch.Tensor, dst_pages: torch.Tensor, k_pool: torch.Tensor,
                          v_pool: torch.Tensor, dev_flags: Optional[torch.Tensor] = None, stream=None) -> None:
    """k, v: fp16 [n_blocks*128, Hkv, 128]; dst_pages int32 [n_blocks]; pools uint8 [pages, Hkv, page_bytes]."""
    n_tok, hkv = k.shape[0], k.shape[1]
    _check(_lib.kvarn_quantize_blocks(ctypes.byref(cfg), _ptr(k), _ptr(v), n_tok // 128, hkv, _ptr(dst_pages),
                                      _ptr(k_pool), _ptr(v_pool), k_pool.shape[0], _ptr(dev_flags), _stream(stream)))


def kvarn_dequantize_blocks(cfg, k_pool: torch.Tensor, v_pool: torch.Tensor, pages: torch.Tensor,
                            k_out: Optional[torch.Tensor], v_out: Optional[torch.Tensor],
                            dev_flags: Optional[torch.Tensor] = None, stream=None) -> None:
    out = k_out if k_out is not None else v_out
    hkv = out.shape[1]
    _check(_lib.kvarn_dequantize_blocks(ctypes.byref(cfg), _ptr(k_pool), _ptr(v_pool), k_pool.shape[0], _ptr(pages),
                                        pages.shape[0], hkv, _ptr(k_out), _ptr(v_out), _ptr(dev_flags),
                                        _stream(stream)))


def kvarn_decode_workspace_bytes(cfg, batch: int, num_q_heads: int, num_kv_heads: int, max_blocks_per_seq: int) -> int:
    return int(_lib.kvarn_decode_workspace_bytes(ctypes.byref(cfg), batch, num_q_heads, num_kv_heads,
                                                 max_blocks_per_seq))


def kvarn_decode_attention(cfg, q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                           block_table: torch.Tensor, seq_lens: torch.Tensor, num_kv_heads: int, out: torch.Tensor,
                           workspace: torch.Tensor, softmax_scale: float = 0.0,
                           dev_flags: Optional[torch.Tensor] = None, stream=None) -> None:
    """q fp16 [B, Hq, 128]; block_table int32 [B, max_blocks]; seq_lens int32 [B]; out fp32 [B, Hq, 128]."""
    batch, hq = q.shape[0], q.shape[1]
    _check(_lib.kvarn_decode_attention(ctypes.byref(cfg), _ptr(q), _ptr(k_pool), _ptr(v_pool), k_pool.shape[0],
                                       _ptr(block_table), block_table.shape[1], _ptr(seq_lens), batch, hq,
                                       num_kv_heads, float(softmax_scale), _ptr(out), _ptr(workspace),
                                       workspace.numel() * workspace.element_size(), _ptr(dev_flags),
                                       _stream(stream)))


def kvarn_decode_attention_tail(cfg, q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                                block_table: torch.Tensor, seq_lens: torch.Tensor, k_tail: torch.Tensor,
                                v_tail: torch.Tensor, num_kv_heads: int, out: torch.Tensor, workspace: torch.Tensor,
                                softmax_scale: float = 0.0, dev_flags: Optional[torch.Tensor] = None,
                                stream=None) -> None:
    """As kvarn_decode_attention, plus fp16 tails k_tail, v_tail [B, 128, Hkv, 128] holding seq_lens % 128 tokens."""
    batch, hq = q.shape[0], q.shape[1]
    _check(_lib.kvarn_decode_attention_tail(ctypes.byref(cfg), _ptr(q), _ptr(k_pool), _ptr(v_pool), k_pool.shape[0],
                                            _ptr(block_table), block_table.shape[1], _ptr(seq_lens), _ptr(k_tail),
                                            _ptr(v_tail), batch, hq, num_kv_heads, float(softmax_scale), _ptr(out),
                                            _ptr(workspace), workspace.numel() * workspace.element_size(),
                                            _ptr(dev_flags), _stream(stream)))


def kvarn_fp16_page_bytes(cfg) -> int:
    return int(_lib.kvarn_fp16_page_bytes(ctypes.byref(cfg)))


def kvarn_fp16_decode_attention(cfg, q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                                block_table: torch.Tensor, seq_lens: torch.Tensor, num_kv_heads: int,
                                out: torch.Tensor, workspace: torch.Tensor, softmax_scale: float = 0.0,
                                dev_flags: Optional[torch.Tensor] = None, stream=None) -> None:
    """The fp16 baseline: k_cache, v_cache fp16 [num_pages, Hkv, 128, 128]; other arguments as kvarn_decode_attention."""
    batch, hq = q.shape[0], q.shape[1]
    _check(_lib.kvarn_fp16_decode_attention(ctypes.byref(cfg), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                            k_cache.shape[0], _ptr(block_table), block_table.shape[1],
                                            _ptr(seq_lens), batch, hq, num_kv_heads, float(softmax_scale), _ptr(out),
                                            _ptr(workspace), workspace.numel() * workspace.element_size(),
                                            _ptr(dev_flags), _stream(stream)))


def kvarn_prefill_attention(cfg, q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                            block_table: torch.Tensor, prefix_lens: torch.Tensor, k_new: torch.Tensor,
                            v_new: torch.Tensor, new_lens: torch.Tensor, q_lens: torch.Tensor, num_kv_heads: int,
                            out: torch.Tensor, softmax_scale: float = 0.0, dev_flags: Optional[torch.Tensor] = None,
                            stream=None) -> None:
    """Chunked prefill: q fp16 [B, max_q, Hq, 128] over packed pages and fp16 rows k_new, v_new [B, max_new, Hkv, 128]."""
    batch, max_q, hq = q.shape[0], q.shape[1], q.shape[2]
    _check(_lib.kvarn_prefill_attention(ctypes.byref(cfg), _ptr(q), max_q, _ptr(k_pool), _ptr(v_pool), k_pool.shape[0],
                                        _ptr(block_table), block_table.shape[1], _ptr(prefix_lens), _ptr(k_new),
                                        _ptr(v_new), k_new.shape[1], _ptr(new_lens), _ptr(q_lens), batch, hq,
                                        num_kv_heads, float(softmax_scale), _ptr(out), _ptr(dev_flags),
                                        _stream(stream)))


def kvarn_read_flags(dev_flags: torch.Tensor, stream=None) -> int:
    host = ctypes.c_uint32(0)
    _check(_lib.kvarn_read_flags(_ptr(dev_flags), ctypes.byref(host), _stream(stream)))
    return int(host.value)


# ---- allocation helpers (device memory through torch) ----------------------
def alloc_pools(cfg, num_pages: int, hkv: int, device="cuda"):
    kb, vb = kvarn_page_bytes(cfg, False), kvarn_page_bytes(cfg, True)
    return (torch.empty((num_pages, hkv, kb), dtype=torch.uint8, device=device),
            torch.empty((num_pages, hkv, vb), dtype=torch.uint8, device=device))


def alloc_workspace(cfg, batch: int, hq: int, hkv: int, max_blocks: int, device="cuda") -> torch.Tensor:
    """Zero-filled workspace (the arrival counters must start at zero)."""
    nbytes = max(kvarn_decode_workspace_bytes(cfg, batch, hq, hkv, max_blocks), 256)
    return torch.zeros(nbytes, dtype=torch.uint8, device=device)
