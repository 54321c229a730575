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
           "kvarn_decode_workspace_bytes", "kvarn_decode_attention", "kvarn_decode_attention_noalloc",
           "kvarn_decode_attention_tail",
           "kvarn_fp16_page_bytes",
           "kvarn_fp16_decode_attention", "kvarn_prefill_attention", "kvarn_read_flags", "kvarn_set_debug_checks",
           "kvarn_status_string", "kvarn_last_error")

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
        "kvarn_decode_attention_noalloc": (I32, [CFG, P, P, P, I32, P, I32, P, I32, I32, I32, F32, P, P, P]),
        "kvarn_decode_attention_tail": (I32, [CFG, P, P, P, I32, P, I32, P, P, P, I32, I32, I32, F32, P, P, SZ, P, P]),
        "kvarn_fp16_page_bytes": (SZ, [CFG]),
        "kvarn_fp16_decode_attention": (I32, [CFG, P, P, P, I32, P, I32, P, I32, I32, I32, F32, P, P, SZ, P, P]),
        "kvarn_prefill_attention": (I32, [CFG, P, I32, P, P, I32, P, I32, P, P, P, I32, P, P, I32, I32, I32, F32, P,
                                          P, P]),
        "kvarn_read_flags": (I32, [P, P, P]),
        "kvarn_set_debug_checks": (None, [ctypes.c_int]),
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


def _need(t: Optional[torch.Tensor], name: str, dtype: torch.dtype, shape=None, optional: bool = False) -> None:
    """Reject an argument the C entry points would misread: wrong dtype, shape or layout.

    ``shape`` lists the expected sizes, None for a size the caller is free to choose.  Each entry point
    checks the device of its tensors (``_on_gpu``) after all of these, so that the layout rules can be
    exercised with host tensors."""
    if t is None:
        if optional:
            return
        raise ValueError("%s is required" % name)
    if t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if shape is not None:
        if t.dim() != len(shape) or any(e is not None and int(a) != int(e) for a, e in zip(t.shape, shape)):
            raise ValueError("%s must have shape %s, got %s"
                             % (name, tuple("*" if e is None else int(e) for e in shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _on_gpu(**tensors) -> None:
    """Every tensor argument (None for an omitted optional one) must be in GPU memory."""
    for name, t in tensors.items():
        if t is not None and t.device.type != "cuda":
            raise ValueError("%s must be in GPU memory, got %s" % (name, t.device))


def _need_pools(cfg, k_pool: torch.Tensor, v_pool: torch.Tensor, hkv: Optional[int] = None) -> None:
    """Pools are uint8 [num_pages, Hkv, page_bytes] with the config's page sizes and equal page counts."""
    _need(k_pool, "k_pool", torch.uint8, (None, hkv, kvarn_page_bytes(cfg, False)))
    _need(v_pool, "v_pool", torch.uint8, (k_pool.shape[0], k_pool.shape[1], kvarn_page_bytes(cfg, True)))


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _need_decode(q, block_table, seq_lens, num_kv_heads, out, workspace, dev_flags, head_dim: int = 128) -> None:
    """Arguments every decode entry point shares: q fp16 [B, Hq, D], block_table int32 [B, max_blocks],
    seq_lens int32 [B], out fp32 [B, Hq, D], a byte workspace and optional int32 flags."""
    _need(q, "q", torch.float16, (None, None, head_dim))
    batch, hq = q.shape[0], q.shape[1]
    if num_kv_heads <= 0 or hq % num_kv_heads:
        raise ValueError("%d query heads are not a multiple of %d KV heads" % (hq, num_kv_heads))
    _need(block_table, "block_table", torch.int32, (batch, None))
    _need(seq_lens, "seq_lens", torch.int32, (batch,))
    _need(out, "out", torch.float32, (batch, hq, head_dim))
    _need(workspace, "workspace", torch.uint8, (None,))
    _need(dev_flags, "dev_flags", torch.int32, None, optional=True)


def kvarn_config_parse(name: str = "kvarn_k4v2_g128", head_dim: int = 128) -> kvarn_config:
    """The format of a cache dtype name, for heads of `head_dim` channels (the name carries no head size;
    the library parses it with head_dim 128, and 64 and 256 are the other sizes it builds)."""
    cfg = kvarn_config()
    _check(_lib.kvarn_config_parse(name.encode(), ctypes.byref(cfg)))
    cfg.head_dim = head_dim
    if _lib.kvarn_page_bytes(ctypes.byref(cfg), 0) == 0:
        raise KvarnError(KVARN_ERR_UNSUPPORTED, "head_dim %d is not supported (64, 128 or 256)" % head_dim)
    return cfg


def kvarn_page_bytes(cfg: kvarn_config, is_v: bool) -> int:
    return int(_lib.kvarn_page_bytes(ctypes.byref(cfg), int(bool(is_v))))


def kvarn_quantize_blocks(cfg, k: torch.Tensor, v: torch.Tensor, dst_pages: torch.Tensor, k_pool: torch.Tensor,
                          v_pool: torch.Tensor, dev_flags: Optional[torch.Tensor] = None, stream=None) -> None:
    """k, v: fp16 [n_blocks*128, Hkv, D]; dst_pages int32 [n_blocks]; pools uint8 [pages, Hkv, page_bytes]."""
    _need(k, "k", torch.float16, (None, None, cfg.head_dim))
    n_tok, hkv = k.shape[0], k.shape[1]
    if n_tok % 128:
        raise ValueError("k holds %d tokens, not a whole number of 128-token blocks" % n_tok)
    _need(v, "v", torch.float16, (n_tok, hkv, cfg.head_dim))
    _need(dst_pages, "dst_pages", torch.int32, (n_tok // 128,))
    _need_pools(cfg, k_pool, v_pool, hkv)
    _need(dev_flags, "dev_flags", torch.int32, None, optional=True)
    _on_gpu(k=k, v=v, dst_pages=dst_pages, k_pool=k_pool, v_pool=v_pool, dev_flags=dev_flags)
    _check(_lib.kvarn_quantize_blocks(ctypes.byref(cfg), _ptr(k), _ptr(v), n_tok // 128, hkv, _ptr(dst_pages),
                                      _ptr(k_pool), _ptr(v_pool), k_pool.shape[0], _ptr(dev_flags), _stream(stream)))


def kvarn_dequantize_blocks(cfg, k_pool: torch.Tensor, v_pool: torch.Tensor, pages: torch.Tensor,
                            k_out: Optional[torch.Tensor], v_out: Optional[torch.Tensor],
                            dev_flags: Optional[torch.Tensor] = None, stream=None) -> None:
    """k_out, v_out: fp32 [n_blocks*128, Hkv, D] (either may be None); pages int32 [n_blocks]."""
    out = k_out if k_out is not None else v_out
    if out is None:
        raise ValueError("at least one of k_out and v_out is required")
    _need(pages, "pages", torch.int32, (None,))
    shape = (128 * pages.shape[0], k_pool.shape[1], cfg.head_dim)
    _need(k_out, "k_out", torch.float32, shape, optional=True)
    _need(v_out, "v_out", torch.float32, shape, optional=True)
    _need_pools(cfg, k_pool, v_pool)
    _need(dev_flags, "dev_flags", torch.int32, None, optional=True)
    hkv = out.shape[1]
    _on_gpu(k_pool=k_pool, v_pool=v_pool, pages=pages, k_out=k_out, v_out=v_out, dev_flags=dev_flags)
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
    """q fp16 [B, Hq, D]; block_table int32 [B, max_blocks]; seq_lens int32 [B]; out fp32 [B, Hq, D]."""
    _need_decode(q, block_table, seq_lens, num_kv_heads, out, workspace, dev_flags, cfg.head_dim)
    _need_pools(cfg, k_pool, v_pool, num_kv_heads)
    batch, hq = q.shape[0], q.shape[1]
    _on_gpu(q=q, k_pool=k_pool, v_pool=v_pool, block_table=block_table, seq_lens=seq_lens, out=out,
            workspace=workspace, dev_flags=dev_flags)
    _check(_lib.kvarn_decode_attention(ctypes.byref(cfg), _ptr(q), _ptr(k_pool), _ptr(v_pool), k_pool.shape[0],
                                       _ptr(block_table), block_table.shape[1], _ptr(seq_lens), batch, hq,
                                       num_kv_heads, float(softmax_scale), _ptr(out), _ptr(workspace),
                                       workspace.numel() * workspace.element_size(), _ptr(dev_flags),
                                       _stream(stream)))


def kvarn_decode_attention_noalloc(cfg, q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                                   block_table: torch.Tensor, seq_lens: torch.Tensor, num_kv_heads: int,
                                   out: torch.Tensor, softmax_scale: float = 0.0,
                                   dev_flags: Optional[torch.Tensor] = None, stream=None) -> None:
    """kvarn_decode_attention with the library's fixed scratch memory instead of a workspace."""
    _need_decode(q, block_table, seq_lens, num_kv_heads, out, torch.zeros(0, dtype=torch.uint8), dev_flags,
                 cfg.head_dim)
    _need_pools(cfg, k_pool, v_pool, num_kv_heads)
    _on_gpu(q=q, k_pool=k_pool, v_pool=v_pool, block_table=block_table, seq_lens=seq_lens, out=out,
            dev_flags=dev_flags)
    batch, hq = q.shape[0], q.shape[1]
    _check(_lib.kvarn_decode_attention_noalloc(ctypes.byref(cfg), _ptr(q), _ptr(k_pool), _ptr(v_pool), k_pool.shape[0],
                                               _ptr(block_table), block_table.shape[1], _ptr(seq_lens), batch, hq,
                                               num_kv_heads, float(softmax_scale), _ptr(out), _ptr(dev_flags),
                                               _stream(stream)))


def kvarn_decode_attention_tail(cfg, q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                                block_table: torch.Tensor, seq_lens: torch.Tensor, k_tail: torch.Tensor,
                                v_tail: torch.Tensor, num_kv_heads: int, out: torch.Tensor, workspace: torch.Tensor,
                                softmax_scale: float = 0.0, dev_flags: Optional[torch.Tensor] = None,
                                stream=None) -> None:
    """As kvarn_decode_attention, plus fp16 tails k_tail, v_tail [B, 128, Hkv, 128] holding seq_lens % 128 tokens."""
    _need_decode(q, block_table, seq_lens, num_kv_heads, out, workspace, dev_flags)
    _need_pools(cfg, k_pool, v_pool, num_kv_heads)
    _need(k_tail, "k_tail", torch.float16, (q.shape[0], 128, num_kv_heads, 128))
    _need(v_tail, "v_tail", torch.float16, (q.shape[0], 128, num_kv_heads, 128))
    batch, hq = q.shape[0], q.shape[1]
    _on_gpu(q=q, k_pool=k_pool, v_pool=v_pool, block_table=block_table, seq_lens=seq_lens, k_tail=k_tail,
            v_tail=v_tail, out=out, workspace=workspace, dev_flags=dev_flags)
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
    _need_decode(q, block_table, seq_lens, num_kv_heads, out, workspace, dev_flags)
    _need(k_cache, "k_cache", torch.float16, (None, num_kv_heads, 128, 128))
    _need(v_cache, "v_cache", torch.float16, (k_cache.shape[0], num_kv_heads, 128, 128))
    batch, hq = q.shape[0], q.shape[1]
    _on_gpu(q=q, k_cache=k_cache, v_cache=v_cache, block_table=block_table, seq_lens=seq_lens, out=out,
            workspace=workspace, dev_flags=dev_flags)
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
    _need(q, "q", torch.float16, (None, None, None, 128))
    batch, max_q, hq = q.shape[0], q.shape[1], q.shape[2]
    if num_kv_heads <= 0 or hq % num_kv_heads:
        raise ValueError("%d query heads are not a multiple of %d KV heads" % (hq, num_kv_heads))
    _need_pools(cfg, k_pool, v_pool, num_kv_heads)
    _need(block_table, "block_table", torch.int32, (batch, None))
    for name, t in (("prefix_lens", prefix_lens), ("new_lens", new_lens), ("q_lens", q_lens)):
        _need(t, name, torch.int32, (batch,))
    _need(k_new, "k_new", torch.float16, (batch, None, num_kv_heads, 128))
    _need(v_new, "v_new", torch.float16, tuple(k_new.shape))
    _need(out, "out", torch.float32, (batch, max_q, hq, 128))
    _need(dev_flags, "dev_flags", torch.int32, None, optional=True)
    _on_gpu(q=q, k_pool=k_pool, v_pool=v_pool, block_table=block_table, prefix_lens=prefix_lens, k_new=k_new,
            v_new=v_new, new_lens=new_lens, q_lens=q_lens, out=out, dev_flags=dev_flags)
    _check(_lib.kvarn_prefill_attention(ctypes.byref(cfg), _ptr(q), max_q, _ptr(k_pool), _ptr(v_pool), k_pool.shape[0],
                                        _ptr(block_table), block_table.shape[1], _ptr(prefix_lens), _ptr(k_new),
                                        _ptr(v_new), k_new.shape[1], _ptr(new_lens), _ptr(q_lens), batch, hq,
                                        num_kv_heads, float(softmax_scale), _ptr(out), _ptr(dev_flags),
                                        _stream(stream)))


def kvarn_read_flags(dev_flags: torch.Tensor, stream=None) -> int:
    host = ctypes.c_uint32(0)
    _check(_lib.kvarn_read_flags(_ptr(dev_flags), ctypes.byref(host), _stream(stream)))
    return int(host.value)


def kvarn_set_debug_checks(on: bool) -> None:
    """Process-wide debug checks: while on, kvarn_quantize_blocks raises KvarnError (SHAPE) when two
    entries of dst_pages name the same page, before anything is written (it waits for the stream)."""
    _lib.kvarn_set_debug_checks(1 if on else 0)


# ---- allocation helpers (device memory through torch) ----------------------
def alloc_pools(cfg, num_pages: int, hkv: int, device="cuda"):
    kb, vb = kvarn_page_bytes(cfg, False), kvarn_page_bytes(cfg, True)
    return (torch.empty((num_pages, hkv, kb), dtype=torch.uint8, device=device),
            torch.empty((num_pages, hkv, vb), dtype=torch.uint8, device=device))


def alloc_workspace(cfg, batch: int, hq: int, hkv: int, max_blocks: int, device="cuda") -> torch.Tensor:
    """Zero-filled workspace (the arrival counters must start at zero)."""
    nbytes = max(kvarn_decode_workspace_bytes(cfg, batch, hq, hkv, max_blocks), 256)
    return torch.zeros(nbytes, dtype=torch.uint8, device=device)
