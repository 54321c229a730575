"""Host-side checks of the C ABI that need no GPU: exports, config parsing, page
sizes, argument validation (every rejected call returns before any HIP call)
and the benchmark's byte accounting against the pages' printed figures."""
import ctypes
import os
import re

import pytest

from kv_cache_quantization_kvarn_amd import accounting
from kv_cache_quantization_kvarn_amd import kvarn as K

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "kvarn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kvarn_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    names = header_functions()
    assert len(names) >= 9
    lib = ctypes.CDLL(K.LIB_PATH)
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(K.EXPORTS)


def test_config_parse():
    cfg = K.kvarn_config_parse("kvarn_k4v2_g128")
    assert (cfg.head_dim, cfg.block_tokens, cfg.k_bits, cfg.v_bits, cfg.group_size, cfg.norm_iters) == \
        (128, 128, 4, 2, 128, 4)
    assert abs(cfg.eps - 1e-6) < 1e-12
    for kb, vb in ((4, 2), (4, 4), (8, 2), (8, 4)):
        for gs in (128, 64):
            c = K.kvarn_config_parse("kvarn_k%dv%d_g%d" % (kb, vb, gs))
            assert (c.k_bits, c.v_bits, c.group_size) == (kb, vb, gs)
    for bad in ("kvarn_k8v4_g32", "kvarn_k4v2_g256", "kvarn_k4v2_g128x", "fp8", "kvarn_k4v2", "kvarn_k2v2_g128",
                "kvarn_k4v8_g128", "kvarn_k16v4_g128"):
        with pytest.raises(K.KvarnError) as e:
            K.kvarn_config_parse(bad)
        assert e.value.status == K.KVARN_ERR_UNSUPPORTED
    lib = K.library()
    assert lib.kvarn_config_parse(None, None) == K.KVARN_ERR_NULL


def test_page_bytes_match_the_oracle_format():
    from oracle import kvarn_oracle as o
    cfg = K.kvarn_config_parse()
    assert K.kvarn_page_bytes(cfg, False) == o.K_PAGE_BYTES == 9728
    assert K.kvarn_page_bytes(cfg, True) == o.V_PAGE_BYTES == 5632
    for kb, vb in ((4, 2), (4, 4), (8, 2), (8, 4)):
        for gs in (128, 64):
            c = K.kvarn_config_parse("kvarn_k%dv%d_g%d" % (kb, vb, gs))
            assert K.kvarn_page_bytes(c, False) == o.page_bytes(kb, gs)
            assert K.kvarn_page_bytes(c, True) == o.page_bytes(vb, gs)
    assert (o.page_bytes(8), o.page_bytes(4)) == (17920, 9728)
    assert (o.page_bytes(4, 64), o.page_bytes(2, 64)) == (10240, 6144)
    bad = K.kvarn_config()
    assert K.kvarn_page_bytes(bad, False) == 0


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first


def quant(cfg, k=FAKE, v=FAKE, n=1, h=8, pages=FAKE, kp=FAKE, vp=FAKE, npages=4):
    return K.library().kvarn_quantize_blocks(ctypes.byref(cfg) if cfg is not None else None, k, v, n, h, pages, kp,
                                             vp, npages, None, None)


def test_quantize_validation():
    cfg = K.kvarn_config_parse()
    assert quant(None) == K.KVARN_ERR_NULL
    assert quant(K.kvarn_config()) == K.KVARN_ERR_UNSUPPORTED
    assert quant(cfg, n=-1) == K.KVARN_ERR_SHAPE
    assert quant(cfg, h=0) == K.KVARN_ERR_SHAPE
    assert quant(cfg, n=0) == K.KVARN_OK  # empty call is a no-op
    assert quant(cfg, k=None) == K.KVARN_ERR_NULL
    assert quant(cfg, pages=None) == K.KVARN_ERR_NULL
    assert quant(cfg, npages=0) == K.KVARN_ERR_SHAPE
    assert quant(cfg, k=ctypes.c_void_p(0x1004)) == K.KVARN_ERR_SHAPE  # misaligned
    assert "aligned" in K.library().kvarn_last_error().decode()


def decode(cfg, q=FAKE, kp=FAKE, vp=FAKE, npages=4, bt=FAKE, mb=2, sl=FAKE, b=1, hq=32, hkv=8, out=FAKE,
           ws=ctypes.c_void_p(0x10000), wsb=1 << 30):
    return K.library().kvarn_decode_attention(ctypes.byref(cfg), q, kp, vp, npages, bt, mb, sl, b, hq, hkv, 0.0, out,
                                              ws, wsb, None, None)


def test_decode_validation():
    cfg = K.kvarn_config_parse()
    assert decode(cfg, hq=30) == K.KVARN_ERR_SHAPE          # not a multiple of Hkv
    assert decode(cfg, hq=128, hkv=8) == K.KVARN_ERR_UNSUPPORTED  # 16 query heads per KV head
    assert decode(cfg, b=-1) == K.KVARN_ERR_SHAPE
    assert decode(cfg, b=0) == K.KVARN_OK
    assert decode(cfg, q=None) == K.KVARN_ERR_NULL
    assert decode(cfg, bt=None) == K.KVARN_ERR_NULL
    assert decode(cfg, wsb=16) == K.KVARN_ERR_WORKSPACE
    assert decode(cfg, ws=None) == K.KVARN_ERR_WORKSPACE
    assert decode(cfg, ws=ctypes.c_void_p(0x10010)) == K.KVARN_ERR_WORKSPACE  # not 256-byte aligned
    assert decode(cfg, kp=ctypes.c_void_p(0x1002)) == K.KVARN_ERR_SHAPE
    assert decode(cfg, q=ctypes.c_void_p(0x1004)) == K.KVARN_ERR_SHAPE   # q not 16-byte aligned
    assert decode(cfg, out=ctypes.c_void_p(0x1008)) == K.KVARN_ERR_SHAPE  # out not 16-byte aligned
    assert decode(cfg, npages=0) == K.KVARN_ERR_SHAPE                     # pages referenced, none exist


def test_workspace_sizes():
    cfg = K.kvarn_config_parse()
    a = K.kvarn_decode_workspace_bytes(cfg, 16, 32, 8, 64)
    b = K.kvarn_decode_workspace_bytes(cfg, 16, 32, 8, 1024)
    assert a > 0 and b >= a
    assert K.kvarn_decode_workspace_bytes(cfg, 0, 32, 8, 64) == 0
    assert K.kvarn_decode_workspace_bytes(cfg, 4, 32, 8, 0) > 0  # empty tables still need the counters
    assert K.kvarn_decode_workspace_bytes(K.kvarn_config(), 16, 32, 8, 64) == 0


def test_status_strings():
    lib = K.library()
    for s in range(-5, 1):
        assert lib.kvarn_status_string(s)


def golden():
    vals = {}
    for line in open(os.path.join(ROOT, "tests", "golden", "page_figures.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split(None, 1)
            vals[k] = v
    return vals


def test_byte_accounting_reproduces_page_figures():
    g = golden()
    cfg = K.kvarn_config_parse(g["format_name"])
    kb, vb = K.kvarn_page_bytes(cfg, False), K.kvarn_page_bytes(cfg, True)
    ratio = accounting.capacity_ratio(kb, vb)
    assert float(g["capacity_ratio_vs_fp16_min"]) <= ratio <= float(g["capacity_ratio_vs_fp16_max"])
    # 7B-class model at 4096 tokens: about 500 MB
    b7 = accounting.fp16_kv_bytes(int(g["kv7b_layers"]), int(g["kv7b_kv_heads"]), int(g["kv7b_tokens"]))
    assert abs(b7 / 1e6 - float(g["kv7b_approx_mb"])) / float(g["kv7b_approx_mb"]) < 0.1
    # Qwen2.5-1.5B: about 29 KB per token
    per_tok = accounting.fp16_kv_bytes(int(g["qwen_layers"]), int(g["qwen_kv_heads"]), 1)
    assert abs(per_tok / 1000 - float(g["qwen_kb_per_token"])) / float(g["qwen_kb_per_token"]) < 0.05
    # quantize moves 64 KiB of fp16 in and one K+V page pair out per (block, KV head)
    assert accounting.quantize_bytes(1, 1, kb, vb) == 65536 + 15360


def test_fp16_decode_validation():
    cfg = K.kvarn_config_parse()
    assert K.kvarn_fp16_page_bytes(cfg) == 32768
    assert K.kvarn_fp16_page_bytes(K.kvarn_config()) == 0

    def f16(q=FAKE, kc=FAKE, vc=FAKE, npages=4, bt=FAKE, mb=2, sl=FAKE, b=1, hq=32, hkv=8, out=FAKE,
            ws=ctypes.c_void_p(0x10000), wsb=1 << 30):
        return K.library().kvarn_fp16_decode_attention(ctypes.byref(cfg), q, kc, vc, npages, bt, mb, sl, b, hq, hkv,
                                                       0.0, out, ws, wsb, None, None)

    assert f16(hq=30) == K.KVARN_ERR_SHAPE
    assert f16(hq=128, hkv=8) == K.KVARN_ERR_UNSUPPORTED
    assert f16(b=0) == K.KVARN_OK
    assert f16(kc=None) == K.KVARN_ERR_NULL
    assert f16(wsb=16) == K.KVARN_ERR_WORKSPACE
    assert f16(vc=ctypes.c_void_p(0x1002)) == K.KVARN_ERR_SHAPE
    assert f16(q=ctypes.c_void_p(0x1004)) == K.KVARN_ERR_SHAPE
    assert f16(npages=0) == K.KVARN_ERR_SHAPE


def test_prefill_validation():
    cfg = K.kvarn_config_parse()

    def pf(q=FAKE, mq=64, kp=FAKE, vp=FAKE, npages=4, bt=FAKE, mb=2, pl=FAKE, kn=FAKE, vn=FAKE, mn=64, nl=FAKE,
           ql=FAKE, b=1, hq=32, hkv=8, out=FAKE):
        return K.library().kvarn_prefill_attention(ctypes.byref(cfg), q, mq, kp, vp, npages, bt, mb, pl, kn, vn, mn,
                                                   nl, ql, b, hq, hkv, 0.0, out, None, None)

    # every call below either fails validation or has no work: nothing is launched
    assert pf(hq=30) == K.KVARN_ERR_SHAPE
    assert pf(hq=128, hkv=8) == K.KVARN_ERR_UNSUPPORTED
    assert pf(b=0) == K.KVARN_OK
    assert pf(mq=0) == K.KVARN_OK
    assert pf(mq=-1) == K.KVARN_ERR_SHAPE
    assert pf(mn=-1) == K.KVARN_ERR_SHAPE
    assert pf(ql=None) == K.KVARN_ERR_NULL
    assert pf(kn=None) == K.KVARN_ERR_NULL
    assert pf(bt=None) == K.KVARN_ERR_NULL
    assert pf(npages=0) == K.KVARN_ERR_SHAPE
    assert pf(mb=1 << 24) == K.KVARN_ERR_SHAPE
    assert pf(b=70000) == K.KVARN_ERR_SHAPE
    assert pf(q=ctypes.c_void_p(0x1008)) == K.KVARN_ERR_SHAPE
    assert pf(vn=ctypes.c_void_p(0x1002)) == K.KVARN_ERR_SHAPE
    assert pf(kp=ctypes.c_void_p(0x1004)) == K.KVARN_ERR_SHAPE
    assert pf(out=ctypes.c_void_p(0x1001)) == K.KVARN_ERR_SHAPE


def test_prefill_accounting_matches_brute_force():
    prefix, new, q, hq = [256, 0, 384], [40, 7, 130], [25, 7, 1], 6
    brute = sum(p + (n - k) + i + 1 for p, n, k in zip(prefix, new, q) for i in range(k)) * hq
    assert accounting.prefill_pairs(prefix, new, q, hq) == brute
    assert accounting.prefill_flops(brute) == 4 * 128 * brute


def test_tail_accounting_adds_one_k_and_one_v_row_per_tail_token():
    base = accounting.decode_bytes(640, 8, 5, 32, 9728, 5632)
    # 5 sequences with tails of 1..5 tokens, 8 KV heads: fp16 rows of 128 channels for K and for V
    tail = accounting.tail_decode_bytes(640, 8, 5, 32, 9728, 5632, 1 + 2 + 3 + 4 + 5)
    assert tail - base == 15 * 8 * (128 * 2) * 2


def test_dequantize_validation():
    cfg = K.kvarn_config_parse()

    def dq(kp=FAKE, vp=FAKE, npages=4, pages=FAKE, n=1, h=8, ko=FAKE, vo=FAKE):
        return K.library().kvarn_dequantize_blocks(ctypes.byref(cfg), kp, vp, npages, pages, n, h, ko, vo, None, None)

    assert dq(n=-1) == K.KVARN_ERR_SHAPE
    assert dq(h=0) == K.KVARN_ERR_SHAPE
    assert dq(n=0) == K.KVARN_OK
    assert dq(ko=None, vo=None) == K.KVARN_OK  # nothing requested
    assert dq(pages=None) == K.KVARN_ERR_NULL
    assert dq(kp=None) == K.KVARN_ERR_NULL
    assert dq(npages=0) == K.KVARN_ERR_SHAPE
    # 2 * n_blocks * Hkv tiles must fit the 32-bit grid and tile index
    assert dq(n=1 << 20, h=1 << 10) == K.KVARN_ERR_SHAPE
    assert "too many tiles" in K.library().kvarn_last_error().decode()


def test_binding_rejects_what_the_abi_would_misread():
    """The Python binding checks dtype, shape, layout and device before any C call (host tensors
    here: every rule but the device one fires first, and the device rule fires last)."""
    import torch
    cfg = K.kvarn_config_parse()
    kb, vb = K.kvarn_page_bytes(cfg, False), K.kvarn_page_bytes(cfg, True)
    k = torch.zeros(256, 2, 128, dtype=torch.float16)
    pages = torch.zeros(2, dtype=torch.int32)
    kp = torch.zeros(4, 2, kb, dtype=torch.uint8)
    vp = torch.zeros(4, 2, vb, dtype=torch.uint8)

    def bad(fn, *a, match):
        with pytest.raises(ValueError, match=match):
            fn(*a)

    bad(K.kvarn_quantize_blocks, cfg, k[:200], k[:200], pages, kp, vp, match="whole number of 128-token blocks")
    bad(K.kvarn_quantize_blocks, cfg, k.float(), k, pages, kp, vp, match="k must be torch.float16")
    bad(K.kvarn_quantize_blocks, cfg, k, k[:128], pages, kp, vp, match="v must have shape")
    bad(K.kvarn_quantize_blocks, cfg, k, k, pages[:1], kp, vp, match="dst_pages must have shape")
    bad(K.kvarn_quantize_blocks, cfg, k, k, pages.long(), kp, vp, match="dst_pages must be torch.int32")
    bad(K.kvarn_quantize_blocks, cfg, k, k, pages, kp[:, :1], vp, match="k_pool must have shape")
    bad(K.kvarn_quantize_blocks, cfg, k, k, pages, kp, vp[:3], match="v_pool must have shape")
    bad(K.kvarn_quantize_blocks, cfg, k, k.transpose(0, 1).contiguous().transpose(0, 1), pages, kp, vp,
        match="v must be contiguous")
    bad(K.kvarn_quantize_blocks, cfg, k, k, pages, kp, vp, match="k must be in GPU memory")

    q = torch.zeros(3, 8, 128, dtype=torch.float16)
    bt = torch.zeros(3, 5, dtype=torch.int32)
    sl = torch.zeros(3, dtype=torch.int32)
    out = torch.zeros(3, 8, 128, dtype=torch.float32)
    ws = torch.zeros(1024, dtype=torch.uint8)
    bad(K.kvarn_decode_attention, cfg, q, kp, vp, bt, sl, 3, out, ws, match="not a multiple")
    bad(K.kvarn_decode_attention, cfg, q, kp, vp, bt[:2], sl, 2, out, ws, match="block_table must have shape")
    bad(K.kvarn_decode_attention, cfg, q, kp, vp, bt, sl, 2, out.half(), ws, match="out must be torch.float32")
    bad(K.kvarn_decode_attention, cfg, q, kp, vp, bt, sl, 4, out, ws, match="k_pool must have shape")
    bad(K.kvarn_decode_attention, cfg, q, kp, vp, bt, sl, 2, out, ws, match="q must be in GPU memory")
    tail = torch.zeros(3, 128, 2, 128, dtype=torch.float16)
    bad(K.kvarn_decode_attention_tail, cfg, q, kp, vp, bt, sl, tail[:, :64], tail, 2, out, ws,
        match="k_tail must have shape")
    kc = torch.zeros(4, 2, 128, 128, dtype=torch.float16)
    bad(K.kvarn_fp16_decode_attention, cfg, q, kc, kc[:, :1], bt, sl, 2, out, ws, match="v_cache must have shape")
    ko = torch.zeros(256, 2, 128, dtype=torch.float32)
    bad(K.kvarn_dequantize_blocks, cfg, kp, vp, pages, ko[:128], None, match="k_out must have shape")
    bad(K.kvarn_dequantize_blocks, cfg, kp, vp, pages, None, None, match="at least one")
    qp = torch.zeros(3, 16, 8, 128, dtype=torch.float16)
    kn = torch.zeros(3, 32, 2, 128, dtype=torch.float16)
    outp = torch.zeros(3, 16, 8, 128, dtype=torch.float32)
    bad(K.kvarn_prefill_attention, cfg, qp, kp, vp, bt, sl, kn, kn[:, :16], sl, sl, 2, outp,
        match="v_new must have shape")
    bad(K.kvarn_prefill_attention, cfg, qp, kp, vp, bt, sl, kn, kn, sl, sl, 2, outp[:, :8],
        match="out must have shape")
