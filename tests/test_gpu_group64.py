"""GPU parity of group size 64 (kvarn_k{4,8}v{2,4}_g64) against the oracle.

Reading: each group of the group-128 format splits into two halves of 64 consecutive elements (keys: one
channel over tokens 64h .. 64h+63; values: one token over channels 64h .. 64h+63) with their own fp16
scale and zero, stored half-major.  Bars as for group 128: codes within one level (mismatch fraction
<= 1e-4), scale / zero within one fp16 ulp, normalisers 1e-5, dequantised values max-abs 2e-3.
"""
import numpy as np
import pytest
import torch

from kv_cache_quantization_kvarn_amd import synth
from oracle import kvarn_oracle as o
import kvarn_check as chk

pytestmark = pytest.mark.gpu

FORMATS = ["kvarn_k4v2_g64", "kvarn_k4v4_g64", "kvarn_k8v2_g64", "kvarn_k8v4_g64"]


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def K():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from kv_cache_quantization_kvarn_amd import kvarn
    return kvarn


def quantize(K, cfg, k, v, pages, num_pages, poison):
    kp, vp = K.alloc_pools(cfg, num_pages, k.shape[1])
    kp.fill_(poison)
    vp.fill_(poison)
    fl = torch.zeros(1, dtype=torch.int32, device="cuda")
    K.kvarn_quantize_blocks(cfg, k, v, pages.to("cuda", torch.int32), kp, vp, fl)
    torch.cuda.synchronize()
    assert K.kvarn_read_flags(fl) == 0
    return kp, vp


@pytest.mark.parametrize("name", FORMATS)
def test_quantize_dequantize_every_tile_g64(K, name):
    cfg = K.kvarn_config_parse(name)
    w = synth.WORKLOADS["tiny_1x1024"]
    say("case: %s quantise + dequantise, %s, every tile, every page byte" % (name, w.name))
    pm = synth.make_page_map(w)
    k, v = synth.layer_kv(w, 0, 1024, "cuda")
    kp, vp = quantize(K, cfg, k, v, pm.prefix_pages, pm.num_pages, 0xA5)
    kp2, vp2 = quantize(K, cfg, k, v, pm.prefix_pages, pm.num_pages, 0x5A)
    assert torch.equal(kp, kp2) and torch.equal(vp, vp2)  # every byte written, deterministically
    assert kp.shape[2] == o.page_bytes(cfg.k_bits, 64) and vp.shape[2] == o.page_bytes(cfg.v_bits, 64)
    stats = chk.TileStats()
    kh, vh, kph, vph = k.cpu().numpy(), v.cpu().numpy(), kp.cpu().numpy(), vp.cpu().numpy()
    for blk in range(8):
        p = int(pm.prefix_pages[blk])
        for h in range(w.hkv):
            sl = slice(128 * blk, 128 * blk + 128)
            chk.compare_tile(stats, kh[sl, h], kph[p, h].tobytes(), False)
            chk.compare_tile(stats, vh[sl, h], vph[p, h].tobytes(), True)
    say("  " + stats.summary())
    stats.check()
    assert stats.groups == 8 * w.hkv * 2 * 256  # two halves of 128 groups per page, K and V
    ko = torch.empty(1024, w.hkv, 128, dtype=torch.float32, device="cuda")
    vo = torch.empty_like(ko)
    K.kvarn_dequantize_blocks(cfg, kp, vp, pm.prefix_pages.cuda(), ko, vo)
    torch.cuda.synchronize()
    koh, voh = ko.cpu().numpy(), vo.cpu().numpy()
    worst = 0.0
    for blk in range(8):
        p = int(pm.prefix_pages[blk])
        for h in range(w.hkv):
            for pool, outh, is_v in ((kph, koh, False), (vph, voh, True)):
                ref = o.dequantize_tile(o.decode_page(pool[p, h].tobytes(), is_v), is_v)
                worst = max(worst, float(np.abs(outh[128 * blk:128 * blk + 128, h] - ref).max()))
    say("  dequantised max-abs diff %.3e" % worst)
    assert worst <= chk.DEQUANT_TOL


def test_llama3_layer_g64_sampled_tiles(K):
    cfg = K.kvarn_config_parse("kvarn_k4v2_g64")
    w = synth.WORKLOADS["llama3_8b_layer_16x8192"]
    say("case: kvarn_k4v2_g64, %s full size, sampled tiles" % w.name)
    pm = synth.make_page_map(w)
    n = synth.total_prefix_blocks(w)
    k, v = synth.layer_kv(w, 0, n * 128, "cuda")
    kp, vp = quantize(K, cfg, k, v, pm.prefix_pages, pm.num_pages, 0)
    kh, vh = k.cpu().numpy(), v.cpu().numpy()
    stats = chk.TileStats()
    kph, vph = kp.cpu().numpy(), vp.cpu().numpy()
    for blk, h in ((0, 0), (511, 3), (1023, 7)):
        p = int(pm.prefix_pages[blk])
        sl = slice(128 * blk, 128 * blk + 128)
        chk.compare_tile(stats, kh[sl, h], kph[p, h].tobytes(), False)
        chk.compare_tile(stats, vh[sl, h], vph[p, h].tobytes(), True)
    say("  " + stats.summary())
    stats.check()


def randn_kv(g, n, hkv):
    k = torch.randn(n, hkv, 128, generator=g).mul_(torch.where(torch.rand(128, generator=g) < 0.04, 20.0, 1.0))
    v = torch.randn(n, hkv, 128, generator=g) * torch.exp(0.5 * torch.randn(n, hkv, 1, generator=g))
    return k.half(), v.half()


@pytest.mark.parametrize("name", FORMATS)
@pytest.mark.parametrize("G", [1, 4, 8])
def test_decode_g64(K, name, G):
    """Decode over packed pages, then with an fp16 tail, ragged and paged; a bad page id flagged."""
    cfg = K.kvarn_config_parse(name)
    hkv = 2
    hq = G * hkv
    say("case: %s decode and decode with a tail, G = %d, ragged, paged" % (name, G))
    g = torch.Generator().manual_seed(900 + 10 * G + len(name) + cfg.k_bits + cfg.v_bits)
    nblk = [3, 0, 6, 1]
    total = sum(nblk)
    k, v = randn_kv(g, total * 128, hkv)
    perm = torch.randperm(total, generator=g).to(torch.int32)
    kp, vp = quantize(K, cfg, k.cuda(), v.cuda(), perm, total, 0)
    bt = torch.full((4, 7), -1, dtype=torch.int32)
    off = 0
    for b, nb in enumerate(nblk):
        bt[b, :nb] = perm[off:off + nb]
        off += nb
    q = torch.randn(4, hq, 128, generator=g).half().cuda()
    kph, vph = kp.cpu().numpy(), vp.cpu().numpy()
    ws = K.alloc_workspace(cfg, 4, hq, hkv, bt.shape[1])
    fl = torch.zeros(1, dtype=torch.int32, device="cuda")
    sl = torch.tensor([128 * nb for nb in nblk], dtype=torch.int32)
    out = torch.full((4, hq, 128), float("nan"), device="cuda")
    K.kvarn_decode_attention(cfg, q, kp, vp, bt.cuda(), sl.cuda(), hkv, out, ws, dev_flags=fl)
    torch.cuda.synchronize()
    assert K.kvarn_read_flags(fl) == 0
    ref = o.decode(q.cpu().numpy(), kph, vph, bt.numpy(), sl.numpy(), hkv)
    got = out.cpu().numpy()
    assert np.all(got[1] == 0)
    d = float(np.abs(got - ref).max())
    say("  decode max-abs diff %.3e" % d)
    assert d <= chk.ATTN_TOL
    kt, vt = randn_kv(g, 4 * 128, hkv)
    kt, vt = kt.view(4, 128, hkv, 128).cuda(), vt.view(4, 128, hkv, 128).cuda()
    slt = torch.tensor([128 * 3 + 50, 127, 128 * 6, 128 + 1], dtype=torch.int32)
    K.kvarn_decode_attention_tail(cfg, q, kp, vp, bt.cuda(), slt.cuda(), kt, vt, hkv, out, ws, dev_flags=fl)
    torch.cuda.synchronize()
    assert K.kvarn_read_flags(fl) == 0
    ref = o.decode_tail(q.cpu().numpy(), kph, vph, bt.numpy(), slt.numpy(), kt.cpu().numpy(), vt.cpu().numpy(), hkv)
    d = float(np.abs(out.cpu().numpy() - ref).max())
    say("  decode with tail max-abs diff %.3e" % d)
    assert d <= chk.ATTN_TOL
    bad = bt.clone()
    bad[2, 4] = total + 3
    K.kvarn_decode_attention(cfg, q, kp, vp, bad.cuda(), sl.cuda(), hkv, out, ws, dev_flags=fl)
    torch.cuda.synchronize()
    assert K.kvarn_read_flags(fl) & 1


def test_llama3_layer_g64_decode_sampled(K):
    cfg = K.kvarn_config_parse("kvarn_k4v2_g64")
    w = synth.WORKLOADS["llama3_8b_layer_16x8192"]
    say("case: kvarn_k4v2_g64, %s full size decode, sampled heads" % w.name)
    pm = synth.make_page_map(w)
    n = synth.total_prefix_blocks(w)
    k, v = synth.layer_kv(w, 0, n * 128, "cuda")
    kp, vp = quantize(K, cfg, k, v, pm.prefix_pages, pm.num_pages, 0)
    del k, v
    q = synth.make_q(w, 0, "cuda")
    ws = K.alloc_workspace(cfg, w.batch, w.hq, w.hkv, pm.block_table.shape[1])
    out = torch.empty(w.batch, w.hq, 128, device="cuda")
    fl = torch.zeros(1, dtype=torch.int32, device="cuda")
    K.kvarn_decode_attention(cfg, q, kp, vp, pm.block_table.cuda(), pm.seq_lens.cuda(), w.hkv, out, ws, dev_flags=fl)
    torch.cuda.synchronize()
    assert K.kvarn_read_flags(fl) == 0
    got = out.cpu().numpy()
    kph, vph = kp.cpu().numpy(), vp.cpu().numpy()
    worst = 0.0
    for b, h in ((0, 0), (9, 17), (15, 31)):
        ref = o.decode(q.cpu().numpy(), kph, vph, pm.block_table.numpy(), pm.seq_lens.numpy(), w.hkv,
                       seqs=[b], heads=[h])
        worst = max(worst, float(np.abs(got[b, h] - ref[b, h]).max()))
    say("  decode max-abs diff %.3e over sampled heads" % worst)
    assert worst <= chk.ATTN_TOL


@pytest.mark.parametrize("name,G", [("kvarn_k4v2_g64", 4), ("kvarn_k4v4_g64", 8), ("kvarn_k8v2_g64", 1),
                                    ("kvarn_k8v4_g64", 3)])
def test_prefill_g64(K, name, G):
    """Chunked prefill over group-64 packed pages plus fp16 rows, ragged, against the oracle."""
    cfg = K.kvarn_config_parse(name)
    hkv = 2
    hq = G * hkv
    say("case: %s chunked prefill, G = %d, ragged, paged" % (name, G))
    g = torch.Generator().manual_seed(1200 + 10 * G + cfg.k_bits + cfg.v_bits)
    nblk = [2, 0, 4, 1]
    total = sum(nblk)
    k, v = randn_kv(g, total * 128, hkv)
    perm = torch.randperm(total, generator=g).to(torch.int32)
    kp, vp = quantize(K, cfg, k.cuda(), v.cuda(), perm, total, 0)
    bt = torch.full((4, 5), -1, dtype=torch.int32)
    off = 0
    for b, nb in enumerate(nblk):
        bt[b, :nb] = perm[off:off + nb]
        off += nb
    sl = torch.tensor([128 * nb for nb in nblk], dtype=torch.int32)
    new_lens = torch.tensor([100, 40, 130, 7], dtype=torch.int32)
    q_lens = torch.tensor([60, 40, 130, 0], dtype=torch.int32)
    kn, vn = randn_kv(g, 4 * 136, hkv)
    kn, vn = kn.view(4, 136, hkv, 128).cuda(), vn.view(4, 136, hkv, 128).cuda()
    qp = torch.randn(4, 130, hq, 128, generator=g).half().cuda()
    outp = torch.full((4, 130, hq, 128), float("nan"), device="cuda")
    fl = torch.zeros(1, dtype=torch.int32, device="cuda")
    K.kvarn_prefill_attention(cfg, qp, kp, vp, bt.cuda(), sl.cuda(), kn, vn, new_lens.cuda(), q_lens.cuda(), hkv, outp,
                              dev_flags=fl)
    torch.cuda.synchronize()
    assert K.kvarn_read_flags(fl) == 0
    ref = o.prefill(qp.cpu().numpy(), kp.cpu().numpy(), vp.cpu().numpy(), bt.numpy(), sl.numpy(), kn.cpu().numpy(),
                    vn.cpu().numpy(), new_lens.numpy(), q_lens.numpy(), hkv)
    got = outp.cpu().numpy()
    d = float(np.abs(got - ref).max())  # rows past q_len are zero on both sides; a NaN fails
    say("  prefill max-abs diff %.3e" % d)
    assert d <= chk.ATTN_TOL


def test_g64_half_constant_keys(K):
    """Tokens 0..63 of every key block identical: each key group of token half 0 is constant, so its fp16
    scale is 0 (all codes 0, the zero carries the value) while half 1's groups are not.  Quantise and
    decode (with one zero-scale half per page) against the oracle."""
    cfg = K.kvarn_config_parse("kvarn_k4v2_g64")
    hkv, hq = 2, 8
    say("case: kvarn_k4v2_g64 with constant-in-time key halves, decode G = 4")
    g = torch.Generator().manual_seed(777)
    nb = 3
    k = torch.randn(nb * 128, hkv, 128, generator=g)
    for b in range(nb):
        k[128 * b:128 * b + 64] = k[128 * b:128 * b + 1]
    v = torch.randn(nb * 128, hkv, 128, generator=g)
    k, v = k.half().cuda(), v.half().cuda()
    pages = torch.tensor([2, 0, 1], dtype=torch.int32)
    kp, vp = quantize(K, cfg, k, v, pages, nb, 0)
    kph, vph = kp.cpu().numpy(), vp.cpu().numpy()
    stats = chk.TileStats()
    kh, vh = k.cpu().numpy(), v.cpu().numpy()
    for b in range(nb):
        for h in range(hkv):
            sl = slice(128 * b, 128 * b + 128)
            chk.compare_tile(stats, kh[sl, h], kph[int(pages[b]), h].tobytes(), False)
            chk.compare_tile(stats, vh[sl, h], vph[int(pages[b]), h].tobytes(), True)
            f = o.decode_page(kph[int(pages[b]), h].tobytes(), False)
            assert np.all(f["scale"][0] == 0) and np.all(f["scale"][1] > 0)
    say("  " + stats.summary())
    stats.check()
    q = torch.randn(1, hq, 128, generator=g).half().cuda()
    bt = pages.view(1, nb)
    sl = torch.tensor([nb * 128], dtype=torch.int32)
    ws = K.alloc_workspace(cfg, 1, hq, hkv, nb)
    out = torch.full((1, hq, 128), float("nan"), device="cuda")
    fl = torch.zeros(1, dtype=torch.int32, device="cuda")
    K.kvarn_decode_attention(cfg, q, kp, vp, bt.cuda(), sl.cuda(), hkv, out, ws, dev_flags=fl)
    torch.cuda.synchronize()
    assert K.kvarn_read_flags(fl) == 0
    ref = o.decode(q.cpu().numpy(), kph, vph, bt.numpy(), sl.numpy(), hkv)
    d = float(np.abs(out.cpu().numpy() - ref).max())
    say("  decode max-abs diff %.3e" % d)
    assert d <= chk.ATTN_TOL
