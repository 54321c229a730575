"""GPU parity of the wider code formats kvarn_k4v4_g128, kvarn_k8v2_g128 and kvarn_k8v4_g128.

Quantise, dequantise, decode (packed pages, and packed pages plus an fp16 tail) and chunked prefill
in each format against the oracle, which reads the format off the page sizes.  Bars as for the
format the post names: codes within one level (mismatch fraction <= 1e-4), scale / zero within one
fp16 ulp, normalisers 1e-5, dequantised values and attention outputs max-abs 2e-3.
"""
import numpy as np
import pytest
import torch

from kv_cache_quantization_kvarn_amd import synth
from oracle import kvarn_oracle as o
import kvarn_check as chk

pytestmark = pytest.mark.gpu

FORMATS = ["kvarn_k4v4_g128", "kvarn_k8v2_g128", "kvarn_k8v4_g128"]


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


def randn_kv(g, n, hkv):
    k = torch.randn(n, hkv, 128, generator=g).mul_(torch.where(torch.rand(128, generator=g) < 0.04, 20.0, 1.0))
    v = torch.randn(n, hkv, 128, generator=g) * torch.exp(0.5 * torch.randn(n, hkv, 1, generator=g))
    return k.half(), v.half()


@pytest.mark.parametrize("name", FORMATS)
def test_quantize_dequantize_every_tile(K, name):
    cfg = K.kvarn_config_parse(name)
    w = synth.WORKLOADS["tiny_1x1024"]
    say("case: %s quantise + dequantise, %s, every tile, every page byte" % (name, w.name))
    pm = synth.make_page_map(w)
    k, v = synth.layer_kv(w, 0, 1024, "cuda")
    kp, vp = quantize(K, cfg, k, v, pm.prefix_pages, pm.num_pages, 0xA5)
    kp2, vp2 = quantize(K, cfg, k, v, pm.prefix_pages, pm.num_pages, 0x5A)
    assert torch.equal(kp, kp2) and torch.equal(vp, vp2)  # every byte written, deterministically
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


@pytest.mark.parametrize("name", FORMATS)
def test_decode_tail_and_prefill(K, name):
    cfg = K.kvarn_config_parse(name)
    hq, hkv = 8, 2
    say("case: %s decode, decode with a tail, prefill (ragged, paged)" % name)
    g = torch.Generator().manual_seed(606 + len(name))
    nblk = [3, 0, 5, 1]
    total = sum(nblk)
    k, v = randn_kv(g, total * 128, hkv)
    perm = torch.randperm(total, generator=g).to(torch.int32)
    kp, vp = quantize(K, cfg, k.cuda(), v.cuda(), perm, total, 0)
    bt = torch.full((4, 6), -1, dtype=torch.int32)
    off = 0
    for b, nb in enumerate(nblk):
        bt[b, :nb] = perm[off:off + nb]
        off += nb
    q = torch.randn(4, hq, 128, generator=g).half().cuda()
    kph, vph = kp.cpu().numpy(), vp.cpu().numpy()
    ws = K.alloc_workspace(cfg, 4, hq, hkv, bt.shape[1])
    fl = torch.zeros(1, dtype=torch.int32, device="cuda")
    # packed pages only
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
    # packed pages plus an fp16 tail
    kt, vt = randn_kv(g, 4 * 128, hkv)
    kt, vt = kt.view(4, 128, hkv, 128).cuda(), vt.view(4, 128, hkv, 128).cuda()
    slt = torch.tensor([128 * 3 + 77, 5, 128 * 5, 128 + 127], dtype=torch.int32)
    K.kvarn_decode_attention_tail(cfg, q, kp, vp, bt.cuda(), slt.cuda(), kt, vt, hkv, out, ws, dev_flags=fl)
    torch.cuda.synchronize()
    assert K.kvarn_read_flags(fl) == 0
    ref = o.decode_tail(q.cpu().numpy(), kph, vph, bt.numpy(), slt.numpy(), kt.cpu().numpy(), vt.cpu().numpy(), hkv)
    d = float(np.abs(out.cpu().numpy() - ref).max())
    say("  decode with tail max-abs diff %.3e" % d)
    assert d <= chk.ATTN_TOL
    # chunked prefill
    new_lens = torch.tensor([100, 40, 130, 0], dtype=torch.int32)
    q_lens = torch.tensor([60, 40, 130, 0], dtype=torch.int32)
    kn, vn = randn_kv(g, 4 * 136, hkv)
    kn, vn = kn.view(4, 136, hkv, 128).cuda(), vn.view(4, 136, hkv, 128).cuda()
    qp = torch.randn(4, 130, hq, 128, generator=g).half().cuda()
    outp = torch.full((4, 130, hq, 128), float("nan"), device="cuda")
    K.kvarn_prefill_attention(cfg, qp, kp, vp, bt.cuda(), sl.cuda(), kn, vn, new_lens.cuda(), q_lens.cuda(), hkv, outp,
                              dev_flags=fl)
    torch.cuda.synchronize()
    assert K.kvarn_read_flags(fl) == 0
    ref = o.prefill(qp.cpu().numpy(), kph, vph, bt.numpy(), sl.numpy(), kn.cpu().numpy(), vn.cpu().numpy(),
                    new_lens.numpy(), q_lens.numpy(), hkv)
    d = float(np.abs(outp.cpu().numpy() - ref).max())
    say("  prefill max-abs diff %.3e" % d)
    assert d <= chk.ATTN_TOL
    # bad lengths are flagged in these formats too
    K.kvarn_decode_attention(cfg, q, kp, vp, bt.cuda(), torch.tensor([128, 0, 200, 0], dtype=torch.int32).cuda(), hkv,
                             out, ws, dev_flags=fl)
    torch.cuda.synchronize()
    assert K.kvarn_read_flags(fl) & 2
    assert torch.all(out[2] == 0)


@pytest.mark.parametrize("name", FORMATS)
@pytest.mark.parametrize("G", [1, 3, 8])
def test_decode_group_sizes(K, name, G):
    """Decode with a tail at 1, 3 and 8 query heads per KV head: every column count of the
    coefficient operands, ragged lengths, a bad page id flagged and skipped."""
    cfg = K.kvarn_config_parse(name)
    hkv = 2
    hq = G * hkv
    say("case: %s decode with a tail, G = %d, ragged, paged" % (name, G))
    g = torch.Generator().manual_seed(700 + 10 * G + len(name))
    nblk = [2, 7, 0, 4]
    total = sum(nblk)
    k, v = randn_kv(g, total * 128, hkv)
    perm = torch.randperm(total, generator=g).to(torch.int32)
    kp, vp = quantize(K, cfg, k.cuda(), v.cuda(), perm, total, 0)
    bt = torch.full((4, 8), -1, dtype=torch.int32)
    off = 0
    for b, nb in enumerate(nblk):
        bt[b, :nb] = perm[off:off + nb]
        off += nb
    q = torch.randn(4, hq, 128, generator=g).half().cuda()
    kt, vt = randn_kv(g, 4 * 128, hkv)
    kt, vt = kt.view(4, 128, hkv, 128).cuda(), vt.view(4, 128, hkv, 128).cuda()
    slt = torch.tensor([128 * 2 + 1, 128 * 7 + 126, 64, 128 * 4], dtype=torch.int32)
    ws = K.alloc_workspace(cfg, 4, hq, hkv, bt.shape[1])
    fl = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = torch.full((4, hq, 128), float("nan"), device="cuda")
    K.kvarn_decode_attention_tail(cfg, q, kp, vp, bt.cuda(), slt.cuda(), kt, vt, hkv, out, ws, dev_flags=fl)
    torch.cuda.synchronize()
    assert K.kvarn_read_flags(fl) == 0
    kph, vph = kp.cpu().numpy(), vp.cpu().numpy()
    ref = o.decode_tail(q.cpu().numpy(), kph, vph, bt.numpy(), slt.numpy(), kt.cpu().numpy(), vt.cpu().numpy(), hkv)
    d = float(np.abs(out.cpu().numpy() - ref).max())
    say("  decode with tail max-abs diff %.3e" % d)
    assert d <= chk.ATTN_TOL
    # a page id past the pool: flagged, that page skipped, the other sequences untouched
    bad = bt.clone()
    bad[1, 3] = total + 5
    sl = torch.tensor([128 * nb for nb in nblk], dtype=torch.int32)
    K.kvarn_decode_attention(cfg, q, kp, vp, bad.cuda(), sl.cuda(), hkv, out, ws, dev_flags=fl)
    torch.cuda.synchronize()
    assert K.kvarn_read_flags(fl) & 1
    ref = o.decode(q.cpu().numpy(), kph, vph, bt.numpy(), sl.numpy(), hkv, seqs=[0, 3])
    got = out.cpu().numpy()
    d = max(float(np.abs(got[b] - ref[b]).max()) for b in (0, 3))
    assert d <= chk.ATTN_TOL
    assert np.all(got[2] == 0)


def test_k8v4_llama3_layer_decode_sampled(K):
    cfg = K.kvarn_config_parse("kvarn_k8v4_g128")
    w = synth.WORKLOADS["llama3_8b_layer_16x8192"]
    say("case: kvarn_k8v4_g128, %s full size: quantise + decode, sampled tiles and heads" % w.name)
    pm = synth.make_page_map(w)
    n = synth.total_prefix_blocks(w)
    k, v = synth.layer_kv(w, 0, n * 128, "cuda")
    kp, vp = quantize(K, cfg, k, v, pm.prefix_pages, pm.num_pages, 0)
    kh, vh = k.cpu().numpy(), v.cpu().numpy()
    stats = chk.TileStats()
    kph_all, vph_all = kp.cpu().numpy(), vp.cpu().numpy()
    for blk, h in ((0, 0), (333, 5), (1023, 7)):
        p = int(pm.prefix_pages[blk])
        sl = slice(128 * blk, 128 * blk + 128)
        chk.compare_tile(stats, kh[sl, h], kph_all[p, h].tobytes(), False)
        chk.compare_tile(stats, vh[sl, h], vph_all[p, h].tobytes(), True)
    say("  " + stats.summary())
    stats.check()
    del k, v, kh, vh
    q = synth.make_q(w, 0, "cuda")
    ws = K.alloc_workspace(cfg, w.batch, w.hq, w.hkv, pm.block_table.shape[1])
    out = torch.empty(w.batch, w.hq, 128, device="cuda")
    fl = torch.zeros(1, dtype=torch.int32, device="cuda")
    K.kvarn_decode_attention(cfg, q, kp, vp, pm.block_table.cuda(), pm.seq_lens.cuda(), w.hkv, out, ws, dev_flags=fl)
    torch.cuda.synchronize()
    assert K.kvarn_read_flags(fl) == 0
    got = out.cpu().numpy()
    worst = 0.0
    for b, h in ((0, 0), (7, 21), (15, 31)):
        ref = o.decode(q.cpu().numpy(), kph_all, vph_all, pm.block_table.numpy(), pm.seq_lens.numpy(), w.hkv,
                       seqs=[b], heads=[h])
        worst = max(worst, float(np.abs(got[b, h] - ref[b, h]).max()))
    say("  decode max-abs diff %.3e over sampled heads" % worst)
    assert worst <= chk.ATTN_TOL


def test_wide_decode_most_splits(K):
    """1,024 blocks of one KV head plus a 90-token tail: 63 page splits and the tail split in one merge."""
    cfg = K.kvarn_config_parse("kvarn_k4v4_g128")
    say("case: kvarn_k4v4_g128 decode with a tail over 1,024 blocks (64 splits)")
    g = torch.Generator().manual_seed(4096)
    k, v = randn_kv(g, 1024 * 128, 1)
    perm = torch.randperm(1024, generator=g).to(torch.int32)
    kp, vp = quantize(K, cfg, k.cuda(), v.cuda(), perm, 1024, 0)
    bt = perm.view(1, 1024).clone()
    kt, vt = randn_kv(g, 128, 1)
    kt, vt = kt.view(1, 128, 1, 128).cuda(), vt.view(1, 128, 1, 128).cuda()
    q = torch.randn(1, 4, 128, generator=g).half().cuda()
    sl = torch.tensor([1024 * 128 + 90], dtype=torch.int32)
    ws = K.alloc_workspace(cfg, 1, 4, 1, 1024)
    out = torch.full((1, 4, 128), float("nan"), device="cuda")
    fl = torch.zeros(1, dtype=torch.int32, device="cuda")
    for rep in range(2):  # the counters are back at zero after every call
        K.kvarn_decode_attention_tail(cfg, q, kp, vp, bt.cuda(), sl.cuda(), kt, vt, 1, out, ws, dev_flags=fl)
        torch.cuda.synchronize()
        assert K.kvarn_read_flags(fl) == 0
        ref = o.decode_tail(q.cpu().numpy(), kp.cpu().numpy(), vp.cpu().numpy(), bt.numpy(), sl.numpy(),
                            kt.cpu().numpy(), vt.cpu().numpy(), 1)
        d = float(np.abs(out.cpu().numpy() - ref).max())
        say("  call %d: max-abs diff %.3e" % (rep, d))
        assert d <= chk.ATTN_TOL
