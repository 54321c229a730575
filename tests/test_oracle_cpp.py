"""Pins of the C++ oracle (oracle/kvarn_oracle.cpp), on the CPU.

The C++ oracle is pinned two ways:
  * on its own, against what the mathematics fixes: the binary16 definition (every bit pattern, every
    tie), the Hadamard matrix (Sylvester definition, scipy, orthonormality, FWHT = dense), the
    normalisation (brute force on small shapes, closed forms), attention special cases;
  * against the Python oracle, which carries the full set of pins in test_oracle_pins.py: page bytes
    identical tile by tile (codes, scale, zero, rho, gamma) in every format, dequantised blocks and
    decode outputs equal to rounding.
"""
import math

import numpy as np
import pytest
import scipy.linalg

from kv_cache_quantization_kvarn_amd import synth
from oracle import kvarn_oracle as o
from oracle import kvarn_oracle_cpp as C


@pytest.fixture(scope="module", autouse=True)
def built():
    C.build()


def rng(seed=0):
    return np.random.default_rng(seed)


# ----------------------------------------------------------------------------- binary16
def test_half_decode_every_bit_pattern():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = C.half_to_double(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_half_encode_exact_values_ties_and_neighbours():
    finite = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = finite.view(np.float16)
    vals = vals[np.isfinite(vals)]
    assert np.array_equal(C.double_to_half(vals.astype(np.float64)), vals.view(np.uint16))
    # every tie between neighbouring positive halves, and the fp32 numbers just either side of it
    pos = np.sort(np.unique(vals[vals >= 0].astype(np.float64)))
    mid = (pos[:-1] + pos[1:]) / 2  # exact in double, and in fp32 for every binary16 neighbour pair
    mid32 = mid.astype(np.float32)
    assert np.array_equal(mid32.astype(np.float64), mid)
    below = np.nextafter(mid32, np.float32(0))
    above = np.nextafter(mid32, np.float32(np.inf))
    for x in (mid32, below, above, -mid32):
        assert np.array_equal(C.double_to_half(x.astype(np.float64)), x.astype(np.float16).view(np.uint16))
    # overflow boundary: 65504 is the largest half; the tie at 65520 rounds to infinity
    edge = np.array([65504.0, 65519.996, 65520.0, 1e9, -65520.0, 2.0 ** -25, 2.0 ** -24 * 1.5], dtype=np.float32)
    r = rng(1).standard_normal(20000).astype(np.float32) * np.float32(2.0) ** rng(2).integers(-30, 18, 20000)
    with np.errstate(over="ignore"):  # numpy warns on the values that overflow to infinity
        for x in (edge, r.astype(np.float32)):
            assert np.array_equal(C.double_to_half(x.astype(np.float64)), x.astype(np.float16).view(np.uint16))


# ----------------------------------------------------------------------------- rotation
@pytest.mark.parametrize("d", [64, 128, 256])
def test_dense_rotation_is_the_sylvester_matrix(d):
    h = C.rotate(np.eye(d), fwht=False)  # row k of the output is H e_k = column k of H
    assert np.array_equal(h, scipy.linalg.hadamard(d).T / np.sqrt(d))
    assert np.abs(h @ h.T - np.eye(d)).max() < 1e-15
    j, k = np.meshgrid(np.arange(d), np.arange(d), indexing="ij")
    sign = np.vectorize(lambda a: -1.0 if bin(a).count("1") % 2 else 1.0)(j & k)
    assert np.array_equal(h, sign / math.sqrt(d))


@pytest.mark.parametrize("d", [64, 128, 256])
def test_fwht_equals_dense_to_1e_12(d):
    x = rng(d).standard_normal((64, d)) * np.exp(rng(d + 1).standard_normal((64, 1)) * 3)
    a = C.rotate(x, fwht=True)
    b = C.rotate(x, fwht=False)
    assert np.abs(a - b).max() <= 1e-12 * np.abs(x).max()
    # e_0 spreads evenly; a constant row concentrates on channel 0; norms are kept
    e0 = np.zeros((1, d))
    e0[0, 0] = 1.0
    assert np.allclose(C.rotate(e0, fwht=True), 1 / np.sqrt(d), rtol=0, atol=1e-16)
    c = C.rotate(np.full((1, d), 2.5), fwht=True)
    assert abs(c[0, 0] - 2.5 * np.sqrt(d)) < 1e-12 and np.abs(c[0, 1:]).max() < 1e-12
    assert np.allclose(np.linalg.norm(a, axis=1), np.linalg.norm(x, axis=1), rtol=1e-14)


def test_fwht_of_fp16_rows_is_the_correctly_rounded_sum():
    """fp16 inputs add exactly in double, so each FWHT output is one rounding of the exact value."""
    from fractions import Fraction
    x16 = (rng(3).standard_normal((2, 128)) * 30).astype(np.float16)
    got = C.rotate(x16.astype(np.float64), fwht=True)
    hs = scipy.linalg.hadamard(128)
    for t in range(2):
        for j in (0, 1, 77, 127):
            exact = sum(Fraction(float(x16[t, k])) * int(hs[j, k]) for k in range(128))
            assert got[t, j] == float(exact) * (1 / np.sqrt(128)) or \
                abs(got[t, j] - float(exact) / np.sqrt(128)) <= 2e-16 * abs(float(exact))


# ----------------------------------------------------------------------------- normalisation
def brute_normalize(r, iters, eps):
    rows, cols = r.shape
    rho, gam = [0.0] * rows, [0.0] * cols
    for _ in range(iters):
        for t in range(rows):
            y = [r[t, j] * 2.0 ** -(rho[t] + gam[j]) for j in range(cols)]
            m = sum(y) / cols
            rho[t] += 0.5 * math.log2(sum((a - m) ** 2 for a in y) / cols + eps)
        for j in range(cols):
            y = [r[t, j] * 2.0 ** -(rho[t] + gam[j]) for t in range(rows)]
            m = sum(y) / rows
            gam[j] += 0.5 * math.log2(sum((a - m) ** 2 for a in y) / rows + eps)
    return np.array(rho), np.array(gam)


@pytest.mark.parametrize("shape,iters", [((6, 5), 1), ((8, 8), 4), ((3, 7), 3), ((128, 64), 4)])
def test_normalize_matches_brute_force(shape, iters):
    r = rng(shape[0]).standard_normal(shape) * np.exp(rng(shape[1]).standard_normal(shape[1]) * 2)
    a = C.normalize(r, iters, 1e-6)
    b = brute_normalize(r, iters, 1e-6)
    assert np.abs(a[0] - b[0]).max() < 1e-12 and np.abs(a[1] - b[1]).max() < 1e-12


def test_normalize_closed_forms():
    r = rng(4).standard_normal((128, 128)) * 3
    r[17] = 0.0
    rho, gam = C.normalize(r, 4, 1e-6)
    # an all-zero row: each row pass adds half of log2(eps)
    assert abs(rho[17] - 4 * 0.5 * math.log2(1e-6)) < 1e-12
    # after the final column pass every column of the normalised block has variance v / (v + eps)
    y = r * np.exp2(-(rho[:, None] + gam[None, :]))
    assert np.abs(y.var(axis=0) - 1.0).max() < 1e-5
    # a token scaled by 2^k moves its rho by k
    r2 = r.copy()
    r2[5] *= 2.0 ** 7
    rho2, gam2 = C.normalize(r2, 4, 1e-6)
    assert abs(rho2[5] - rho[5] - 7) < 1e-6


# ----------------------------------------------------------------------------- quantise: identity with the Python oracle
FORMATS = [(4, 2, 128), (4, 4, 128), (8, 2, 128), (8, 4, 128), (4, 2, 64), (4, 4, 64), (8, 2, 64), (8, 4, 64)]


def degenerate_tiles():
    g = rng(77)
    row = g.standard_normal((1, 128))
    const = np.repeat(row, 128, axis=0)
    zrows = g.standard_normal((128, 128))
    zrows[[0, 17, 127]] = 0
    wide = g.standard_normal((128, 128)) * np.logspace(-3, 3, 128)[:, None]
    return [x.astype(np.float16) for x in (const, zrows, np.zeros((128, 128)), wide)]


def test_pages_identical_to_python_oracle_tiny_all_tiles_both_modes():
    w = synth.WORKLOADS["tiny_1x1024"]
    k, v = synth.layer_kv(w, 0, 1024, "cpu")
    kh, vh = k.numpy(), v.numpy()
    for b in range(8):
        for h in range(8):
            for is_v, x in ((False, kh), (True, vh)):
                tile = x[128 * b:128 * b + 128, h]
                ref = o.encode_page(o.quantize_tile(tile, is_v), is_v)
                for fwht in (False, True):
                    assert C.quantize_tile_page(tile, is_v, 2 if is_v else 4, 128, fwht) == ref, (b, h, is_v, fwht)


@pytest.mark.parametrize("kb,vb,group", FORMATS)
def test_pages_identical_to_python_oracle_every_format(kb, vb, group):
    w = synth.WORKLOADS["long_context_1x131072"]  # 8 outlier channels x 50
    k, v = synth.layer_kv(w, 0, 256, "cpu")
    tiles = [(k.numpy()[:128, 3], False), (v.numpy()[128:, 5], True)]
    tiles += [(t, is_v) for t in degenerate_tiles() for is_v in (False, True)]
    for x, is_v in tiles:
        bits = vb if is_v else kb
        ref = o.encode_page(o.quantize_tile(x, is_v, bits=bits, group=group), is_v, bits)
        assert C.quantize_tile_page(x, is_v, bits, group, fwht=True) == ref


def test_quantize_blocks_pools_identical_and_thread_count_free():
    g = rng(9)
    hkv = 3
    k = (g.standard_normal((5 * 128, hkv, 128)) * np.where(g.random(128) < 0.05, 20, 1)).astype(np.float16)
    v = (g.standard_normal((5 * 128, hkv, 128)) * np.exp(0.5 * g.standard_normal((5 * 128, hkv, 1)))).astype(np.float16)
    pages = np.array([4, 0, 6, 2, 1], np.int32)
    pools = []
    for threads in (1, 7):
        kp = np.zeros((7, hkv, o.K_PAGE_BYTES), np.uint8)
        vp = np.zeros((7, hkv, o.V_PAGE_BYTES), np.uint8)
        assert C.quantize_blocks(k, v, pages, kp, vp, threads=threads) == 0
        pools.append((kp, vp))
    assert np.array_equal(pools[0][0], pools[1][0]) and np.array_equal(pools[0][1], pools[1][1])
    kpo = np.zeros_like(pools[0][0])
    vpo = np.zeros_like(pools[0][1])
    o.quantize_blocks(k, v, pages, kpo, vpo)
    assert np.array_equal(kpo, pools[0][0]) and np.array_equal(vpo, pools[0][1])
    # an out-of-range page id skips its block and is counted
    kp = np.zeros((7, hkv, o.K_PAGE_BYTES), np.uint8)
    vp = np.zeros((7, hkv, o.V_PAGE_BYTES), np.uint8)
    assert C.quantize_blocks(k, v, np.array([4, 0, 9, -1, 1], np.int32), kp, vp) == 2
    assert np.array_equal(kp[[4, 0, 1]], kpo[[4, 0, 1]]) and not kp[[2, 3, 5, 6]].any()


# ----------------------------------------------------------------------------- dequantise and decode
def small_cache(seed, nblocks, hkv, kb=4, vb=2, group=128):
    g = rng(seed)
    k = (g.standard_normal((nblocks * 128, hkv, 128)) * np.where(g.random(128) < 0.05, 20, 1)).astype(np.float16)
    v = (g.standard_normal((nblocks * 128, hkv, 128)) * np.exp(0.5 * g.standard_normal((nblocks * 128, hkv, 1)))
         ).astype(np.float16)
    kp = np.zeros((nblocks, hkv, o.page_bytes(kb, group)), np.uint8)
    vp = np.zeros((nblocks, hkv, o.page_bytes(vb, group)), np.uint8)
    C.quantize_blocks(k, v, np.arange(nblocks, dtype=np.int32), kp, vp)
    return k, v, kp, vp


@pytest.mark.parametrize("kb,vb,group", [(4, 2, 128), (8, 4, 64)])
def test_dequantize_equals_python_oracle(kb, vb, group):
    _, _, kp, vp = small_cache(11, 2, 2, kb, vb, group)
    for pool, is_v, bits in ((kp, False, kb), (vp, True, vb)):
        for p in range(2):
            ref = o.dequantize_tile(o.decode_page(pool[p, 1].tobytes(), is_v), is_v)
            for fwht in (False, True):
                got = C.dequantize_page(pool[p, 1].tobytes(), is_v, bits, group, fwht=fwht)
                assert np.abs(got - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())


@pytest.mark.parametrize("hq,hkv,lens", [(8, 2, [384, 0, 256, 128]), (6, 1, [640]), (4, 4, [128, 512])])
def test_decode_equals_python_oracle(hq, hkv, lens):
    nb = sum(l // 128 for l in lens)
    _, _, kp, vp = small_cache(hq + hkv, max(nb, 1), hkv)
    g = rng(5)
    perm = g.permutation(max(nb, 1)).astype(np.int32)
    bt = np.full((len(lens), max(max(lens) // 128, 1) + 2), -1, np.int32)
    off = 0
    for b, l in enumerate(lens):
        bt[b, :l // 128] = perm[off:off + l // 128]
        off += l // 128
    q = g.standard_normal((len(lens), hq, 128)).astype(np.float16)
    sl = np.array(lens, np.int32)
    for scale in (0.0, 0.05):
        ref = o.decode(q, kp, vp, bt, sl, hkv, scale)
        got = C.decode(q, kp, vp, bt, sl, hkv, scale)
        assert np.abs(got - ref).max() < 1e-10
    # a sample of pairs leaves the other rows untouched (NaN)
    part = C.decode(q, kp, vp, bt, sl, hkv, pairs=[(0, 1)])
    assert np.abs(part[0, 1] - ref[0, 1]).max() < 1
    assert np.isnan(part[0, 0]).all()


def test_decode_special_cases():
    _, _, kp, vp = small_cache(21, 3, 1)
    bt = np.array([[2, 0, 1]], np.int32)
    sl = np.array([384], np.int32)
    v_hat = np.concatenate([C.dequantize_page(vp[p, 0].tobytes(), True, 2) for p in (2, 0, 1)])
    # q = 0: uniform weights, the mean of the dequantised values
    out = C.decode(np.zeros((1, 1, 128), np.float16), kp, vp, bt, sl, 1)
    assert np.abs(out[0, 0] - v_hat.mean(axis=0)).max() < 1e-12
    # a bad page id is left out: the same as a table without it
    bad = C.decode(np.ones((1, 1, 128), np.float16), kp, vp, np.array([[2, 7, 1]], np.int32), sl, 1)
    good = C.decode(np.ones((1, 1, 128), np.float16), kp, vp, np.array([[2, 1, 0]], np.int32),
                    np.array([256], np.int32), 1)
    assert np.abs(bad - good).max() < 1e-12
    # an empty sequence gives zeros
    assert not C.decode(np.ones((1, 2, 128), np.float16), kp, vp, bt, np.array([0], np.int32), 1).any()


def test_decode_with_tail_equals_python_oracle():
    _, _, kp, vp = small_cache(31, 4, 2)
    g = rng(6)
    kt = g.standard_normal((3, 128, 2, 128)).astype(np.float16)
    vt = g.standard_normal((3, 128, 2, 128)).astype(np.float16)
    bt = np.array([[0, 1, -1], [2, -1, -1], [3, 0, 1]], np.int32)
    sl = np.array([256 + 37, 127, 384], np.int32)
    q = g.standard_normal((3, 8, 128)).astype(np.float16)
    ref = o.decode_tail(q, kp, vp, bt, sl, kt, vt, 2)
    got = C.decode(q, kp, vp, bt, sl, 2, k_tail=kt, v_tail=vt)
    assert np.abs(got - ref).max() < 1e-10


# ----------------------------------------------------------------------------- the whole-pool comparison
@pytest.mark.parametrize("kb,vb,group", [(4, 2, 128), (8, 4, 64), (4, 4, 128), (8, 2, 64)])
def test_pool_comparison_unpacks_like_the_python_oracle_and_catches_changes(kb, vb, group):
    import kvarn_check as chk
    _, _, kp, vp = small_cache(41, 3, 2, kb, vb, group)
    for pool, is_v, bits in ((kp, False, kb), (vp, True, vb)):
        codes = chk.unpack_codes(pool, is_v, bits)
        s, z, rho, gam = chk.meta_views(pool, is_v, bits, group)
        for p in range(3):
            for h in range(2):
                f = o.decode_page(pool[p, h].tobytes(), is_v)
                assert np.array_equal(codes[p, h], f["codes"])
                assert np.array_equal(s[p, h], np.asarray(f["scale"]).ravel())
                assert np.array_equal(z[p, h], np.asarray(f["zero"]).ravel())
                assert np.array_equal(rho[p, h], f["rho"]) and np.array_equal(gam[p, h], f["gamma"])
        st = chk.TileStats()
        chk.compare_pools(st, pool, pool.copy(), is_v, bits, group)
        assert (st.code_mismatch, st.sz_maxulp, st.norm_maxerr, st.tiles) == (0, 0, 0.0, 6)
        st.check()
        # one code off by one level, one scale one ulp off, one normaliser moved
        bad = pool.copy()
        bad[1, 1, 0] ^= 1
        code_bytes = 128 * 128 * bits // 8
        bad[2, 0, code_bytes] ^= 1
        bad[0, 1, -1] ^= 0x40
        st = chk.TileStats()
        chk.compare_pools(st, bad, pool, is_v, bits, group)
        assert st.code_mismatch == 1 and st.code_maxdiff == 1 and st.sz_maxulp == 1 and st.norm_maxerr > 1e-3
        with pytest.raises(AssertionError):
            st.check()
