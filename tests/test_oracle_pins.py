"""Pins of the CPU oracle against facts the pages and the mathematics fix.

Every test here checks the oracle against something other than itself: a
closed form, an independent construction, a library routine, brute force on a
tiny input, or a figure printed on the pages (tests/golden/page_figures.txt).
They run on the CPU only.
"""
import os

import numpy as np
import pytest
import scipy.linalg
import scipy.special
import torch

from oracle import kvarn_oracle as o

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_figures.txt")


def golden():
    vals = {}
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split(None, 1)
            vals[k] = v
    return vals


def rng(seed=0):
    return np.random.default_rng(seed)


def fp16_block(seed=0, outliers=4, mult=20.0):
    r = rng(seed)
    x = r.standard_normal((128, 128))
    if outliers:
        x[:, r.choice(128, outliers, replace=False)] *= mult
    return x.astype(np.float16)


# ----------------------------------------------------------------- rotation
def test_hadamard_equals_sylvester_recursion():
    h = np.array([[1.0]])
    while h.shape[0] < 128:
        h = np.block([[h, h], [h, -h]])
    assert np.array_equal(o.hadamard() * np.sqrt(128), h)


def test_hadamard_equals_scipy():
    assert np.allclose(o.hadamard(), scipy.linalg.hadamard(128) / np.sqrt(128), rtol=0, atol=1e-15)


def test_hadamard_orthonormal_symmetric_involution():
    h = o.hadamard()
    assert np.array_equal(h, h.T)
    assert np.abs(h @ h.T - np.eye(128)).max() < 1e-14
    assert np.all(np.abs(np.abs(h) - 2.0 ** -3.5) < 1e-16)


def test_rotate_acts_along_channels_of_each_token():
    x = np.zeros((128, 128))
    x[5, 3] = 1.0
    r = o.rotate(x)
    assert np.count_nonzero(np.abs(r).sum(axis=1)) == 1  # only token 5 is touched
    # a unit impulse at channel 3 maps to column 3 of H: sign (-1)^popcount(j & 3)
    expect = np.array([(-1.0) ** bin(j & 3).count("1") for j in range(128)]) / np.sqrt(128)
    assert np.allclose(r[5], expect, atol=1e-15)


def test_rotate_constant_row_and_parseval():
    x = np.full((1, 128), 0.75)
    r = o.rotate(x)
    e0 = np.zeros(128)
    e0[0] = np.sqrt(128) * 0.75
    assert np.allclose(r[0], e0, atol=1e-13)
    y = rng(1).standard_normal((128, 128))
    assert np.allclose(np.linalg.norm(o.rotate(y), axis=1), np.linalg.norm(y, axis=1), rtol=1e-13)


def test_joint_rotation_preserves_scores_fp32():
    # The rotation is orthonormal, so attention scores are unchanged (rotated-cache stage).
    r = rng(2)
    q = r.standard_normal((64, 128))
    k = r.standard_normal((64, 128)) * np.where(r.random(128) < 0.05, 30.0, 1.0)
    qr = o.rotate(q).astype(np.float32)
    kr = o.rotate(k).astype(np.float32)
    s_rot = np.einsum("ij,ij->i", qr, kr, dtype=np.float32)
    s_ref = np.einsum("ij,ij->i", q, k)
    assert np.all(np.abs(s_rot - s_ref) <= 1e-5 * np.linalg.norm(q, axis=1) * np.linalg.norm(k, axis=1))


# ------------------------------------------------------------ normalisation
def brute_normalize(r, iters, eps):
    """Loop-by-loop textbook version on a small matrix (independent of numpy.var)."""
    nr, nc = len(r), len(r[0])
    rho = [0.0] * nr
    gam = [0.0] * nc
    for _ in range(iters):
        for t in range(nr):
            ys = [r[t][j] * 2.0 ** (-(rho[t] + gam[j])) for j in range(nc)]
            m = sum(ys) / nc
            v = sum((y - m) ** 2 for y in ys) / nc
            rho[t] += 0.5 * np.log2(v + eps)
        for j in range(nc):
            ys = [r[t][j] * 2.0 ** (-(rho[t] + gam[j])) for t in range(nr)]
            m = sum(ys) / nr
            v = sum((y - m) ** 2 for y in ys) / nr
            gam[j] += 0.5 * np.log2(v + eps)
    return np.array(rho), np.array(gam)


@pytest.mark.parametrize("shape,iters", [((6, 5), 1), ((8, 8), 4), ((3, 7), 3)])
def test_normalize_matches_brute_force(shape, iters):
    r = rng(3).standard_normal(shape) * rng(4).lognormal(0, 1, shape)
    rho, gam = o.normalize(r, iters, 1e-6)
    rb, gb = brute_normalize(r.tolist(), iters, 1e-6)
    assert np.allclose(rho, rb, atol=1e-12) and np.allclose(gam, gb, atol=1e-12)


def test_final_column_pass_gives_unit_column_variance():
    r = o.rotate(fp16_block(5).astype(np.float64))
    rho, gam = o.normalize(r)
    n = r * np.exp2(-(rho[:, None] + gam[None, :]))
    v = n.var(axis=0)
    assert np.all(np.abs(v - 1.0) < 1e-5)
    # columns are equalised last, so rows are only approximately unit variance
    assert np.abs(np.log2(n.var(axis=1))).max() < 0.5


def test_rows_are_normalised_before_columns():
    # With one iteration the column pass runs last, so columns are exact and rows are not.
    r = rng(6).standard_normal((128, 128)) * rng(7).lognormal(0, 1.0, (128, 1)) * rng(8).lognormal(0, 1.0, (1, 128))
    rho, gam = o.normalize(r, 1)
    n = r * np.exp2(-(rho[:, None] + gam[None, :]))
    # closed form of the last (column) pass: variance v becomes v / (v + eps)
    v_before = (r * np.exp2(-rho[:, None])).var(axis=0)
    assert np.allclose(n.var(axis=0), v_before / (v_before + 1e-6), rtol=1e-12)
    # and the row pass ran first on the raw rows: rho = log2(row variance + eps) / 2
    assert np.allclose(rho, 0.5 * np.log2(r.var(axis=1) + 1e-6), rtol=0, atol=1e-12)
    assert np.abs(n.var(axis=1) - 1).max() > 1e-2


def test_sinkhorn_fixed_point_with_many_iterations():
    r = o.rotate(fp16_block(9).astype(np.float64)) * rng(10).lognormal(0, 1.0, (128, 1))
    rho, gam = o.normalize(r, 60)
    n = r * np.exp2(-(rho[:, None] + gam[None, :]))
    rho1, gam1 = o.normalize(r, 61)
    n1 = r * np.exp2(-(rho1[:, None] + gam1[None, :]))
    # the alternating passes reach a fixed point of the normalised block: columns at unit
    # variance, every row at one common variance (centred variances of rows and columns
    # need not both be 1, since removing row means and column means differ)
    assert np.abs(n1 - n).max() < 1e-9
    assert np.abs(n.var(axis=0) - 1).max() < 1e-5
    rv = np.log2(n.var(axis=1))
    assert rv.max() - rv.min() < 1e-6 and abs(rv.mean()) < 0.05


def test_row_log_variance_spread_shrinks_with_iterations():
    r = o.rotate(fp16_block(11).astype(np.float64)) * rng(12).lognormal(0, 1.5, (128, 1))
    spreads = []
    for t in (0, 1, 2, 4):
        rho, gam = o.normalize(r, t)
        n = r * np.exp2(-(rho[:, None] + gam[None, :]))
        spreads.append(np.log2(n.var(axis=1)).std())
    assert spreads[0] > spreads[1] > spreads[2] > spreads[3]


def test_zero_token_row_closed_form():
    x = fp16_block(13).astype(np.float64)
    x[17, :] = 0
    r = o.rotate(x)
    rho, _ = o.normalize(r)
    # the zero row's variance is 0 every iteration, so rho gains log2(eps)/2 four times (log base 2)
    assert abs(rho[17] - 2.0 * np.log2(1e-6)) < 1e-9
    fv = o.quantize_tile(x.astype(np.float16), True)
    assert np.all(fv["codes"][17] == 0) and fv["scale"][17] == 0
    assert np.all(o.dequantize_tile(fv, True)[17] == 0.0)
    fk = o.quantize_tile(x.astype(np.float16), False)
    assert np.abs(o.dequantize_tile(fk, False)[17]).max() < 1e-9


def test_power_of_two_token_scaling_shifts_rho():
    x = fp16_block(14).astype(np.float64)
    y = x.copy()
    y[3] *= 8.0  # exact in fp16 for these magnitudes
    assert np.array_equal(y.astype(np.float16).astype(np.float64), y)
    fx = o.quantize_tile(x.astype(np.float16), False)
    fy = o.quantize_tile(y.astype(np.float16), False)
    assert abs((fy["rho"][3] - fx["rho"][3]) - 3.0) < 1e-4
    assert np.abs(np.delete(fy["rho"] - fx["rho"], 3)).max() < 1e-4
    assert np.mean(fy["codes"] != fx["codes"]) < 1e-3


# ---------------------------------------------------------------- rounding
@pytest.mark.parametrize("levels", [255, 15, 3])
def test_rtn_picks_nearest_grid_point(levels):
    r = rng(15)
    for trial in range(50):
        v = (r.standard_normal(128) * r.lognormal(0, 1)).astype(np.float32)
        q, s, z = o.rtn_group(v, levels)
        s, z = float(s), float(z)
        grid = z + s * np.arange(levels + 1)
        for i in range(128):
            d = np.abs(grid - float(v[i]))
            best = d.min()
            # the chosen level is a nearest grid point (ties within fp32 noise may go either way)
            assert d[q[i]] <= best + 1e-6 * s
        assert q.min() == 0 and q.max() == levels
        assert q[np.argmin(v)] == 0 and q[np.argmax(v)] == levels


@pytest.mark.parametrize("levels", [255, 15, 3])
def test_rtn_scale_zero_and_error_bound(levels):
    r = rng(16)
    for trial in range(50):
        v = (r.standard_normal(128) * 3.0).astype(np.float32)
        q, s, z = o.rtn_group(v, levels)
        mn, mx = float(v.min()), float(v.max())
        assert abs(float(z) - mn) <= 2.0 ** -11 * abs(mn)           # fp16 rounding of the minimum
        assert abs(float(s) - (mx - mn) / levels) <= 2.0 ** -11 * (mx - mn) / levels * 1.01
        err = np.abs(float(s) * q + float(z) - v.astype(np.float64))
        slack = abs(float(z) - mn) + levels * abs(float(s) - (mx - mn) / levels)
        assert err.max() <= float(s) / 2 * (1 + 1e-5) + slack
        assert q.dtype == np.uint8 and q.max() <= levels


def test_rtn_constant_group_is_degenerate():
    v = np.full(128, 1.2345, dtype=np.float32)
    q, s, z = o.rtn_group(v, 15)
    assert float(s) == 0.0 and np.all(q == 0) and float(z) == float(np.float16(1.2345))


def test_group_axes_key_per_channel_value_per_token():
    x = fp16_block(17)
    fk = o.quantize_tile(x, False)
    fv = o.quantize_tile(x, True)
    # every K group is a channel column: its min maps to 0 and its max to 15
    assert np.all(fk["codes"].min(axis=0) == 0) and np.all(fk["codes"].max(axis=0) == 15)
    # every V group is a token row: its min maps to 0 and its max to 3
    assert np.all(fv["codes"].min(axis=1) == 0) and np.all(fv["codes"].max(axis=1) == 3)
    assert fk["codes"].max() <= 15 and fv["codes"].max() <= 3


def test_constant_in_time_block_gives_zero_key_scales():
    row = rng(18).standard_normal(128).astype(np.float16)
    x = np.tile(row, (128, 1))
    fk = o.quantize_tile(x, False)
    assert np.all(fk["scale"] == 0) and np.all(fk["codes"] == 0)
    xh = o.dequantize_tile(fk, False)
    # only the fp16 rounding of the stored zero remains
    assert np.abs(xh - x.astype(np.float64)).max() <= 2.0 ** -10 * np.abs(x).max() * 4


# ----------------------------------------------------------------- packing
def test_k_pack_roundtrip_every_byte_value():
    b = np.arange(8192, dtype=np.int64) * 7 % 256
    buf = b.astype(np.uint8).tobytes()
    assert o.pack_k_codes(o.unpack_k_codes(buf)) == buf
    codes = rng(19).integers(0, 16, (128, 128)).astype(np.uint8)
    assert np.array_equal(o.unpack_k_codes(o.pack_k_codes(codes)), codes)


def test_v_pack_roundtrip_every_byte_value():
    b = np.arange(4096, dtype=np.int64) * 11 % 256
    buf = b.astype(np.uint8).tobytes()
    assert o.pack_v_codes(o.unpack_v_codes(buf)) == buf
    codes = rng(20).integers(0, 4, (128, 128)).astype(np.uint8)
    assert np.array_equal(o.unpack_v_codes(o.pack_v_codes(codes)), codes)


@pytest.mark.parametrize("t,c", [(0, 0), (0, 1), (5, 64), (127, 127), (33, 2)])
def test_single_code_bit_positions(t, c):
    ck = np.zeros((128, 128), np.uint8)
    ck[t, c] = 9
    bk = np.frombuffer(o.pack_k_codes(ck), np.uint8)
    assert np.flatnonzero(bk).tolist() == [64 * t + c // 2]
    assert bk[64 * t + c // 2] == 9 << (4 * (c % 2))
    cv = np.zeros((128, 128), np.uint8)
    cv[t, c] = 2
    bv = np.frombuffer(o.pack_v_codes(cv), np.uint8)
    assert np.flatnonzero(bv).tolist() == [32 * c + t // 4]
    assert bv[32 * c + t // 4] == 2 << (2 * (t % 4))


def test_page_roundtrip_and_sizes():
    x = fp16_block(21)
    for is_v, size in ((False, 9728), (True, 5632)):
        f = o.quantize_tile(x, is_v)
        pg = o.encode_page(f, is_v)
        assert len(pg) == size
        g = o.decode_page(pg, is_v)
        for k in f:
            assert np.array_equal(np.asarray(f[k]), np.asarray(g[k]))


# ------------------------------------------------------------- dequantise
def test_dequantize_closed_form():
    f = {"codes": np.zeros((128, 128), np.uint8), "scale": np.zeros(128, np.float16),
         "zero": np.ones(128, np.float16), "rho": np.zeros(128, np.float32), "gamma": np.zeros(128, np.float32)}
    f["rho"][7] = 1.0
    xh = o.dequantize_tile(f, False)
    expect = np.zeros((128, 128))
    expect[:, 0] = np.sqrt(128)
    expect[7, 0] = 2 * np.sqrt(128)
    assert np.allclose(xh, expect, atol=1e-12)


def test_kvarn_beats_plain_rtn_on_outlier_keys():
    # The rotation and normalisation exist to cut the quantisation error (normalised-cache stage).
    x = fp16_block(22, outliers=4, mult=20.0)
    xd = x.astype(np.float64)
    err_kvarn = np.linalg.norm(o.dequantize_tile(o.quantize_tile(x, False), False) - xd)
    plain = np.zeros_like(xd)
    for j in range(128):
        q, s, z = o.rtn_group(xd[:, j].astype(np.float32), 15)
        plain[:, j] = q * float(s) + float(z)
    err_plain = np.linalg.norm(plain - xd)
    assert err_kvarn < err_plain
    assert err_kvarn / np.linalg.norm(xd) < 0.12


# --------------------------------------------------------------- attention
def small_cache(seed, nblocks, hkv, perm=None):
    r = rng(seed)
    k = (r.standard_normal((nblocks * 128, hkv, 128))).astype(np.float16)
    v = (r.standard_normal((nblocks * 128, hkv, 128))).astype(np.float16)
    pages = np.arange(nblocks) if perm is None else np.asarray(perm)
    kp = np.zeros((nblocks, hkv, 9728), np.uint8)
    vp = np.zeros((nblocks, hkv, 5632), np.uint8)
    o.quantize_blocks(k, v, pages, kp, vp)
    return k, v, kp, vp, pages


def test_zero_query_gives_mean_of_values():
    _, _, kp, vp, pages = small_cache(23, 2, 1)
    q = np.zeros((1, 1, 128), np.float16)
    out = o.decode(q, kp, vp, pages[None, :], np.array([256]), 1)
    vh = o.dequantize_pages(vp, pages, 0, True)
    assert np.allclose(out[0, 0], vh.mean(axis=0), atol=1e-12)


def test_aligned_query_selects_one_value_row():
    _, _, kp, vp, pages = small_cache(24, 1, 1)
    kh = o.dequantize_pages(kp, pages, 0, False)
    vh = o.dequantize_pages(vp, pages, 0, True)
    q = (kh[40] / np.linalg.norm(kh[40]) * 200.0).astype(np.float16)[None, None, :]
    out = o.decode(q, kp, vp, pages[None, :], np.array([128]), 1, softmax_scale=1.0)
    assert np.allclose(out[0, 0], vh[40], atol=1e-6)


def test_gqa_head_mapping_and_sdpa():
    _, _, kp, vp, pages = small_cache(25, 3, 2)
    q = rng(26).standard_normal((1, 6, 128)).astype(np.float16)
    out = o.decode(q, kp, vp, pages[None, :], np.array([384]), 2)
    for h in range(6):
        g = h // 3
        kh = torch.from_numpy(o.dequantize_pages(kp, pages, g, False))
        vh = torch.from_numpy(o.dequantize_pages(vp, pages, g, True))
        qq = torch.from_numpy(q[0, h].astype(np.float64))
        ref = torch.nn.functional.scaled_dot_product_attention(qq[None, None, None], kh[None, None], vh[None, None])
        assert np.allclose(out[0, h], ref[0, 0, 0].numpy(), atol=1e-10)


def test_page_permutation_invariance():
    perm = [2, 0, 3, 1]
    k, v, kp, vp, pages = small_cache(27, 4, 1)
    kp2 = np.zeros_like(kp)
    vp2 = np.zeros_like(vp)
    o.quantize_blocks(k, v, perm, kp2, vp2)
    q = rng(28).standard_normal((1, 2, 128)).astype(np.float16)
    a = o.decode(q, kp, vp, np.arange(4)[None, :], np.array([512]), 1)
    b = o.decode(q, kp2, vp2, np.array(perm)[None, :], np.array([512]), 1)
    assert np.array_equal(a, b)


def test_empty_sequence_gives_zero_output():
    _, _, kp, vp, pages = small_cache(29, 1, 1)
    q = rng(30).standard_normal((2, 1, 128)).astype(np.float16)
    out = o.decode(q, kp, vp, np.array([[0], [0]]), np.array([0, 128]), 1)
    assert np.all(out[0, 0] == 0) and np.all(np.isfinite(out[1, 0]))


# ------------------------------------------------------- page figures (golden)
def test_format_capacity_inside_published_range():
    g = golden()
    ratio = (2 * 128 * 128 * 2) / (o.K_PAGE_BYTES + o.V_PAGE_BYTES)
    assert float(g["capacity_ratio_vs_fp16_min"]) <= ratio <= float(g["capacity_ratio_vs_fp16_max"])
    assert g["format_name"] == "kvarn_k4v2_g128"
    assert int(g["key_bits"]) == 4 and int(g["value_bits"]) == 2 and int(g["group_size"]) == 128
    # the page sizes follow from the bit widths: codes plus 2 fp16 and 2 fp32 vectors of 128
    assert o.K_PAGE_BYTES == 128 * 128 * int(g["key_bits"]) // 8 + 1536
    assert o.V_PAGE_BYTES == 128 * 128 * int(g["value_bits"]) // 8 + 1536


def test_page_metadata_offsets():
    f = {"codes": np.zeros((128, 128), np.uint8), "scale": np.full(128, 1.0, np.float16),
         "zero": np.full(128, 2.0, np.float16), "rho": np.full(128, 0.5, np.float32),
         "gamma": np.full(128, -1.0, np.float32)}
    for is_v, base in ((False, 8192), (True, 4096)):
        pg = np.frombuffer(o.encode_page(f, is_v), np.uint8)
        assert pg[base:base + 2].tolist() == [0x00, 0x3C]            # fp16 1.0, little endian
        assert pg[base + 256:base + 258].tolist() == [0x00, 0x40]    # fp16 2.0
        assert pg[base + 512:base + 516].tolist() == [0, 0, 0, 0x3F]  # fp32 0.5
        assert pg[base + 1024:base + 1028].tolist() == [0, 0, 0x80, 0xBF]  # fp32 -1.0


# ---- the fp16 baseline decode ------------------------------------------------
def fp16_cache(seed, seqs, hkv, num_pages):
    """Token-major fp16 K/V per sequence, scattered into fp16 pages through a random permutation."""
    r = rng(seed)
    perm = r.permutation(num_pages)
    kc = np.zeros((num_pages, hkv, 128, 128), np.float16)
    vc = np.zeros_like(kc)
    rows, table, nxt = [], np.zeros((len(seqs), max(seqs) // 128), np.int32), 0
    for b, n in enumerate(seqs):
        k = r.standard_normal((n, hkv, 128)).astype(np.float16)
        v = r.standard_normal((n, hkv, 128)).astype(np.float16)
        for blk in range(n // 128):
            p = perm[nxt]
            nxt += 1
            table[b, blk] = p
            kc[p] = k[128 * blk:128 * (blk + 1)].transpose(1, 0, 2)
            vc[p] = v[128 * blk:128 * (blk + 1)].transpose(1, 0, 2)
        rows.append((k, v))
    return rows, kc, vc, table


def test_fp16_decode_matches_sdpa_on_token_rows():
    seqs = [256, 384]
    rows, kc, vc, table = fp16_cache(40, seqs, 2, 6)
    q = rng(41).standard_normal((2, 6, 128)).astype(np.float16)
    out = o.fp16_decode(q, kc, vc, table, np.array(seqs), 2)
    for b in range(2):
        k, v = rows[b]
        for h in range(6):
            g = h // 3
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(q[b, h].astype(np.float64))[None, None, None],
                torch.from_numpy(k[:, g].astype(np.float64))[None, None],
                torch.from_numpy(v[:, g].astype(np.float64))[None, None])
            assert np.allclose(out[b, h], ref[0, 0, 0].numpy(), atol=1e-12)


def test_fp16_decode_equal_keys_give_mean_of_values():
    rows, kc, vc, table = fp16_cache(42, [256], 1, 2)
    kc[:] = kc[0, 0, 0]  # every key row the same: uniform weights
    q = rng(43).standard_normal((1, 1, 128)).astype(np.float16)
    out = o.fp16_decode(q, kc, vc, table, np.array([256]), 1)
    assert np.allclose(out[0, 0], rows[0][1][:, 0].astype(np.float64).mean(axis=0), atol=1e-12)


def test_fp16_decode_empty_sequence_is_zero():
    _, kc, vc, table = fp16_cache(44, [128], 1, 1)
    q = rng(45).standard_normal((1, 1, 128)).astype(np.float16)
    assert np.all(o.fp16_decode(q, kc, vc, table, np.array([0]), 1) == 0.0)


# ---- packed pages plus an fp16 tail ------------------------------------------
def test_decode_tail_reduces_to_packed_decode_and_to_plain_attention():
    k, v, kp, vp, pages = small_cache(46, 2, 2)
    q = rng(47).standard_normal((1, 4, 128)).astype(np.float16)
    tails = rng(48).standard_normal((2, 1, 128, 2, 128)).astype(np.float16)  # (K, V) x [B=1, 128, Hkv, 128]
    # no tail tokens: the packed decode
    a = o.decode_tail(q, kp, vp, pages[None, :], np.array([256]), tails[0], tails[1], 2)
    b = o.decode(q, kp, vp, pages[None, :], np.array([256]), 2)
    assert np.array_equal(a, b)
    # tail only: attention over the fp16 rows, checked with torch
    t = 77
    a = o.decode_tail(q, kp, vp, pages[None, :], np.array([t]), tails[0], tails[1], 2)
    for h in range(4):
        g = h // 2
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[0, h].astype(np.float64))[None, None, None],
            torch.from_numpy(tails[0][0, :t, g].astype(np.float64))[None, None],
            torch.from_numpy(tails[1][0, :t, g].astype(np.float64))[None, None])
        assert np.allclose(a[0, h], ref[0, 0, 0].numpy(), atol=1e-12)


def test_decode_tail_equals_softmax_over_pages_and_tail_rows():
    k, v, kp, vp, pages = small_cache(49, 2, 1)
    q = rng(50).standard_normal((1, 1, 128)).astype(np.float16)
    kt = rng(51).standard_normal((1, 128, 1, 128)).astype(np.float16)
    vt = rng(52).standard_normal((1, 128, 1, 128)).astype(np.float16)
    got = o.decode_tail(q, kp, vp, pages[None, :], np.array([256 + 5]), kt, vt, 1)
    kh = np.concatenate([o.dequantize_pages(kp, pages, 0, False), kt[0, :5, 0].astype(np.float64)])
    vh = np.concatenate([o.dequantize_pages(vp, pages, 0, True), vt[0, :5, 0].astype(np.float64)])
    logits = kh @ q[0, 0].astype(np.float64) / np.sqrt(128.0)
    w = scipy.special.softmax(logits)
    assert np.allclose(got[0, 0], w @ vh, atol=1e-12)


# ----------------------------------------------------------- chunked prefill
def _sdpa(q, k, v, mask=None, causal=False):
    """torch SDPA in fp64 for one head: q [n, 128], k/v [m, 128], boolean mask [n, m] (True = attend)."""
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))[None, None]
    m = None if mask is None else torch.from_numpy(mask)[None, None]
    return torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=m, is_causal=causal)[0, 0].numpy()


def test_prefill_equals_masked_sdpa_over_prefix_and_rows():
    # 2 packed blocks, 40 fp16 rows of which the last 25 are queries; G = 2
    _, _, kp, vp, pages = small_cache(61, 2, 2)
    r = rng(62)
    n_new, n_q = 40, 25
    kn = r.standard_normal((1, 48, 2, 128)).astype(np.float16)
    vn = r.standard_normal((1, 48, 2, 128)).astype(np.float16)
    q = r.standard_normal((1, 32, 4, 128)).astype(np.float16)
    got = o.prefill(q, kp, vp, pages[None, :], np.array([256]), kn, vn, np.array([n_new]), np.array([n_q]), 2)
    assert np.all(got[0, n_q:] == 0)
    for h in range(4):
        g = h // 2
        k = np.concatenate([o.dequantize_pages(kp, pages, g, False), kn[0, :n_new, g].astype(np.float64)])
        v = np.concatenate([o.dequantize_pages(vp, pages, g, True), vn[0, :n_new, g].astype(np.float64)])
        # query i (position 256 + 15 + i) sees keys 0 .. 256 + 15 + i
        mask = np.arange(256 + n_new)[None, :] <= (256 + n_new - n_q + np.arange(n_q))[:, None]
        ref = _sdpa(q[0, :n_q, h], k, v, mask)
        assert np.abs(got[0, :n_q, h] - ref).max() < 1e-12


def test_prefill_single_query_is_decode_with_tail():
    _, _, kp, vp, pages = small_cache(63, 3, 1)
    r = rng(64)
    kt = r.standard_normal((1, 128, 1, 128)).astype(np.float16)
    vt = r.standard_normal((1, 128, 1, 128)).astype(np.float16)
    q = r.standard_normal((1, 1, 3, 128)).astype(np.float16)
    for n_new in (1, 77, 127):
        a = o.prefill(q, kp, vp, pages[None, :], np.array([384]), kt, vt, np.array([n_new]), np.array([1]), 1)
        b = o.decode_tail(q[:, 0], kp, vp, pages[None, :], np.array([384 + n_new]), kt, vt, 1)
        assert np.abs(a[:, 0] - b).max() < 1e-12


def test_prefill_is_causal_and_empty_prefix_is_causal_sdpa():
    r = rng(65)
    n = 60
    kn = r.standard_normal((1, n, 1, 128)).astype(np.float16)
    vn = r.standard_normal((1, n, 1, 128)).astype(np.float16)
    q = r.standard_normal((1, n, 2, 128)).astype(np.float16)
    kp = np.zeros((1, 1, 9728), np.uint8)
    vp = np.zeros((1, 1, 5632), np.uint8)
    bt = np.full((1, 2), -1, np.int32)
    args = (kp, vp, bt, np.array([0]))
    a = o.prefill(q, *args, kn, vn, np.array([n]), np.array([n]), 1)
    for h in range(2):
        ref = _sdpa(q[0, :, h], kn[0, :, 0], vn[0, :, 0], causal=True)
        assert np.abs(a[0, :, h] - ref).max() < 1e-12
    # rows after a query's own position do not reach it
    kn2, vn2 = kn.copy(), vn.copy()
    kn2[0, 30:] = r.standard_normal((n - 30, 1, 128)).astype(np.float16)
    vn2[0, 30:] = 7.0
    b = o.prefill(q, *args, kn2, vn2, np.array([n]), np.array([n]), 1)
    assert np.array_equal(a[0, :30], b[0, :30])
    assert not np.allclose(a[0, 30:], b[0, 30:])


# ------------------------------------------------- format variants (8-bit keys, 4-bit values)
def test_wide_pack_roundtrips_and_sizes():
    assert (o.page_bytes(4), o.page_bytes(8), o.page_bytes(2)) == (9728, 17920, 5632)
    assert o.bits_of_page(17920, False) == 8 and o.bits_of_page(9728, True) == 4 and o.bits_of_page(9728, False) == 4
    with pytest.raises(ValueError):
        o.bits_of_page(5632, False)
    b8 = (np.arange(16384, dtype=np.int64) * 13 % 256).astype(np.uint8).tobytes()
    assert o.pack_k_codes(o.unpack_k_codes(b8, 8), 8) == b8
    b4 = (np.arange(8192, dtype=np.int64) * 7 % 256).astype(np.uint8).tobytes()
    assert o.pack_v_codes(o.unpack_v_codes(b4, 4), 4) == b4
    ck = rng(70).integers(0, 256, (128, 128)).astype(np.uint8)
    cv = rng(71).integers(0, 16, (128, 128)).astype(np.uint8)
    assert np.array_equal(o.unpack_k_codes(o.pack_k_codes(ck, 8), 8), ck)
    assert np.array_equal(o.unpack_v_codes(o.pack_v_codes(cv, 4), 4), cv)


@pytest.mark.parametrize("t,c", [(0, 0), (1, 0), (5, 64), (127, 127), (34, 3)])
def test_wide_single_code_bit_positions(t, c):
    ck = np.zeros((128, 128), np.uint8)
    ck[t, c] = 201
    bk = np.frombuffer(o.pack_k_codes(ck, 8), np.uint8)
    assert np.flatnonzero(bk).tolist() == [128 * t + c] and bk[128 * t + c] == 201
    cv = np.zeros((128, 128), np.uint8)
    cv[t, c] = 11
    bv = np.frombuffer(o.pack_v_codes(cv, 4), np.uint8)
    assert np.flatnonzero(bv).tolist() == [64 * c + t // 2]
    assert bv[64 * c + t // 2] == 11 << (4 * (t % 2))


def test_wide_rtn_nearest_grid_point_255_levels():
    r = rng(72)
    for trial in range(20):
        v = (r.standard_normal(128) * r.lognormal(0, 1)).astype(np.float32)
        q, s, z = o.rtn_group(v, 255)
        grid = float(z) + float(s) * np.arange(256)
        for i in range(128):
            d = np.abs(grid - float(v[i]))
            assert d[q[i]] <= d.min() + 1e-6 * float(s)
        assert q.min() == 0 and q.max() == 255


def test_wide_group_axes_and_error_falls_with_bits():
    x = fp16_block(73, outliers=4, mult=20.0)
    xd = x.astype(np.float64)
    fk8, fv4 = o.quantize_tile(x, False, bits=8), o.quantize_tile(x, True, bits=4)
    assert np.all(fk8["codes"].min(axis=0) == 0) and np.all(fk8["codes"].max(axis=0) == 255)
    assert np.all(fv4["codes"].min(axis=1) == 0) and np.all(fv4["codes"].max(axis=1) == 15)
    # same rotation and normalisers whatever the width; only the grid changes
    fk4 = o.quantize_tile(x, False)
    assert np.array_equal(fk8["rho"], fk4["rho"]) and np.array_equal(fk8["gamma"], fk4["gamma"])
    ek4 = np.linalg.norm(o.dequantize_tile(fk4, False) - xd)
    ek8 = np.linalg.norm(o.dequantize_tile(fk8, False) - xd)
    ev2 = np.linalg.norm(o.dequantize_tile(o.quantize_tile(x, True), True) - xd)
    ev4 = np.linalg.norm(o.dequantize_tile(fv4, True) - xd)
    # 16x and 5x finer grids: the error falls by well over the width ratio's square root
    assert ek8 < ek4 / 8 and ev4 < ev2 / 3
    for f, is_v, b in ((fk8, False, 8), (fv4, True, 4)):
        g = o.decode_page(o.encode_page(f, is_v, b), is_v)
        for key in f:
            assert np.array_equal(np.asarray(f[key]), np.asarray(g[key]))


def test_wide_pools_decode_closer_to_fp16_attention():
    r = rng(74)
    k = r.standard_normal((256, 1, 128)).astype(np.float16)
    v = r.standard_normal((256, 1, 128)).astype(np.float16)
    q = r.standard_normal((1, 4, 128)).astype(np.float16)
    pages = np.arange(2)
    exact = np.stack([o.attention(q[0, h].astype(np.float64), k[:, 0].astype(np.float64),
                                  v[:, 0].astype(np.float64), 1 / np.sqrt(128)) for h in range(4)])
    errs = {}
    for kb, vb in ((4, 2), (8, 4)):
        kp = np.zeros((2, 1, o.page_bytes(kb)), np.uint8)
        vp = np.zeros((2, 1, o.page_bytes(vb)), np.uint8)
        o.quantize_blocks(k, v, pages, kp, vp)
        errs[kb, vb] = np.abs(o.decode(q, kp, vp, pages[None, :], np.array([256]), 1)[0] - exact).max()
    assert errs[8, 4] < errs[4, 2] / 3


# ---- group size 64 ----------------------------------------------------------------------------------------
# Reading: every group of the group-128 format splits into two halves of 64 consecutive elements (keys: one
# channel over tokens 64h .. 64h+63; values: one token over channels 64h .. 64h+63), each with its own scale
# and zero stored half-major; every other step is unchanged.

def test_g64_page_sizes_and_format_lookup():
    assert (o.page_bytes(4, 64), o.page_bytes(8, 64), o.page_bytes(2, 64)) == (10240, 18432, 6144)
    for is_v, widths in ((False, (4, 8)), (True, (2, 4))):
        for b in widths:
            for gs in (128, 64):
                assert o.format_of_page(o.page_bytes(b, gs), is_v) == (b, gs)


@pytest.mark.parametrize("is_v,bits", [(False, 4), (True, 2), (False, 8), (True, 4)])
def test_g64_groups_are_subsets_of_g128_groups(is_v, bits):
    """A half group's range lies inside its whole group's: scale no larger, zero no smaller (fp16 rounding
    is monotone), and strictly inside for at least one half of every group of random data."""
    x = fp16_block(81 + bits, outliers=4, mult=20.0)
    f128 = o.quantize_tile(x, is_v, bits=bits)
    f64 = o.quantize_tile(x, is_v, bits=bits, group=64)
    assert f64["scale"].shape == (2, 128) and f64["zero"].shape == (2, 128)
    assert np.array_equal(f64["rho"], f128["rho"]) and np.array_equal(f64["gamma"], f128["gamma"])
    s128, z128 = f128["scale"].astype(np.float64), f128["zero"].astype(np.float64)
    s64, z64 = f64["scale"].astype(np.float64), f64["zero"].astype(np.float64)
    assert np.all(s64 <= s128[None, :]) and np.all(z64 >= z128[None, :])
    # each whole group's minimum sits in one of its halves, whose zero then equals the whole group's
    assert np.all(np.minimum(z64[0], z64[1]) == z128)
    # every whole group has a strictly narrower half (the half without its minimum or its maximum); the
    # half holding both (about one group in two) keeps the whole range
    assert np.all(np.minimum(s64[0], s64[1]) < s128)
    assert 0.6 < (s64 < s128[None, :]).mean() < 0.95


@pytest.mark.parametrize("is_v,bits", [(False, 4), (True, 2), (False, 8), (True, 4)])
def test_g64_codes_reconstruct_on_their_own_half_grid(is_v, bits):
    """Every element lies within half a step of z + s*code on the grid of the half it belongs to (keys: the
    token's half, values: the channel's half), up to the fp16 rounding of the grid's ends; the other half's
    grid misses some elements by far more."""
    x = fp16_block(91 + bits, outliers=4, mult=20.0)
    f = o.quantize_tile(x, is_v, bits=bits, group=64)
    n = o.normalized(o.rotate(x.astype(np.float64)), f["rho"], f["gamma"])
    levels = (1 << bits) - 1

    def worst(scale, zero):
        g = {"scale": scale, "zero": zero}
        s, z = [a.astype(np.float64) for a in o.group_params(g, is_v)]
        err = np.abs(n - (z + s * f["codes"]))
        slack = 2.0 ** -10 * np.maximum(np.abs(z), np.abs(z + levels * s)) + 1e-6
        return float((err / (s / 2 + slack)).max())

    assert worst(f["scale"], f["zero"]) <= 1.0
    assert worst(f["scale"][::-1], f["zero"][::-1]) > 2.0


def test_g64_equals_g128_when_the_halves_repeat():
    """Tokens 64..127 repeating tokens 0..63 and channels 64..127 empty make both halves of every group hold
    the same normalised values (H maps [a, 0] to [H64 a, H64 a] / sqrt 2), so the half groups carry the
    whole groups' scale, zero and codes."""
    r = rng(95)
    x = np.zeros((128, 128))
    x[:64, :64] = r.standard_normal((64, 64)) * np.where(r.random(64) < 0.1, 15.0, 1.0)[None, :]
    x[64:, :64] = x[:64, :64]
    x = x.astype(np.float16)
    for is_v, bits in ((False, 4), (True, 2), (False, 8), (True, 4)):
        f128 = o.quantize_tile(x, is_v, bits=bits)
        f64 = o.quantize_tile(x, is_v, bits=bits, group=64)
        assert np.array_equal(f64["codes"], f128["codes"])
        for key in ("scale", "zero"):
            assert np.array_equal(f64[key][0], f128[key]) and np.array_equal(f64[key][1], f128[key])


def test_g64_page_layout_half_major():
    sc = np.arange(256, dtype=np.float16).reshape(2, 128)
    f = {"codes": np.zeros((128, 128), np.uint8), "scale": sc, "zero": -sc,
         "rho": np.full(128, 0.5, np.float32), "gamma": np.full(128, -1.0, np.float32)}
    for is_v, bits, base in ((False, 4, 8192), (True, 2, 4096), (False, 8, 16384), (True, 4, 8192)):
        pg = o.encode_page(f, is_v, bits)
        assert len(pg) == o.page_bytes(bits, 64)
        a = np.frombuffer(pg, np.uint8)
        # entry 128*h + j: scale of half 1, index 2 is 130.0 at byte 2 * 130
        assert np.frombuffer(a[base + 260:base + 262].tobytes(), "<f2")[0] == 130.0
        assert np.frombuffer(a[base + 512 + 260:base + 512 + 262].tobytes(), "<f2")[0] == -130.0
        assert a[base + 1024:base + 1028].tolist() == [0, 0, 0, 0x3F]
        assert a[base + 1536:base + 1540].tolist() == [0, 0, 0x80, 0xBF]
        g = o.decode_page(pg, is_v)
        for key in f:
            assert np.array_equal(np.asarray(f[key]), np.asarray(g[key]))


def test_g64_reconstruction_error_below_g128():
    x = fp16_block(97, outliers=4, mult=20.0)
    xd = x.astype(np.float64)
    for is_v in (False, True):
        e128 = np.linalg.norm(o.dequantize_tile(o.quantize_tile(x, is_v), is_v) - xd)
        e64 = np.linalg.norm(o.dequantize_tile(o.quantize_tile(x, is_v, group=64), is_v) - xd)
        assert e64 < e128
