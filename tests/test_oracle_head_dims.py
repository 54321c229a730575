"""Pins of the oracles at head_dim 64 and 256 (CPU).

Readings for a head of D channels, each the head_dim-128 format with D in place of 128 along the
channel axis (the post names kvarn_k4v2_g128; the name carries no head size):
  * rotation by the D-point Sylvester Hadamard matrix divided by sqrt(D);
  * row passes take the variance over D channels, column passes over the block's 128 tokens;
  * key groups: one channel over `group` tokens (as at D = 128);
  * value groups: one token over min(group, D) channels, so a 64-channel head has one value group per
    token at either group size, and a 256-channel head two (group 128) or four (group 64);
  * page = codes | scale | zero | rho fp32[128] | gamma fp32[D]; scale/zero entry D*h + j for keys,
    128*h + t for values;
  * decode scales logits by 1/sqrt(D).
"""
import math

import numpy as np
import pytest
import scipy.linalg
import torch

from oracle import kvarn_oracle as o
from oracle import kvarn_oracle_cpp as C

DIMS = [64, 256]
FORMATS = [(4, 2, 128), (8, 4, 128), (4, 2, 64), (8, 4, 64), (4, 4, 128), (8, 2, 64)]


@pytest.fixture(scope="module", autouse=True)
def built():
    C.build()


def block(d, seed, outliers=4, mult=20.0):
    g = np.random.default_rng(seed)
    x = g.standard_normal((128, d))
    x[:, g.choice(d, outliers, replace=False)] *= mult
    return x.astype(np.float16)


def vblock(d, seed):
    g = np.random.default_rng(seed)
    return (g.standard_normal((128, d)) * np.exp(0.5 * g.standard_normal((128, 1)))).astype(np.float16)


@pytest.mark.parametrize("d", DIMS)
def test_hadamard_and_rotation_at_d(d):
    h = o.hadamard(d)
    assert np.allclose(h, scipy.linalg.hadamard(d) / np.sqrt(d), rtol=0, atol=1e-15)
    assert np.abs(h @ h - np.eye(d)).max() < 1e-14
    x = block(d, 1).astype(np.float64)
    r = o.rotate(x)
    assert np.allclose(np.linalg.norm(r, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    q = np.random.default_rng(2).standard_normal(d)
    assert np.allclose(r @ (h @ q), x @ q, rtol=1e-12, atol=1e-10)  # scores kept under joint rotation


@pytest.mark.parametrize("d", DIMS)
@pytest.mark.parametrize("kb,vb,group", FORMATS)
def test_page_sizes_and_layout_at_d(d, kb, vb, group):
    nk = (128 // group) * d
    nv = (d // min(group, d)) * 128
    assert o.page_bytes(kb, group, d, False) == 128 * d * kb // 8 + 4 * nk + 512 + 4 * d
    assert o.page_bytes(vb, group, d, True) == 128 * d * vb // 8 + 4 * nv + 512 + 4 * d
    assert o.format_of_page(o.page_bytes(kb, group, d, False), False, d) == (kb, group)
    vfmt = o.format_of_page(o.page_bytes(vb, group, d, True), True, d)
    # at D = 64 one value group spans the token row at either group size: the pages are the same
    assert vfmt == (vb, group) or (d == 64 and vfmt == (vb, 128))
    assert C.page_bytes(kb, group, d, False) == o.page_bytes(kb, group, d, False)
    assert C.page_bytes(vb, group, d, True) == o.page_bytes(vb, group, d, True)
    for is_v, bits, x in ((False, kb, block(d, 3)), (True, vb, vblock(d, 4))):
        f = o.quantize_tile(x, is_v, bits=bits, group=group)
        page = o.encode_page(f, is_v, bits)
        assert len(page) == o.page_bytes(bits, group, d, is_v)
        back = o.decode_page(page, is_v, d)
        for key in ("codes", "scale", "zero", "rho", "gamma"):
            assert np.array_equal(np.asarray(back[key]), np.asarray(f[key])), key
        assert f["codes"].shape == (128, d) and f["gamma"].shape == (d,) and f["rho"].shape == (128,)
        # one code: byte positions of the layout
        t, c = 37, d - 3
        codes = np.zeros((128, d), np.uint8)
        codes[t, c] = (1 << bits) - 1
        packed = np.frombuffer(o.pack_v_codes(codes, bits) if is_v else o.pack_k_codes(codes, bits), np.uint8)
        nz = np.nonzero(packed)[0]
        if not is_v:
            assert list(nz) == [d * t + c if bits == 8 else (d // 2) * t + c // 2]
        else:
            assert list(nz) == [32 * c + t // 4 if bits == 2 else 64 * c + t // 2]


@pytest.mark.parametrize("d", DIMS)
@pytest.mark.parametrize("is_v,bits,group", [(False, 4, 128), (True, 2, 128), (False, 8, 64), (True, 4, 64)])
def test_rtn_nearest_grid_point_and_error_bound_at_d(d, is_v, bits, group):
    x = vblock(d, 5) if is_v else block(d, 6)
    f = o.quantize_tile(x, is_v, bits=bits, group=group)
    n32 = o.normalized(o.rotate(x.astype(np.float64)), f["rho"], f["gamma"]).astype(np.float32)
    s, z = [a.astype(np.float64) for a in o.group_params(f, is_v)]
    levels = (1 << bits) - 1
    assert f["codes"].max() <= levels
    # brute force: each code is the nearest grid point of its own group (ties aside)
    grid = z[..., None] + s[..., None] * np.arange(levels + 1)
    dist = np.abs(n32[..., None].astype(np.float64) - grid)
    best = dist.min(axis=-1)
    chosen = np.take_along_axis(dist, f["codes"][..., None].astype(np.int64), axis=-1)[..., 0]
    assert np.all(chosen <= best + 1e-3 * s + 1e-12)
    err = np.abs(n32 - (z + s * f["codes"]))
    assert np.all(err <= s / 2 + 1e-3 * s + 2.0 ** -11 * np.abs(z) + 1e-30)


@pytest.mark.parametrize("d", DIMS)
def test_group_axes_at_d(d):
    """Key groups are per channel (one scale per channel); value groups are per token over min(128, D)
    channels, and each one reaches both ends of its own grid (its minimum is code 0, its maximum L)."""
    x = block(d, 7)
    f = o.quantize_tile(x, False, group=128)
    assert np.asarray(f["scale"]).shape == (d,)
    fv = o.quantize_tile(vblock(d, 8), True, group=128)
    gv = min(128, d)
    assert np.asarray(fv["scale"]).shape == ((128,) if d // gv == 1 else (d // gv, 128))
    # every value group reaches both ends of its grid: the group min is code 0, the max code L
    s, z = o.group_params(fv, True)
    n32 = o.normalized(o.rotate(vblock(d, 8).astype(np.float64)), fv["rho"], fv["gamma"]).astype(np.float32)
    for h in range(d // gv):
        seg = slice(gv * h, gv * (h + 1))
        for t in (0, 50, 127):
            row = n32[t, seg]
            assert fv["codes"][t, seg][np.argmin(row)] == 0
            assert fv["codes"][t, seg][np.argmax(row)] == 3


def test_d64_value_groups_span_the_row_at_both_group_sizes():
    x = vblock(64, 9)
    a = o.encode_page(o.quantize_tile(x, True, group=128), True)
    b = o.encode_page(o.quantize_tile(x, True, group=64), True)
    assert a == b and len(a) == o.page_bytes(2, 128, 64, True) == o.page_bytes(2, 64, 64, True)


def test_d256_value_rows_are_two_groups():
    """At D = 256 a value row is two groups of 128 channels, each with its own scale and zero, and every
    element lies on the grid of its own half."""
    x = vblock(256, 10)
    f = o.quantize_tile(x, True, group=128)
    s = np.asarray(f["scale"])
    assert s.shape == (2, 128)
    # not equal in general ...
    assert not np.array_equal(s[0], s[1])
    # ... but every element lies on its own half's grid
    sg, zg = [a.astype(np.float64) for a in o.group_params(f, True)]
    n = o.normalized(o.rotate(x.astype(np.float64)), f["rho"], f["gamma"])
    assert np.all(np.abs(n - (zg + sg * f["codes"])) <= sg / 2 * (1 + 1e-3) + 2.0 ** -10 * np.abs(zg) + 1e-30)


@pytest.mark.parametrize("d", DIMS)
def test_dequantize_closed_form_and_rotation_back(d):
    x = block(d, 11)
    f = o.quantize_tile(x, False, bits=8)
    xh = o.dequantize_tile(f, False)
    s, z = o.group_params(f, False)
    r_hat = (f["codes"] * s.astype(np.float64) + z.astype(np.float64)) * np.exp2(
        f["rho"].astype(np.float64)[:, None] + f["gamma"].astype(np.float64)[None, :])
    assert np.allclose(xh, r_hat @ o.hadamard(d), rtol=0, atol=1e-9)
    # 8-bit keys rebuild the block closely
    xf = x.astype(np.float64)
    assert np.linalg.norm(xh - xf) / np.linalg.norm(xf) < 0.02


@pytest.mark.parametrize("d", DIMS)
def test_decode_at_d_equals_sdpa_on_the_dequantised_cache(d):
    g = np.random.default_rng(12)
    hkv, hq, nb = 2, 6, 3
    k = np.concatenate([block(d, 20 + i)[:, None] for i in range(hkv)], axis=1)
    k = np.concatenate([k] * nb)
    v = np.concatenate([np.concatenate([vblock(d, 30 + i + j) for j in range(nb)])[:, None] for i in range(hkv)],
                       axis=1)
    kp = np.zeros((nb, hkv, o.page_bytes(4, 128, d, False)), np.uint8)
    vp = np.zeros((nb, hkv, o.page_bytes(2, 128, d, True)), np.uint8)
    o.quantize_blocks(k, v, np.array([2, 0, 1]), kp, vp)
    q = g.standard_normal((2, hq, d)).astype(np.float16)
    bt = np.array([[2, 0, 1], [1, -1, -1]], np.int32)
    sl = np.array([384, 128], np.int32)
    out = o.decode(q, kp, vp, bt, sl, hkv)
    for b in range(2):
        pages = bt[b, :sl[b] // 128]
        for h in range(hq):
            kh = o.dequantize_pages(kp, pages, h // 3, False, d)
            vh = o.dequantize_pages(vp, pages, h // 3, True, d)
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(q[b, h].astype(np.float64))[None, None, None],
                torch.from_numpy(kh)[None, None], torch.from_numpy(vh)[None, None])[0, 0, 0].numpy()
            assert np.abs(out[b, h] - ref).max() < 1e-12
    assert math.isclose(1 / math.sqrt(d), 1 / np.sqrt(d))
    # the C++ oracle agrees
    assert np.abs(C.decode(q, kp, vp, bt, sl, hkv) - out).max() < 1e-10


@pytest.mark.parametrize("d", DIMS)
@pytest.mark.parametrize("kb,vb,group", FORMATS)
def test_cpp_pages_identical_to_python_at_d(d, kb, vb, group):
    for is_v, bits, x in ((False, kb, block(d, 40)), (True, vb, vblock(d, 41))):
        ref = o.encode_page(o.quantize_tile(x, is_v, bits=bits, group=group), is_v, bits)
        for fwht in (False, True):
            assert C.quantize_tile_page(x, is_v, bits, group, fwht) == ref
    f = o.decode_page(ref, True, d)
    assert np.abs(C.dequantize_page(ref, True, vb, group, d) - o.dequantize_tile(f, True)).max() < 1e-12
