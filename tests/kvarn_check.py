"""Comparison of the HIP path against the CPU oracle (test infrastructure).

Tolerances (from the spec parity bar and the fp32 arithmetic of the kernels):
  * codes: mismatch fraction <= 1e-4 and every mismatch within one level;
    near-ties decide differently because the kernel computes the normalised
    value in fp32 in a different order than the fp64 oracle;
  * scale / zero: fp16 values equal or one fp16 ulp apart (a group minimum or
    range that lands within fp32 noise of an fp16 rounding boundary);
  * rho / gamma: |diff| <= NORM_TOL * max(1, |x|) (log2 units); the kernel's
    variances carry fp32 sums of 128 terms and hardware log2/exp2;
  * dequantised cache and attention output: max-abs <= 2e-3 with the same
    packed bytes on both sides (fp32 accumulation on the GPU).
"""
from __future__ import annotations

import numpy as np

from oracle import kvarn_oracle as o

CODE_MISMATCH_FRACTION = 1e-4
NORM_TOL = 1e-5  # relative bar for rho and gamma; the kernels measure <= 5.1e-7
DEQUANT_TOL = 2e-3
ATTN_TOL = 2e-3


def f16_ulp_distance(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in fp16 ulps between two fp16 arrays (sign-magnitude ordering)."""
    ia = np.asarray(a, dtype=np.float16).view(np.int16).astype(np.int32)
    ib = np.asarray(b, dtype=np.float16).view(np.int16).astype(np.int32)
    ia = np.where(ia < 0, -(ia & 0x7FFF), ia)
    ib = np.where(ib < 0, -(ib & 0x7FFF), ib)
    return np.abs(ia - ib)


class TileStats:
    def __init__(self):
        self.codes = 0
        self.code_mismatch = 0
        self.code_maxdiff = 0
        self.cond_mismatch = 0
        self.groups = 0
        self.sz_exact = 0
        self.sz_maxulp = 0
        self.norm_maxerr = 0.0
        self.tiles = 0

    def summary(self) -> str:
        return ("tiles %d codes %d mismatch %d (%.2e) maxdiff %d | given-stored-grid mismatch %d | "
                "scale/zero exact %d/%d max ulp %d | rho/gamma max rel err %.2e"
                % (self.tiles, self.codes, self.code_mismatch, self.code_mismatch / max(1, self.codes),
                   self.code_maxdiff, self.cond_mismatch, self.sz_exact, 2 * self.groups, self.sz_maxulp,
                   self.norm_maxerr))

    def merge(self, other: "TileStats") -> None:
        for key in ("codes", "code_mismatch", "cond_mismatch", "groups", "sz_exact", "tiles"):
            setattr(self, key, getattr(self, key) + getattr(other, key))
        self.code_maxdiff = max(self.code_maxdiff, other.code_maxdiff)
        self.sz_maxulp = max(self.sz_maxulp, other.sz_maxulp)
        self.norm_maxerr = max(self.norm_maxerr, other.norm_maxerr)

    def check(self):
        assert self.code_maxdiff <= 1, self.summary()
        assert self.code_mismatch <= CODE_MISMATCH_FRACTION * self.codes, self.summary()
        assert self.cond_mismatch <= CODE_MISMATCH_FRACTION * self.codes, self.summary()
        assert self.sz_maxulp <= 1, self.summary()
        assert self.norm_maxerr <= NORM_TOL, self.summary()


def compare_tile(stats: TileStats, x16: np.ndarray, page_bytes: bytes, is_v: bool) -> None:
    """Compare one GPU-written page against the oracle's quantisation of the same fp16 tile."""
    bits, group = o.format_of_page(len(page_bytes), is_v)  # the format's code width and group size
    ref = o.quantize_tile(x16, is_v, bits=bits, group=group)
    got = o.decode_page(page_bytes, is_v)
    stats.tiles += 1
    for key in ("rho", "gamma"):
        a = got[key].astype(np.float64)
        b = ref[key].astype(np.float64)
        err = np.abs(a - b) / np.maximum(1.0, np.abs(b))
        stats.norm_maxerr = max(stats.norm_maxerr, float(err.max()))
    for key in ("scale", "zero"):
        d = f16_ulp_distance(got[key], ref[key])
        stats.sz_exact += int((d == 0).sum())
        stats.sz_maxulp = max(stats.sz_maxulp, int(d.max()))
    stats.groups += ref["scale"].size
    diff = np.abs(got["codes"].astype(np.int32) - ref["codes"].astype(np.int32))
    stats.codes += diff.size
    stats.code_mismatch += int((diff != 0).sum())
    stats.code_maxdiff = max(stats.code_maxdiff, int(diff.max()))
    # the rounding decision alone: oracle codes on the GPU's stored normalisers and grid
    n32 = o.normalized(o.rotate(x16.astype(np.float64)), got["rho"], got["gamma"]).astype(np.float32)
    cond = np.zeros_like(got["codes"])
    levels = (1 << bits) - 1
    gs, gz = got["scale"].reshape(-1, 128), got["zero"].reshape(-1, 128)
    for h in range(gs.shape[0]):
        seg = slice(group * h, group * (h + 1))
        for gi in range(128):
            if is_v:
                cond[gi, seg] = o.rtn_codes(n32[gi, seg], gs[h, gi], gz[h, gi], levels)
            else:
                cond[seg, gi] = o.rtn_codes(n32[seg, gi], gs[h, gi], gz[h, gi], levels)
    stats.cond_mismatch += int((cond != got["codes"]).sum())


# ------------------------------------------------------------------ whole pools (vectorised)
def unpack_codes(pool: np.ndarray, is_v: bool, bits: int, head_dim: int = 128) -> np.ndarray:
    """Codes [..., 128 tokens, head_dim channels] of every page in a pool [..., page_bytes]."""
    d = head_dim
    lead = pool.shape[:-1]
    if not is_v:
        if bits == 8:
            return pool[..., :128 * d].reshape(lead + (128, d))
        b = pool[..., :64 * d].reshape(lead + (128, d // 2))
        return np.stack([b & 15, b >> 4], axis=-1).reshape(lead + (128, d))
    per = 8 // bits
    b = pool[..., :d * 128 // per].reshape(lead + (d, 128 // per))
    parts = [(b >> (bits * i)) & ((1 << bits) - 1) for i in range(per)]  # token per*k + i
    return np.swapaxes(np.stack(parts, axis=-1).reshape(lead + (d, 128)), -1, -2)


def meta_views(pool: np.ndarray, is_v: bool, bits: int, group: int, head_dim: int = 128):
    """(scale, zero, rho, gamma) arrays of every page of a pool, from the page layout."""
    d = head_dim
    code = 128 * d * bits // 8
    n = (d // min(group, d)) * 128 if is_v else (128 // group) * d
    meta = np.ascontiguousarray(pool[..., code:])
    scale = meta[..., :2 * n].view("<f2")
    zero = meta[..., 2 * n:4 * n].view("<f2")
    rho = meta[..., 4 * n:4 * n + 512].view("<f4")
    gam = meta[..., 4 * n + 512:4 * n + 512 + 4 * d].view("<f4")
    return scale, zero, rho, gam


def compare_pools(stats: TileStats, got: np.ndarray, ref: np.ndarray, is_v: bool, bits: int, group: int,
                  head_dim: int = 128) -> None:
    """Compare pages the GPU wrote with the oracle's pages for the same inputs, many pages at once.

    got, ref: uint8 [..., page_bytes] holding the same (block, head) units in the same order."""
    assert got.shape == ref.shape
    n_pages = int(np.prod(got.shape[:-1]))
    flat_g = got.reshape(n_pages, got.shape[-1])
    flat_r = ref.reshape(n_pages, ref.shape[-1])
    chunk = 512
    for a in range(0, n_pages, chunk):
        g, r = flat_g[a:a + chunk], flat_r[a:a + chunk]
        diff = np.abs(unpack_codes(g, is_v, bits, head_dim).astype(np.int16)
                      - unpack_codes(r, is_v, bits, head_dim).astype(np.int16))
        stats.codes += diff.size
        stats.code_mismatch += int(np.count_nonzero(diff))
        stats.code_maxdiff = max(stats.code_maxdiff, int(diff.max()))
        mg, mr = meta_views(g, is_v, bits, group, head_dim), meta_views(r, is_v, bits, group, head_dim)
        for x, y in zip(mg[:2], mr[:2]):
            d = f16_ulp_distance(x, y)
            stats.sz_exact += int((d == 0).sum())
            stats.sz_maxulp = max(stats.sz_maxulp, int(d.max()))
        stats.groups += mr[0].size
        for x, y in zip(mg[2:], mr[2:]):
            x64, y64 = x.astype(np.float64), y.astype(np.float64)
            err = np.abs(x64 - y64) / np.maximum(1.0, np.abs(y64))
            stats.norm_maxerr = max(stats.norm_maxerr, float(err.max()))
        stats.tiles += g.shape[0]
