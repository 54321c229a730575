"""CPU oracle for KVarN block quantisation and decode attention over the packed cache.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or link
this module: it exists so that the tests, the package smoke check and the
CPU-baseline leg of the benchmark can compare the HIP path against a plain, slow
and obviously correct definition.  It shares no code, constants table or helper
with the HIP library; it only reads the page byte format, which it implements
on its own from the description below.

Sources.  The method is described in the KVarN blog post ("KVarN: Huawei'den
KV-Cache Kuantizasyonu için Yerel vLLM Backend'i"), section "KVarN Nasıl
Çalışır?": the cache is quantised in fixed-size token blocks, and every block
goes through four stages -- the raw fp16 block, an orthonormal Hadamard rotation
along the channel dimension, a Sinkhorn-like row/column variance normalisation
in log space, and low-bit asymmetric round-to-nearest with 4-bit keys and 2-bit
values.  Section "Pratik Çıkarımlar" of the same post names the format
``kvarn_k4v2_g128`` (group size 128).  Paged storage with a block table and
GQA head sharing come from the "KV Cache" glossary page, sections "Boyutu ve
Yönetimi" and "Türleri".

Parameters the pages leave open, fixed here (each is one reading):
  * block = 128 tokens, head_dim = 128, normalisation iterations T = 4,
    eps = 1e-6 added to the variance, log base 2;
  * rotation: the natural-order Sylvester Hadamard matrix H[j,k] =
    (-1)^popcount(j&k) / sqrt(128), no random signs, applied to K and V;
  * "variance" = centred population variance; each iteration does the row pass
    (over channels, per token) first, then the column pass (over tokens, per
    channel); both normalisers start at 0;
  * key groups: one channel over the 128 tokens of the block (L = 15);
    value groups: one token over the 128 channels (L = 3);
  * scale and zero stored as fp16; the zero is the group minimum (a float
    offset); normalisers stored as fp32 log2 values, and the normalised values
    that get quantised use the stored fp32 normalisers;
  * the rounding decision is taken in fp32 (the precision the kernel computes
    in): u = fp32(fp32(N - z) / s), code = clamp(round-half-even(u), 0, L);
    a group whose fp16 scale is 0 stores all-zero codes;
  * formats: the post names kvarn_k4v2_g128; the same name pattern with 8-bit
    keys and 4-bit values (kvarn_k{4,8}v{2,4}_g128) keeps every step and changes
    only the number of levels (2^bits - 1) and the packing: 8-bit key codes one
    byte each, token-major (byte 128*t + c); 4-bit value codes channel-major, two
    tokens per byte (byte 64*c + t//2, even token in the low nibble).  A page's
    bit width follows from its byte count;
  * group size 64 (kvarn_k{4,8}v{2,4}_g64): each group of the group-128 format
    splits into two halves of 64 consecutive elements -- a key group is one
    channel over tokens 64h .. 64h+63, a value group one token over channels
    64h .. 64h+63 -- each with its own fp16 scale and zero, stored half-major
    (entry 128*h + j); every other step is unchanged;
  * decode: query head h reads KV head h // (Hq / Hkv); logits scaled by
    1/sqrt(128) unless a positive scale is given; plain softmax; output in the
    original (unrotated) basis.

Floating point is fp64 everywhere except where the format stores a narrower
type or where the rounding decision is taken (fp32, see above).
"""
from __future__ import annotations

import numpy as np

BLOCK = 128
HEAD_DIM = 128
ITERS = 4
EPS = 1e-6
K_LEVELS = 15  # 4-bit keys (the format the post names)
V_LEVELS = 3   # 2-bit values
K_BITS_ALLOWED = (4, 8)
V_BITS_ALLOWED = (2, 4)
GROUPS_ALLOWED = (128, 64)
META_BYTES = 2 * 256 + 2 * 512  # group size 128

# Page byte format (one page = one 128-token block of one KV head).
K_CODES_BYTES = BLOCK * HEAD_DIM // 2      # 8192: token-major, two channels per byte
V_CODES_BYTES = BLOCK * HEAD_DIM // 4      # 4096: channel-major, four tokens per byte
K_PAGE_BYTES = K_CODES_BYTES + 2 * 256 + 2 * 512   # 9728
V_PAGE_BYTES = V_CODES_BYTES + 2 * 256 + 2 * 512   # 5632


HEAD_DIMS_ALLOWED = (64, 128, 256)


def value_group_channels(group: int, head_dim: int = HEAD_DIM) -> int:
    """Channels in one value group: the group size, or the whole token row when the head is narrower."""
    return min(group, head_dim)


def n_groups(group: int, head_dim: int = HEAD_DIM, is_v: bool = False) -> int:
    """Scale/zero entries of one page: keys have 128 // group groups per channel, values head_dim //
    value_group_channels groups per token."""
    if is_v:
        return (head_dim // value_group_channels(group, head_dim)) * BLOCK
    return (BLOCK // group) * head_dim


def meta_bytes(group: int = 128, head_dim: int = HEAD_DIM, is_v: bool = False) -> int:
    """Metadata of one page: scale and zero fp16 per group, rho fp32[128 tokens], gamma fp32[head_dim]."""
    return 2 * 2 * n_groups(group, head_dim, is_v) + 4 * BLOCK + 4 * head_dim


def page_bytes(bits: int, group: int = 128, head_dim: int = HEAD_DIM, is_v: bool = False) -> int:
    """Bytes of one page whose codes have `bits` bits: 128 x head_dim codes plus the metadata."""
    return BLOCK * head_dim * bits // 8 + meta_bytes(group, head_dim, is_v)


def format_of_page(nbytes: int, is_v: bool, head_dim: int = HEAD_DIM):
    """(code width, group size) of a page from its byte count (unambiguous within keys and within values
    of one head size)."""
    for b in (V_BITS_ALLOWED if is_v else K_BITS_ALLOWED):
        for gs in GROUPS_ALLOWED:
            if nbytes == page_bytes(b, gs, head_dim, is_v):
                return b, gs
    raise ValueError("a %s page of %d bytes matches no format at head_dim %d"
                     % ("value" if is_v else "key", nbytes, head_dim))


def bits_of_page(nbytes: int, is_v: bool, head_dim: int = HEAD_DIM) -> int:
    """Code width of a page from its byte count."""
    return format_of_page(nbytes, is_v, head_dim)[0]


# --------------------------------------------------------------------------
# Stage 2: rotation (blog post, "KVarN Nasıl Çalışır?", rotated-cache stage)
# --------------------------------------------------------------------------
def hadamard(n: int = HEAD_DIM) -> np.ndarray:
    """Orthonormal Sylvester Hadamard matrix, entry (j, k) = (-1)^popcount(j & k) / sqrt(n)."""
    h = np.empty((n, n), dtype=np.float64)
    for j in range(n):
        for k in range(n):
            h[j, k] = -1.0 if bin(j & k).count("1") % 2 else 1.0
    return h / np.sqrt(n)


_H_BY_SIZE = {}


def _h(n: int) -> np.ndarray:
    if n not in _H_BY_SIZE:
        _H_BY_SIZE[n] = hadamard(n)
    return _H_BY_SIZE[n]


_H = _h(HEAD_DIM)


def rotate(x: np.ndarray) -> np.ndarray:
    """Rotate every token row of a [tokens, D] block along its D channels: R[t] = H_D @ x[t]."""
    x = np.asarray(x, dtype=np.float64)
    return x @ _h(x.shape[-1]).T


# --------------------------------------------------------------------------
# Stage 3: log-space row/column variance normalisation
# (blog post, "KVarN Nasıl Çalışır?", normalised-cache stage)
# --------------------------------------------------------------------------
def normalize(r: np.ndarray, iters: int = ITERS, eps: float = EPS):
    """Return log2 normalisers (rho per token row, gamma per channel column), fp64.

    The normalised block is N[t, j] = R[t, j] * 2^-(rho[t] + gamma[j]).  Each
    iteration: for every row, add half the log2 of (row variance + eps) to rho;
    then for every column, add half the log2 of (column variance + eps) to
    gamma, each variance taken of the current normalised block.
    """
    r = np.asarray(r, dtype=np.float64)
    rho = np.zeros(r.shape[0])
    gam = np.zeros(r.shape[1])
    for _ in range(iters):
        y = r * np.exp2(-(rho[:, None] + gam[None, :]))
        rho = rho + 0.5 * np.log2(y.var(axis=1) + eps)
        y = r * np.exp2(-(rho[:, None] + gam[None, :]))
        gam = gam + 0.5 * np.log2(y.var(axis=0) + eps)
    return rho, gam


def normalized(r: np.ndarray, rho32: np.ndarray, gam32: np.ndarray) -> np.ndarray:
    """N = R * 2^-(rho + gamma) from the stored fp32 normalisers, in fp64."""
    rho = np.asarray(rho32, dtype=np.float32).astype(np.float64)
    gam = np.asarray(gam32, dtype=np.float32).astype(np.float64)
    return np.asarray(r, dtype=np.float64) * np.exp2(-(rho[:, None] + gam[None, :]))


# --------------------------------------------------------------------------
# Stage 4: asymmetric round-to-nearest
# (blog post, "KVarN Nasıl Çalışır?", quantised-cache stage: 4-bit keys, 2-bit
# values; "Pratik Çıkarımlar": group size 128)
# --------------------------------------------------------------------------
def rtn_group(values: np.ndarray, levels: int):
    """Quantise one group of normalised values.  Returns (codes uint8, scale fp16, zero fp16).

    The decision is taken in fp32: the group minimum and maximum of the fp32
    values give scale = fp16(fp32(fp32(max - min) / levels)) and zero =
    fp16(min); each code is round-half-even of fp32(fp32(v - zero) / scale),
    clamped to [0, levels].  A zero scale gives all-zero codes.
    """
    v = np.asarray(values, dtype=np.float32)
    mn = v.min()
    mx = v.max()
    s32 = np.float32(np.float32(mx - mn) / np.float32(levels))
    s16 = np.float16(s32)
    z16 = np.float16(mn)
    return rtn_codes(v, s16, z16, levels), s16, z16


def rtn_codes(values: np.ndarray, s16, z16, levels: int) -> np.ndarray:
    """Codes of fp32 values on the stored grid z + s*c: clamp(rint(fp32(fp32(v - z) / s)), 0, levels); s == 0 gives 0."""
    v = np.asarray(values, dtype=np.float32)
    if float(s16) == 0.0:
        return np.zeros(v.shape, dtype=np.uint8)
    u = (v - np.float32(z16)).astype(np.float32) / np.float32(s16)
    u = u.astype(np.float32)
    return np.clip(np.rint(u), 0, levels).astype(np.uint8)


def quantize_tile(x16: np.ndarray, is_v: bool, iters: int = ITERS, eps: float = EPS, bits: int = 0,
                  group: int = 128) -> dict:
    """Quantise one fp16 block [128 tokens, D channels] of K (is_v False) or V, codes of
    ``bits`` bits (default: 4 for K, 2 for V; levels 2^bits - 1), groups of ``group`` elements.

    Returns the stored fields: codes [128, D] (token, channel), scale and zero (fp16): for K per
    channel, shape [D] for group 128 or [2, D] for group 64 (row h: tokens 64h .. 64h+63); for V per
    token, shape [128] when one group spans the token's channels or [n, 128] (row h: channels
    gv*h .. gv*h + gv - 1, gv = min(group, D)); rho (fp32 per token) and gamma (fp32 per channel).
    """
    x = np.asarray(x16, dtype=np.float16).astype(np.float64)
    d = x.shape[1]
    r = rotate(x)
    rho, gam = normalize(r, iters, eps)
    rho32 = rho.astype(np.float32)
    gam32 = gam.astype(np.float32)
    n32 = normalized(r, rho32, gam32).astype(np.float32)
    bits = bits or (2 if is_v else 4)
    levels = (1 << bits) - 1
    codes = np.zeros((BLOCK, d), dtype=np.uint8)
    span = value_group_channels(group, d) if is_v else group  # elements along the group axis
    nseg = (d if is_v else BLOCK) // span
    scale = np.zeros((nseg, BLOCK if is_v else d), dtype=np.float16)
    zero = np.zeros_like(scale)
    for h in range(nseg):
        seg = slice(span * h, span * (h + 1))
        for g in range(scale.shape[1]):
            if is_v:
                codes[g, seg], scale[h, g], zero[h, g] = rtn_group(n32[g, seg], levels)
            else:
                codes[seg, g], scale[h, g], zero[h, g] = rtn_group(n32[seg, g], levels)
    if nseg == 1:
        scale, zero = scale[0], zero[0]
    return {"codes": codes, "scale": scale, "zero": zero, "rho": rho32, "gamma": gam32}


def group_params(fields: dict, is_v: bool):
    """Scale and zero of every element's own group, as fp16 arrays [128 tokens, D channels] (D from the
    codes or gamma when present, else 128)."""
    if "codes" in fields:
        d = fields["codes"].shape[1]
    elif "gamma" in fields:
        d = len(fields["gamma"])
    else:
        d = np.asarray(fields["scale"]).shape[-1] if not is_v else HEAD_DIM
    n = BLOCK if is_v else d  # entries per group row: tokens (values) or channels (keys)
    s = np.asarray(fields["scale"], dtype=np.float16).reshape(-1, n)
    z = np.asarray(fields["zero"], dtype=np.float16).reshape(-1, n)
    if is_v:
        idx = np.arange(d) // (d // s.shape[0])  # group of each channel
        return s[idx[None, :], np.arange(BLOCK)[:, None]], z[idx[None, :], np.arange(BLOCK)[:, None]]
    idx = np.arange(BLOCK) // (BLOCK // s.shape[0])  # group of each token
    return s[idx[:, None], np.arange(d)[None, :]], z[idx[:, None], np.arange(d)[None, :]]


def dequantize_tile(fields: dict, is_v: bool) -> np.ndarray:
    """Rebuild a block in the original basis: N^ = s*q + z, R^ = N^ * 2^(rho+gamma), X^[t] = H @ R^[t]."""
    q = fields["codes"].astype(np.float64)
    s, z = group_params(fields, is_v)
    n_hat = q * s.astype(np.float64) + z.astype(np.float64)
    rho = fields["rho"].astype(np.float64)
    gam = fields["gamma"].astype(np.float64)
    r_hat = n_hat * np.exp2(rho[:, None] + gam[None, :])
    # H is symmetric and its own inverse, so the inverse rotation is H again.
    return r_hat @ _h(r_hat.shape[1]).T


# --------------------------------------------------------------------------
# Page byte format (stage 4 output; the layout itself is a reading)
# --------------------------------------------------------------------------
def pack_k_codes(codes: np.ndarray, bits: int = 4) -> bytes:
    """K codes [token, channel], token-major.  4 bits -> 8192 bytes: byte 64*t + k = ch 2k (bits 0-3)
    | ch 2k+1 (bits 4-7).  8 bits -> 16384 bytes: byte 128*t + c."""
    c = np.asarray(codes, dtype=np.uint8)
    if bits == 8:
        return c.tobytes()
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8).tobytes()


def unpack_k_codes(buf: bytes, bits: int = 4, head_dim: int = HEAD_DIM) -> np.ndarray:
    d = head_dim
    if bits == 8:
        return np.frombuffer(bytes(buf[:BLOCK * d]), dtype=np.uint8).reshape(BLOCK, d).copy()
    b = np.frombuffer(bytes(buf[:BLOCK * d // 2]), dtype=np.uint8).reshape(BLOCK, d // 2)
    codes = np.zeros((BLOCK, d), dtype=np.uint8)
    codes[:, 0::2] = b & 0xF
    codes[:, 1::2] = b >> 4
    return codes


def pack_v_codes(codes: np.ndarray, bits: int = 2) -> bytes:
    """V codes [token, channel], channel-major.  2 bits -> 4096 bytes: byte 32*c + k holds token 4k+i at
    bits 2i..2i+1.  4 bits -> 8192 bytes: byte 64*c + k holds token 2k (bits 0-3) and 2k+1 (bits 4-7)."""
    c = np.asarray(codes, dtype=np.uint8)
    per = 8 // bits
    out = np.zeros((c.shape[1], BLOCK // per), dtype=np.uint8)
    for i in range(per):
        out |= (c[i::per, :].T << (bits * i)).astype(np.uint8)
    return out.tobytes()


def unpack_v_codes(buf: bytes, bits: int = 2, head_dim: int = HEAD_DIM) -> np.ndarray:
    per = 8 // bits
    b = np.frombuffer(bytes(buf[:BLOCK * head_dim // per]), dtype=np.uint8).reshape(head_dim, BLOCK // per)
    codes = np.zeros((BLOCK, head_dim), dtype=np.uint8)
    for i in range(per):
        codes[i::per, :] = ((b >> (bits * i)) & ((1 << bits) - 1)).T
    return codes


def encode_page(fields: dict, is_v: bool, bits: int = 0) -> bytes:
    """Page = codes | scale fp16[groups] | zero fp16[groups] | rho fp32[128 tokens] | gamma fp32[D channels],
    little endian; the group entries row-major as quantize_tile returns them (group row h, then entry)."""
    bits = bits or (2 if is_v else 4)
    codes = pack_v_codes(fields["codes"], bits) if is_v else pack_k_codes(fields["codes"], bits)
    meta = (np.asarray(fields["scale"], dtype="<f2").tobytes() + np.asarray(fields["zero"], dtype="<f2").tobytes()
            + np.asarray(fields["rho"], dtype="<f4").tobytes() + np.asarray(fields["gamma"], dtype="<f4").tobytes())
    return codes + meta


def decode_page(buf: bytes, is_v: bool, head_dim: int = HEAD_DIM) -> dict:
    buf = bytes(buf)
    d = head_dim
    bits, group = format_of_page(len(buf), is_v, d)
    ncode = BLOCK * d * bits // 8
    codes = unpack_v_codes(buf[:ncode], bits, d) if is_v else unpack_k_codes(buf[:ncode], bits, d)
    o = ncode
    n = n_groups(group, d, is_v)
    scale = np.frombuffer(buf[o:o + 2 * n], dtype="<f2").copy()
    zero = np.frombuffer(buf[o + 2 * n:o + 4 * n], dtype="<f2").copy()
    o += 4 * n
    rho = np.frombuffer(buf[o:o + 4 * BLOCK], dtype="<f4").copy()
    gam = np.frombuffer(buf[o + 4 * BLOCK:o + 4 * BLOCK + 4 * d], dtype="<f4").copy()
    per_row = BLOCK if is_v else d
    if n > per_row:
        scale, zero = scale.reshape(n // per_row, per_row), zero.reshape(n // per_row, per_row)
    return {"codes": codes, "scale": scale, "zero": zero, "rho": rho, "gamma": gam}


# --------------------------------------------------------------------------
# Whole-call drivers (the two entry points of the path)
# --------------------------------------------------------------------------
def quantize_blocks(k16: np.ndarray, v16: np.ndarray, dst_pages, k_pool: np.ndarray, v_pool: np.ndarray) -> None:
    """k16, v16: fp16 [n_blocks*128, Hkv, D]; block b of head h goes to page dst_pages[b] of each pool.

    Pools are uint8 arrays [num_pages, Hkv, page_bytes], written in place; the page sizes give the
    code widths of the format.
    """
    n_tok, hkv, d = k16.shape
    (kb, kg), (vb, vg) = format_of_page(k_pool.shape[2], False, d), format_of_page(v_pool.shape[2], True, d)
    for b in range(n_tok // BLOCK):
        p = int(dst_pages[b])
        for h in range(hkv):
            sl = slice(BLOCK * b, BLOCK * (b + 1))
            k_pool[p, h, :] = np.frombuffer(
                encode_page(quantize_tile(k16[sl, h, :], False, bits=kb, group=kg), False, kb), np.uint8)
            v_pool[p, h, :] = np.frombuffer(
                encode_page(quantize_tile(v16[sl, h, :], True, bits=vb, group=vg), True, vb), np.uint8)


def dequantize_pages(pool: np.ndarray, pages, head: int, is_v: bool, head_dim: int = HEAD_DIM) -> np.ndarray:
    """Concatenate dequantised blocks of one KV head over a page list -> [len(pages)*128, D] fp64."""
    if len(pages) == 0:
        return np.zeros((0, head_dim))
    return np.concatenate([dequantize_tile(decode_page(pool[int(p), head].tobytes(), is_v, head_dim), is_v)
                           for p in pages])


def attention(q: np.ndarray, k_hat: np.ndarray, v_hat: np.ndarray, scale: float) -> np.ndarray:
    """out = softmax(scale * K^ q) V^ for one query vector (fp64, max-subtracted)."""
    if k_hat.shape[0] == 0:
        return np.zeros(len(q))
    logits = scale * (k_hat @ np.asarray(q, dtype=np.float64))
    w = np.exp(logits - logits.max())
    return (w / w.sum()) @ v_hat


def decode(q16: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray, block_table: np.ndarray,
           seq_lens: np.ndarray, num_kv_heads: int, softmax_scale: float = 0.0, seqs=None, heads=None) -> np.ndarray:
    """Decode attention of q [B, Hq, 128] over the packed cache -> fp64 [B, Hq, 128].

    Sequence b attends to pages block_table[b, :seq_lens[b] // 128]; query head
    h reads KV head h // (Hq // Hkv).  ``seqs`` / ``heads`` restrict the work to
    a sample (other rows stay NaN).
    """
    bsz, hq, d = q16.shape
    group = hq // num_kv_heads
    scale = softmax_scale if softmax_scale > 0 else 1.0 / np.sqrt(d)
    out = np.full((bsz, hq, d), np.nan)
    for b in (range(bsz) if seqs is None else seqs):
        pages = block_table[b, : int(seq_lens[b]) // BLOCK]
        hs = range(hq) if heads is None else heads
        cache = {}
        for h in hs:
            g = h // group
            if g not in cache:
                cache[g] = (dequantize_pages(k_pool, pages, g, False, d), dequantize_pages(v_pool, pages, g, True, d))
            out[b, h] = attention(np.asarray(q16[b, h], dtype=np.float64), cache[g][0], cache[g][1], scale)
    return out


# --------------------------------------------------------------------------
# The uncompressed baseline: decode over fp16 pages (blog post, "KVarN (Varyans
# Normalize Edilmiş KV-Cache) Nedir?": the packed cache is compared against FP16
# serving; paged storage and grouped heads as in the "KV Cache" glossary page).
# --------------------------------------------------------------------------
def fp16_pages(cache16: np.ndarray, pages, head: int) -> np.ndarray:
    """Concatenate the fp16 token rows of one KV head over a page list -> [len(pages)*128, 128] fp64.

    cache16: fp16 [num_pages, Hkv, 128 tokens, 128 channels].
    """
    if len(pages) == 0:
        return np.zeros((0, cache16.shape[-1]))
    return np.concatenate([np.asarray(cache16[int(p), head], dtype=np.float64) for p in pages])


def fp16_decode(q16: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, block_table: np.ndarray,
                seq_lens: np.ndarray, num_kv_heads: int, softmax_scale: float = 0.0, seqs=None,
                heads=None) -> np.ndarray:
    """Decode attention of q [B, Hq, 128] over fp16 pages -> fp64 [B, Hq, 128] (no rotation, no quantisation).

    Same addressing and scale as ``decode``; ``seqs`` / ``heads`` restrict the work to a sample.
    """
    bsz, hq, d = q16.shape
    group = hq // num_kv_heads
    scale = softmax_scale if softmax_scale > 0 else 1.0 / np.sqrt(d)
    out = np.full((bsz, hq, d), np.nan)
    for b in (range(bsz) if seqs is None else seqs):
        pages = block_table[b, : int(seq_lens[b]) // BLOCK]
        for h in (range(hq) if heads is None else heads):
            g = h // group
            out[b, h] = attention(np.asarray(q16[b, h], dtype=np.float64), fp16_pages(k_cache, pages, g),
                                  fp16_pages(v_cache, pages, g), scale)
    return out


# --------------------------------------------------------------------------
# Packed pages plus an fp16 tail: blocks are quantised whole (blog post, "KVarN
# Nasıl Çalışır?": the cache is quantised in fixed-size token blocks), so the
# tokens past the last full block are attended in fp16 until their block fills.
# --------------------------------------------------------------------------
def decode_tail(q16: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray, block_table: np.ndarray,
                seq_lens: np.ndarray, k_tail: np.ndarray, v_tail: np.ndarray, num_kv_heads: int,
                softmax_scale: float = 0.0, seqs=None, heads=None) -> np.ndarray:
    """Decode of q [B, Hq, 128] over the first seq_lens[b] // 128 packed blocks followed by the
    seq_lens[b] % 128 tail tokens k_tail[b, :t, g], v_tail[b, :t, g] (fp16 [B, 128, Hkv, 128]) -> fp64.
    """
    bsz, hq, d = q16.shape
    group = hq // num_kv_heads
    scale = softmax_scale if softmax_scale > 0 else 1.0 / np.sqrt(d)
    out = np.full((bsz, hq, d), np.nan)
    for b in (range(bsz) if seqs is None else seqs):
        nblk, ntail = int(seq_lens[b]) // BLOCK, int(seq_lens[b]) % BLOCK
        pages = block_table[b, :nblk]
        cache = {}
        for h in (range(hq) if heads is None else heads):
            g = h // group
            if g not in cache:
                cache[g] = (np.concatenate([dequantize_pages(k_pool, pages, g, False, d),
                                            np.asarray(k_tail[b, :ntail, g], dtype=np.float64)]),
                            np.concatenate([dequantize_pages(v_pool, pages, g, True, d),
                                            np.asarray(v_tail[b, :ntail, g], dtype=np.float64)]))
            out[b, h] = attention(np.asarray(q16[b, h], dtype=np.float64), cache[g][0], cache[g][1], scale)
    return out


# --------------------------------------------------------------------------
# Chunked prefill over the packed cache.  A chunk of new tokens attends to the
# packed blocks before it and, causally, to its own rows, which are still fp16:
# blocks are quantised whole once they fill (blog post, "KVarN Nasıl Çalışır?"),
# and the post's long-context serving reads the packed cache for every earlier
# token ("KVarN (Varyans Normalize Edilmiş KV-Cache) Nedir?").
# --------------------------------------------------------------------------
def prefill(q16: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray, block_table: np.ndarray,
            prefix_lens: np.ndarray, k_new: np.ndarray, v_new: np.ndarray, new_lens: np.ndarray,
            q_lens: np.ndarray, num_kv_heads: int, softmax_scale: float = 0.0, seqs=None, rows=None,
            heads=None) -> np.ndarray:
    """Chunked-prefill attention -> fp64 [B, max_q, Hq, 128].

    q16 fp16 [B, max_q, Hq, 128]; k_new, v_new fp16 [B, max_new, Hkv, 128].  Sequence b holds
    prefix_lens[b] // 128 packed blocks (pages block_table[b, ...]) followed by new_lens[b] fp16
    rows.  Its queries are the last q_lens[b] of those rows: query i sits at fp16 row
    new_lens[b] - q_lens[b] + i and attends to every packed token and to fp16 rows 0 .. that row.
    Query rows at or past q_lens[b] are zero.  ``seqs`` / ``rows`` / ``heads`` restrict the work
    to a sample (the rest stays NaN).
    """
    bsz, max_q, hq, d = q16.shape
    group = hq // num_kv_heads
    scale = softmax_scale if softmax_scale > 0 else 1.0 / np.sqrt(d)
    out = np.full((bsz, max_q, hq, d), np.nan)
    for b in (range(bsz) if seqs is None else seqs):
        pages = block_table[b, : int(prefix_lens[b]) // BLOCK]
        n_new, n_q = int(new_lens[b]), int(q_lens[b])
        n_pre = len(pages) * BLOCK
        cache = {}
        for i in (range(max_q) if rows is None else rows):
            for h in (range(hq) if heads is None else heads):
                if i >= n_q:
                    out[b, i, h] = 0.0
                    continue
                g = h // group
                if g not in cache:
                    cache[g] = (np.concatenate([dequantize_pages(k_pool, pages, g, False, d),
                                                np.asarray(k_new[b, :n_new, g], dtype=np.float64)]),
                                np.concatenate([dequantize_pages(v_pool, pages, g, True, d),
                                                np.asarray(v_new[b, :n_new, g], dtype=np.float64)]))
                last = n_pre + (n_new - n_q) + i  # the query's own row
                out[b, i, h] = attention(np.asarray(q16[b, i, h], dtype=np.float64), cache[g][0][: last + 1],
                                         cache[g][1][: last + 1], scale)
    return out
