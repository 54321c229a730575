"""Seeded synthetic inputs for the KVarN quantize / decode path.

This module only draws random data and lays out page tables.  It holds none of
the method's arithmetic (no rotation, normalisation, rounding or packing), so
both the HIP path and the CPU oracle can take their inputs from it.

Distributions (the workloads the method targets are long-context decode over a
paged, GQA-shaped KV cache; see the KVarN blog post, section "KVarN (Varyans
Normalize Edilmiş KV-Cache) Nedir?", and the "KV Cache" glossary page, sections
"Boyutu ve Yönetimi" and "Türleri"):

* K ~ N(0, 1) per element; for every (layer, KV head) a seeded set of
  ``n_outlier`` channels is multiplied by ``outlier_mult`` for every token.
* V ~ N(0, 1) times a per-(token, KV head) scale drawn from LogNormal(0, 0.5).
* q ~ N(0, 1).
* Everything is rounded to fp16 (round to nearest even) before use.

Token layout of one layer's K or V: ``[n_blocks * 128, Hkv, 128]`` fp16, the
128-token blocks of sequence b stored consecutively.  Page ids: identity, or a
seeded random permutation of all pages for the paged workload.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import torch

BLOCK_TOKENS = 128
HEAD_DIM = 128
BASE_SEED = 0x4B5641524E00  # "KVARN\0"


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    hq: int
    hkv: int
    layers: int = 1
    seq_len: int = 0                 # fixed length (tokens, multiple of 128)
    seq_len_range: Optional[tuple] = None  # (lo, hi) for mixed lengths
    n_outlier: int = 4
    outlier_mult: float = 20.0
    paged: bool = False              # random physical page permutation
    append_blocks: int = 0           # blocks appended per sequence before decode
    index: int = 0
    head_dim: int = HEAD_DIM

    @property
    def gqa(self) -> int:
        return self.hq // self.hkv


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("tiny_1x1024", batch=1, seq_len=1024, hq=32, hkv=8, index=0),
        Workload("llama3_8b_layer_16x8192", batch=16, seq_len=8192, hq=32, hkv=8, index=1),
        Workload("qwen25_1p5b_28layer_64x4096", batch=64, seq_len=4096, hq=12, hkv=2, layers=28, index=2),
        Workload("long_context_1x131072", batch=1, seq_len=131072, hq=32, hkv=8,
                 n_outlier=8, outlier_mult=50.0, index=3),
        Workload("paged_mixed_128xU1k_32k", batch=128, seq_len_range=(1024, 32768), hq=64, hkv=8,
                 paged=True, append_blocks=1, index=4),
    ]
}


# Heads of 64 and 256 channels (the other head sizes of the format), one layer each at full size:
# a Llama-3.2-1B-like layer (32 query / 8 KV heads of 64 channels) and a Gemma-2-9B-like layer
# (16 query / 8 KV heads of 256 channels), 16 sequences of 8192 tokens.
HEAD_DIM_WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("tiny_d64_1x1024", batch=1, seq_len=1024, hq=32, hkv=8, index=20, head_dim=64),
        Workload("tiny_d256_1x1024", batch=1, seq_len=1024, hq=16, hkv=8, index=21, head_dim=256),
        Workload("llama32_1b_layer_d64_16x8192", batch=16, seq_len=8192, hq=32, hkv=8, index=22, head_dim=64),
        Workload("gemma2_9b_layer_d256_16x8192", batch=16, seq_len=8192, hq=16, hkv=8, index=23, head_dim=256),
    ]
}


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed & 0x7FFFFFFFFFFFFFFF)
    return g


def stream_seed(w: Workload, stream: int, layer: int = 0) -> int:
    """Seed of one random stream: 1 K, 2 V, 3 q, 4 outlier channels, 5 lengths, 6 pages, 7/8 appended K/V."""
    return BASE_SEED + w.index * 0x1000003 + stream * 0x10001 + layer * 7919


def seq_lens_for(w: Workload) -> List[int]:
    """Prefix lengths (tokens) of each sequence; multiples of 128."""
    if w.seq_len_range is None:
        return [w.seq_len] * w.batch
    lo, hi = w.seq_len_range
    g = _gen("cpu", stream_seed(w, 5))
    u = torch.rand(w.batch, generator=g, dtype=torch.float64) * (hi - lo) + lo
    return [int(BLOCK_TOKENS * max(1, round(float(x) / BLOCK_TOKENS))) for x in u]


def outlier_channels(w: Workload, layer: int) -> torch.Tensor:
    """[Hkv, n_outlier] distinct channel ids per KV head (seeded shuffle)."""
    g = _gen("cpu", stream_seed(w, 4, layer))
    rows = [torch.randperm(getattr(w, "head_dim", HEAD_DIM), generator=g)[: w.n_outlier] for _ in range(w.hkv)]
    return torch.stack(rows) if rows else torch.zeros(0, w.n_outlier, dtype=torch.long)


def make_kv(n_tokens: int, hkv: int, *, n_outlier: int, outlier_mult: float, outliers: torch.Tensor,
            seed_k: int, seed_v: int, device, head_dim: int = HEAD_DIM) -> tuple:
    """fp16 K, V of shape [n_tokens, hkv, head_dim] with the outlier / log-normal recipe above."""
    gk = _gen(device, seed_k)
    k = torch.randn(n_tokens, hkv, head_dim, generator=gk, device=device, dtype=torch.float32)
    if n_outlier > 0:
        mult = torch.ones(hkv, head_dim, device=device, dtype=torch.float32)
        for h in range(hkv):
            mult[h, outliers[h].to(device)] = outlier_mult
        k.mul_(mult)
    k16 = k.to(torch.float16)
    del k
    gv = _gen(device, seed_v)
    v = torch.randn(n_tokens, hkv, head_dim, generator=gv, device=device, dtype=torch.float32)
    scale = torch.exp(0.5 * torch.randn(n_tokens, hkv, 1, generator=gv, device=device, dtype=torch.float32))
    v.mul_(scale)
    v16 = v.to(torch.float16)
    return k16, v16


def layer_kv(w: Workload, layer: int, n_tokens: int, device, append: bool = False) -> tuple:
    """K, V for ``n_tokens`` tokens of one layer (``append`` selects the appended-token streams)."""
    sk, sv = (7, 8) if append else (1, 2)
    return make_kv(n_tokens, w.hkv, n_outlier=w.n_outlier, outlier_mult=w.outlier_mult,
                   outliers=outlier_channels(w, layer),
                   seed_k=stream_seed(w, sk, layer), seed_v=stream_seed(w, sv, layer), device=device,
                   head_dim=w.head_dim)


def make_q(w: Workload, layer: int, device) -> torch.Tensor:
    g = _gen(device, stream_seed(w, 3, layer))
    return torch.randn(w.batch, w.hq, w.head_dim, generator=g, device=device, dtype=torch.float32).to(torch.float16)


@dataclasses.dataclass
class PageMap:
    """Logical blocks -> physical pages for one layer.

    ``prefix_pages``: int32 [n_prefix_blocks] page of every prefix block (sequence-major order).
    ``append_pages``: int32 [batch * append_blocks] page of every appended block.
    ``block_table``: int32 [batch, max_blocks]; unused slots hold -1.
    ``seq_lens``:    int32 [batch] tokens attended by decode (prefix + appended).
    """
    num_pages: int
    prefix_pages: torch.Tensor
    append_pages: torch.Tensor
    block_table: torch.Tensor
    seq_lens: torch.Tensor
    prefix_lens: List[int]


def make_page_map(w: Workload) -> PageMap:
    prefix = seq_lens_for(w)
    nblk = [p // BLOCK_TOKENS for p in prefix]
    per_seq = [n + w.append_blocks for n in nblk]
    total = sum(per_seq)
    if w.paged:
        perm = torch.randperm(total, generator=_gen("cpu", stream_seed(w, 6))).to(torch.int32)
    else:
        perm = torch.arange(total, dtype=torch.int32)
    max_blocks = max(per_seq)
    table = torch.full((w.batch, max_blocks), -1, dtype=torch.int32)
    prefix_pages, append_pages = [], []
    off = 0
    for b in range(w.batch):
        pages = perm[off:off + per_seq[b]]
        table[b, : per_seq[b]] = pages
        prefix_pages.append(pages[: nblk[b]])
        append_pages.append(pages[nblk[b]:])
        off += per_seq[b]
    seq_lens = torch.tensor([n * BLOCK_TOKENS for n in per_seq], dtype=torch.int32)
    return PageMap(total, torch.cat(prefix_pages), torch.cat(append_pages) if append_pages else
                   torch.zeros(0, dtype=torch.int32), table, seq_lens, prefix)


def total_prefix_blocks(w: Workload) -> int:
    return sum(p // BLOCK_TOKENS for p in seq_lens_for(w))


def fp16_pages(x: torch.Tensor, dst_pages: torch.Tensor, num_pages: int,
               pool: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Lay token-major fp16 K or V ``[n_blocks*128, Hkv, 128]`` out as uncompressed pages.

    Block b goes to page ``dst_pages[b]`` of a pool ``[num_pages, Hkv, 128 tokens, 128 channels]``
    (the layout of the fp16 baseline decode); pages not written stay zero.  A pure copy.
    """
    n_blocks = x.shape[0] // BLOCK_TOKENS
    hkv = x.shape[1]
    if pool is None:
        pool = torch.zeros((num_pages, hkv, BLOCK_TOKENS, HEAD_DIM), dtype=torch.float16, device=x.device)
    blocks = x[: n_blocks * BLOCK_TOKENS].view(n_blocks, BLOCK_TOKENS, hkv, HEAD_DIM).permute(0, 2, 1, 3)
    pool[dst_pages.to(device=x.device, dtype=torch.long)] = blocks.to(torch.float16)
    return pool


# --------------------------------------------------------------------------
# Chunked prefill: every sequence holds ``prefix`` packed tokens, then a chunk of
# ``chunk`` new fp16 rows, all of which are queries (causal within the chunk).
# The chunk's rows use the same outlier channels as the prefix (same layer).
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class PrefillWorkload:
    name: str
    batch: int
    hq: int
    hkv: int
    prefix: int          # packed tokens per sequence (multiple of 128)
    chunk: int           # new fp16 rows per sequence; every one is a query
    n_outlier: int = 4
    outlier_mult: float = 20.0
    index: int = 0

    @property
    def gqa(self) -> int:
        return self.hq // self.hkv


PREFILL_WORKLOADS: Dict[str, PrefillWorkload] = {
    w.name: w
    for w in [
        PrefillWorkload("prefill_tiny_2x256p200", batch=2, hq=8, hkv=2, prefix=256, chunk=200, index=10),
        PrefillWorkload("prefill_llama3_8b_16x7680p512", batch=16, hq=32, hkv=8, prefix=7680, chunk=512, index=11),
    ]
}


@dataclasses.dataclass
class PrefillInputs:
    """Inputs of one chunked-prefill step (device tensors unless noted).

    ``k_prefix``/``v_prefix``: fp16 [batch*prefix, Hkv, 128], sequence-major (quantise input);
    ``pages``: int32 [batch*prefix/128] page of every prefix block (a seeded permutation of the
    pages); ``block_table``: int32
    [batch, prefix/128 + chunk/128 + 1] (-1 past the prefix); ``prefix_lens``, ``new_lens``,
    ``q_lens``: int32 [batch]; ``k_new``/``v_new``: fp16 [batch, chunk, Hkv, 128];
    ``q``: fp16 [batch, chunk, Hq, 128].
    """
    k_prefix: torch.Tensor
    v_prefix: torch.Tensor
    pages: torch.Tensor
    block_table: torch.Tensor
    prefix_lens: torch.Tensor
    k_new: torch.Tensor
    v_new: torch.Tensor
    new_lens: torch.Tensor
    q_lens: torch.Tensor
    q: torch.Tensor
    num_pages: int


def prefill_inputs(w: PrefillWorkload, device) -> PrefillInputs:
    nblk = w.prefix // BLOCK_TOKENS
    outl = outlier_channels(w, 0)
    kp, vp = make_kv(w.batch * w.prefix, w.hkv, n_outlier=w.n_outlier, outlier_mult=w.outlier_mult,
                     outliers=outl, seed_k=stream_seed(w, 1), seed_v=stream_seed(w, 2), device=device)
    kn, vn = make_kv(w.batch * w.chunk, w.hkv, n_outlier=w.n_outlier, outlier_mult=w.outlier_mult,
                     outliers=outl, seed_k=stream_seed(w, 7), seed_v=stream_seed(w, 8), device=device)
    g = _gen(device, stream_seed(w, 3))
    q = torch.randn(w.batch, w.chunk, w.hq, HEAD_DIM, generator=g, device=device, dtype=torch.float32)
    total = max(w.batch * nblk, 1)
    # physical pages in a seeded random permutation, as a paged cache holds them
    pages = torch.randperm(w.batch * nblk, generator=_gen("cpu", stream_seed(w, 6))).to(torch.int32)
    table = torch.full((w.batch, nblk + (w.chunk + BLOCK_TOKENS - 1) // BLOCK_TOKENS + 1), -1, dtype=torch.int32)
    for b in range(w.batch):
        table[b, :nblk] = pages[b * nblk:(b + 1) * nblk]
    lens = lambda v: torch.full((w.batch,), v, dtype=torch.int32, device=device)
    return PrefillInputs(kp, vp, pages.to(device), table.to(device), lens(w.prefix),
                         kn.view(w.batch, w.chunk, w.hkv, HEAD_DIM), vn.view(w.batch, w.chunk, w.hkv, HEAD_DIM),
                         lens(w.chunk), lens(w.chunk), q.to(torch.float16), total)
