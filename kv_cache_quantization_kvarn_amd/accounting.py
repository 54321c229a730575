"""Byte and token accounting for the benchmark (host-side arithmetic only).

KV bytes of an uncompressed cache follow the size formula on the "KV Cache"
glossary page, section "Boyutu ve Yönetimi": 2 x layers x KV heads x head_dim x
tokens x bytes per element.  Packed page sizes come from the library
(``kvarn_page_bytes``) so that this module never restates the format.
"""
from __future__ import annotations

BLOCK_TOKENS = 128
HEAD_DIM = 128
FP16_BYTES = 2
HBM_PEAK_GBPS = 8000.0  # MI355X published HBM3E bandwidth, GB/s


def fp16_kv_bytes(layers: int, kv_heads: int, tokens: int, head_dim: int = HEAD_DIM) -> int:
    """Uncompressed K+V bytes: 2 x layers x heads x head_dim x tokens x 2 bytes."""
    return 2 * layers * kv_heads * head_dim * tokens * FP16_BYTES


def packed_bytes_per_block_head(k_page: int, v_page: int) -> int:
    """Packed K+V bytes of one 128-token block of one KV head."""
    return k_page + v_page


def capacity_ratio(k_page: int, v_page: int) -> float:
    """FP16 bytes / packed bytes for one 128-token block of one KV head."""
    return fp16_kv_bytes(1, 1, BLOCK_TOKENS) / packed_bytes_per_block_head(k_page, v_page)


def quantize_bytes(n_blocks: int, kv_heads: int, k_page: int, v_page: int, head_dim: int = HEAD_DIM) -> int:
    """Algorithmic HBM bytes of one quantize call: fp16 K and V in, packed pages out."""
    return n_blocks * kv_heads * (fp16_kv_bytes(1, 1, BLOCK_TOKENS, head_dim) + k_page + v_page)


def decode_bytes(total_blocks_attended: int, kv_heads: int, batch: int, q_heads: int, k_page: int, v_page: int,
                 max_blocks_per_seq: int = 0, head_dim: int = HEAD_DIM) -> int:
    """Algorithmic HBM bytes of one decode step.

    Packed pages of every attended (block, KV head), the fp16 query (2 B per
    channel and query head), the fp32 output (4 B per channel and query head),
    the block-table entries read (4 B per attended block) and the sequence lengths.
    """
    return (total_blocks_attended * kv_heads * (k_page + v_page)
            + batch * q_heads * (head_dim * 2 + head_dim * 4)
            + total_blocks_attended * 4 + batch * 4)


def tail_decode_bytes(total_blocks_attended: int, kv_heads: int, batch: int, q_heads: int, k_page: int, v_page: int,
                      total_tail_tokens: int) -> int:
    """Algorithmic HBM bytes of one decode step with fp16 tails: the packed decode's bytes plus one
    fp16 K row and one fp16 V row (256 B each) per tail token and KV head."""
    return (decode_bytes(total_blocks_attended, kv_heads, batch, q_heads, k_page, v_page)
            + total_tail_tokens * kv_heads * 2 * HEAD_DIM * 2)


MFMA_FP16_PEAK_TFLOPS = 2500.0  # MI355X published dense fp16 matrix rate, TFLOP/s


def prefill_pairs(prefix_lens, new_lens, q_lens, q_heads: int) -> int:
    """Attended (query head, key) pairs of one chunked-prefill call: query i of sequence b sees
    prefix + (new - q) + i + 1 keys."""
    total = 0
    for p, n, q in zip(prefix_lens, new_lens, q_lens):
        p, n, q = int(p), int(n), int(q)
        total += q * (p + n - q) + q * (q + 1) // 2
    return total * q_heads


def prefill_flops(pairs: int) -> int:
    """Algorithmic flops of attention: 2 x head_dim for the score and 2 x head_dim for the value
    product of every attended pair."""
    return 4 * HEAD_DIM * pairs


def prefill_bytes(prefix_blocks_total: int, kv_heads: int, k_page: int, v_page: int, new_rows_total: int,
                  q_rows_total: int, q_heads: int) -> int:
    """Algorithmic HBM bytes of one prefill call: packed pages and fp16 rows read once, fp16 queries
    in, fp32 output out."""
    return (prefix_blocks_total * kv_heads * (k_page + v_page) + new_rows_total * kv_heads * HEAD_DIM * 2 * FP16_BYTES
            + q_rows_total * q_heads * HEAD_DIM * (FP16_BYTES + 4))
