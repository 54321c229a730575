/*
 * libkvarn: KVarN KV-cache block quantisation and decode attention over the
 * packed, paged cache, for AMD Instinct MI355X (gfx950).
 *
 * Method: the KVarN blog post ("KVarN: Huawei'den KV-Cache Kuantizasyonu için
 * Yerel vLLM Backend'i"), section "KVarN Nasıl Çalışır?": the KV cache is
 * quantised in fixed-size token blocks, each block passing through a Hadamard
 * rotation along channels, a log-space row/column variance normalisation and
 * low-bit asymmetric round-to-nearest (4-bit keys, 2-bit values); section
 * "Pratik Çıkarımlar" names the format "kvarn_k4v2_g128".  Paged storage
 * with a block table and GQA heads: the "KV Cache" glossary page, sections
 * "Boyutu ve Yönetimi" and "Türleri".
 *
 * Conventions for every call:
 *   - All tensor arguments are device pointers owned by the caller; the library
 *     never allocates, frees or synchronises (except kvarn_read_flags, and
 *     kvarn_quantize_blocks while debug checks are on: kvarn_set_debug_checks).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     runs asynchronously.  Calls are re-entrant; two calls that write the
 *     same pages or the same workspace must not overlap.
 *   - The return value reports host-side validation and launch errors only.
 *     Problems that only the device can see (a page id outside [0, num_pages),
 *     a bad sequence length) set bits in the optional `dev_flags` word (device
 *     memory, OR-ed atomically) and the offending unit of work is skipped.
 *   - Shapes: tokens of a 128-token block are consecutive rows; head_dim is
 *     cfg->head_dim (64, 128 or 256; 128 only for the decode with an fp16
 *     tail, the fp16 baseline and prefill).
 *   - No exceptions cross this boundary; kvarn_last_error() describes the last
 *     failure of the calling thread.
 */
#ifndef KVARN_H
#define KVARN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVARN_OK = 0,
  KVARN_ERR_NULL = -1,        /* a required pointer is NULL */
  KVARN_ERR_SHAPE = -2,       /* a size is negative, zero where it must not be, or inconsistent */
  KVARN_ERR_UNSUPPORTED = -3, /* a format other than kvarn_k{4,8}v{2,4}_g{128,64} / head_dim 64, 128, 256 / block 128 */
  KVARN_ERR_WORKSPACE = -4,   /* decode workspace missing or too small */
  KVARN_ERR_LAUNCH = -5       /* the HIP runtime rejected a launch */
} kvarn_status;

/* Device-side flag bits written to *dev_flags. */
#define KVARN_FLAG_BAD_PAGE 1u    /* a page id outside [0, num_pages): that block is skipped */
#define KVARN_FLAG_BAD_SEQLEN 2u  /* seq_len < 0, not a multiple of 128, or above max_blocks*128: sequence output is 0 */

/* Format parameters.  Supported: head_dim 64, 128 or 256, block_tokens 128, k_bits 4 or
 * 8, v_bits 2 or 4, group_size 128 or 64, norm_iters 4, eps 1e-6.  The post
 * names kvarn_k4v2_g128; the wider codes keep every step of the method and
 * change the number of levels (2^bits - 1) and the packing only.  Group size 64
 * splits every group into two halves of 64 consecutive elements (a key group:
 * one channel over tokens 64h .. 64h+63; a value group: one token over channels
 * 64h .. 64h+63), each with its own scale and zero.  Every entry point takes
 * every format; the kernels are instantiated per code widths and group size. */
typedef struct {
  int32_t head_dim;
  int32_t block_tokens;
  int32_t k_bits;
  int32_t v_bits;
  int32_t group_size;
  int32_t norm_iters;
  float eps;
} kvarn_config;

/* Fill *out from a cache dtype name of the form "kvarn_k<K>v<V>_g<G>"
 * (blog post, section "Pratik Çıkarımlar").  Parses any such name; names other
 * than kvarn_k{4,8}v{2,4}_g{128,64} parse but return KVARN_ERR_UNSUPPORTED. */
kvarn_status kvarn_config_parse(const char* name, kvarn_config* out);

/* Bytes of one page (one 128-token block of one KV head): C + M with C =
 * 128*128*bits/8 code bytes and M = 1536 metadata bytes for group size 128,
 * 2048 for group size 64.  Group size 128: K (is_v = 0) 9728 for 4 bits, 17920
 * for 8 bits; V (is_v = 1) 5632 for 2 bits, 9728 for 4 bits.  Group size 64:
 * 512 more each.  0 for an unsupported config.
 *
 * K page: [0, C) codes, token-major: 4 bits: byte 64*t + k holds channel 2k in
 *         bits 0-3 and channel 2k+1 in bits 4-7 of token t; 8 bits: byte 128*t + c;
 *         then scale fp16[128 channels], zero fp16[128 channels], rho fp32[128
 *         tokens], gamma fp32[128 channels] at C, C + 256, C + 512, C + 1024.
 * V page: [0, C) codes, channel-major: 2 bits: byte 32*c + k holds token 4k+i
 *         in bits 2i..2i+1 of channel c; 4 bits: byte 64*c + k holds token 2k in
 *         bits 0-3 and token 2k+1 in bits 4-7;
 *         then scale fp16[128 tokens], zero fp16[128 tokens], rho fp32[128
 *         tokens], gamma fp32[128 channels] at the same offsets from C.
 * Group size 64: scale fp16[2][128] and zero fp16[2][128] (entry 128*h + j: the
 *         group of channel j over tokens 64h .. 64h+63 for K, of token j over
 *         channels 64h .. 64h+63 for V), rho, gamma at C, C + 512, C + 1024,
 *         C + 1536.
 * All little endian.  Dequantisation: x^[t] = H (N^ * 2^(rho[t] + gamma)), with
 * N^ = scale * code + zero and H the orthonormal Sylvester Hadamard matrix. */
size_t kvarn_page_bytes(const kvarn_config* cfg, int is_v);

/* Quantise n_blocks 128-token blocks of K and V (blog post, "KVarN Nasıl
 * Çalışır?": rotate, normalise, round to nearest, pack) into pages of the
 * config's format.
 *   k, v       fp16 [n_blocks*128, num_kv_heads, 128], contiguous; block b is
 *              rows 128b .. 128b+127.
 *   dst_pages  int32 [n_blocks] (device): page receiving block b (all heads).
 *              Entries must be distinct.  An entry outside [0, num_pages)
 *              sets KVARN_FLAG_BAD_PAGE and that block is not written.
 *   k_pool     bytes [num_pages, num_kv_heads, kvarn_page_bytes(cfg, 0)];
 *              v_pool bytes [num_pages, num_kv_heads, kvarn_page_bytes(cfg, 1)];
 *              written in place.  The pools must not overlap k or v.
 *   n_blocks == 0 is a no-op returning KVARN_OK. */
kvarn_status kvarn_quantize_blocks(const kvarn_config* cfg, const void* k, const void* v, int32_t n_blocks,
                                   int32_t num_kv_heads, const int32_t* dst_pages, void* k_pool, void* v_pool,
                                   int32_t num_pages, uint32_t* dev_flags, void* stream);

/* Rebuild fp32 K^ and V^ (original basis) from pages: block b of head h is read
 * from page pages[b].  k_out, v_out: fp32 [n_blocks*128, num_kv_heads, 128].
 * Either output may be NULL to skip it.  A test and inspection export; the
 * decode path never materialises K^ or V^. */
kvarn_status kvarn_dequantize_blocks(const kvarn_config* cfg, const void* k_pool, const void* v_pool,
                                     int32_t num_pages, const int32_t* pages, int32_t n_blocks,
                                     int32_t num_kv_heads, float* k_out, float* v_out, uint32_t* dev_flags,
                                     void* stream);

/* Workspace bytes kvarn_decode_attention needs for these sizes (split
 * partials and per-(sequence, KV head) arrival counters).  The workspace
 * must be zero-filled before its first use; every call leaves the counter
 * region zero again, so later calls with the same or smaller sizes need no
 * clearing.  The split plan spreads over the compute units of the current
 * device, so the size is that device's: query it with the device current that
 * will run the decode.  Returns 0 for an unsupported config, batch <= 0, a
 * non-positive head count, max_blocks_per_seq < 0, batch or num_kv_heads above
 * 65535, or max_blocks_per_seq * 128 above 2^31 - 1. */
size_t kvarn_decode_workspace_bytes(const kvarn_config* cfg, int32_t batch, int32_t num_q_heads,
                                    int32_t num_kv_heads, int32_t max_blocks_per_seq);

/* One decode step: for every sequence b and query head h, attention of q[b, h]
 * over the packed K/V pages of KV head h / (num_q_heads / num_kv_heads), pages
 * block_table[b, 0 .. seq_lens[b]/128).  The query is rotated by the same
 * Hadamard matrix, so scores equal those of the dequantised cache ("KVarN Nasıl
 * Çalışır?": the rotation is orthonormal and keeps attention scores).
 *   q            fp16 [batch, num_q_heads, 128], 16-byte aligned
 *   block_table  int32 [batch, max_blocks_per_seq] (device)
 *   seq_lens     int32 [batch] (device), multiples of 128; 0 gives a zero row
 *   softmax_scale  <= 0 selects 1/sqrt(128)
 *   out          fp32 [batch, num_q_heads, 128], 16-byte aligned
 *   workspace    device bytes, at least kvarn_decode_workspace_bytes(...) */
kvarn_status kvarn_decode_attention(const kvarn_config* cfg, const void* q, const void* k_pool,
                                    const void* v_pool, int32_t num_pages, const int32_t* block_table,
                                    int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t batch,
                                    int32_t num_q_heads, int32_t num_kv_heads, float softmax_scale, float* out,
                                    void* workspace, size_t workspace_bytes, uint32_t* dev_flags, void* stream);

/* kvarn_decode_attention without a workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation).  The split
 * partials and arrival counters live in a fixed scratch array inside the library: 64 MiB per GPU,
 * held from the first call on that GPU until the process ends (1 MiB of counters, 63 MiB of
 * partials).  The call allocates nothing and frees nothing.  Same arguments, plan, results (bit for
 * bit), error model and output as kvarn_decode_attention otherwise.
 *   Limits: batch * num_kv_heads <= 262144, and the partials of the call's split plan,
 *   batch * num_kv_heads * splits * 8 * 130 * 4 bytes, at most 63 MiB (every configuration whose
 *   kvarn_decode_workspace_bytes is at most 64 MiB fits); beyond them the call returns
 *   KVARN_ERR_WORKSPACE and launches nothing.
 *   The first call on a GPU clears the counters with a small kernel on `stream`; every call leaves
 *   them at zero again.  All calls on one GPU share the array: calls that overlap in time on one GPU
 *   (on different streams or from different threads) race and must not be issued. */
kvarn_status kvarn_decode_attention_noalloc(const kvarn_config* cfg, const void* q, const void* k_pool,
                                            const void* v_pool, int32_t num_pages, const int32_t* block_table,
                                            int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t batch,
                                            int32_t num_q_heads, int32_t num_kv_heads, float softmax_scale,
                                            float* out, uint32_t* dev_flags, void* stream);

/* Decode over the packed pages plus an fp16 tail: the tokens past the last
 * full block stay uncompressed until their block fills (blocks are quantised
 * whole, "KVarN Nasıl Çalışır?").  Same arguments, plan, workspace
 * (kvarn_decode_workspace_bytes), error model and output as
 * kvarn_decode_attention, except:
 *   seq_lens   any length in [0, 128*max_blocks_per_seq + 127]: the first
 *              seq_lens[b]/128 blocks are pages block_table[b, ...], the
 *              remaining seq_lens[b] % 128 tokens are rows 0 .. of the tail
 *   k_tail, v_tail  fp16 [batch, 128 tokens, num_kv_heads, 128], 16-byte
 *              aligned; rows at or past seq_lens[b] % 128 are never read
 * The tail of sequence b has the layout of kvarn_quantize_blocks' input for
 * one block, so a full tail is packed by kvarn_quantize_blocks(k_tail + b's
 * offset, v_tail + b's offset, 1, ...) into the page that then joins the
 * block table.  One launch: the tail is one more split of the same merge. */
kvarn_status kvarn_decode_attention_tail(const kvarn_config* cfg, const void* q, const void* k_pool,
                                         const void* v_pool, int32_t num_pages, const int32_t* block_table,
                                         int32_t max_blocks_per_seq, const int32_t* seq_lens, const void* k_tail,
                                         const void* v_tail, int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                         float softmax_scale, float* out, void* workspace, size_t workspace_bytes,
                                         uint32_t* dev_flags, void* stream);

/* The uncompressed baseline on the same harness: decode attention over fp16
 * K/V pages, for comparison with the packed cache ("KVarN (Varyans Normalize
 * Edilmiş KV-Cache) Nedir?": the packed cache against FP16 serving).  Same
 * arguments, plan, workspace (kvarn_decode_workspace_bytes), error model and
 * output as kvarn_decode_attention, except the pools:
 *   k_cache, v_cache  fp16 [num_pages, num_kv_heads, 128 tokens, 128 channels],
 *                     16-byte aligned; page p of KV head g holds the 128 token
 *                     rows of one block, unrotated and unquantised
 * No rotation is involved: out[b, h] = softmax(scale * K q) V over the pages.
 * A page id outside [0, num_pages) sets flag 1 and the page is skipped. */
size_t kvarn_fp16_page_bytes(const kvarn_config* cfg); /* 32768 per (page, KV head), K or V; 0 for an unsupported config */
kvarn_status kvarn_fp16_decode_attention(const kvarn_config* cfg, const void* q, const void* k_cache,
                                         const void* v_cache, int32_t num_pages, const int32_t* block_table,
                                         int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t batch,
                                         int32_t num_q_heads, int32_t num_kv_heads, float softmax_scale, float* out,
                                         void* workspace, size_t workspace_bytes, uint32_t* dev_flags, void* stream);

/* Chunked prefill over the packed cache.  Sequence b holds prefix_lens[b]/128
 * packed blocks (pages block_table[b, ...]) followed by new_lens[b] fp16 rows:
 * the chunk being prefilled, which is quantised block by block only once whole
 * ("KVarN Nasıl Çalışır?": fixed-size blocks).  Its queries are the last
 * q_lens[b] of those rows; query i sits at fp16 row new_lens[b] - q_lens[b] + i
 * and attends to every packed token and, causally, to fp16 rows 0 .. that row.
 * Scores are scaled as in kvarn_decode_attention; query head h reads KV head
 * h / (num_q_heads / num_kv_heads).
 *   q            fp16 [batch, max_q, num_q_heads, 128], 16-byte aligned
 *   block_table  int32 [batch, max_blocks_per_seq] (device)
 *   prefix_lens  int32 [batch] (device): multiples of 128, at most 128*max_blocks_per_seq
 *   k_new, v_new fp16 [batch, max_new, num_kv_heads, 128], 16-byte aligned;
 *                rows at or past new_lens[b] are never read
 *   new_lens     int32 [batch] (device), 0 .. max_new
 *   q_lens       int32 [batch] (device), 0 .. min(new_lens[b], max_q)
 *   out          fp32 [batch, max_q, num_q_heads, 128], 16-byte aligned; every
 *                row is written, rows at or past q_lens[b] with zeros
 * The rows of sequence b in k_new have the layout of kvarn_quantize_blocks'
 * input, so its full blocks are packed by that call after the step.  No
 * workspace.  Device flags: a page id out of range (that page is skipped), a
 * length out of range (every row of the sequence is zero). */
kvarn_status kvarn_prefill_attention(const kvarn_config* cfg, const void* q, int32_t max_q, const void* k_pool,
                                     const void* v_pool, int32_t num_pages, const int32_t* block_table,
                                     int32_t max_blocks_per_seq, const int32_t* prefix_lens, const void* k_new,
                                     const void* v_new, int32_t max_new, const int32_t* new_lens,
                                     const int32_t* q_lens, int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                     float softmax_scale, float* out, uint32_t* dev_flags, void* stream);

/* Copy *dev_flags to *host_out after the work queued on `stream` finishes
 * (synchronises the stream). */
kvarn_status kvarn_read_flags(const uint32_t* dev_flags, uint32_t* host_out, void* stream);

/* Debug checks, process-wide (on by default in a build with -DKVARN_DEBUG, off
 * otherwise).  While on, kvarn_quantize_blocks first checks that the in-range
 * entries of dst_pages are distinct (two blocks quantised into one page in one
 * call would race on its bytes): it allocates a bitmap, waits for `stream`, and returns KVARN_ERR_SHAPE, writing nothing,
 * when two entries name the same page.  Not for graph capture. */
void kvarn_set_debug_checks(int on);

const char* kvarn_status_string(kvarn_status s);
const char* kvarn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KVARN_H */
