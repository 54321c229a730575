// Host-side argument validation, formats and launch planning of the C ABI (include/kvarn.h).
//
// Plain C++17 with no HIP types or calls: the library includes it, and a host self-test
// (host_selftest.cpp) builds it with AddressSanitizer and UndefinedBehaviorSanitizer to drive every
// check with extreme arguments, without a GPU.  Every validate_* function either returns an error
// (message in last_error) or KVARN_OK with *run telling whether there is work to launch.
#pragma once

#include <cmath>
#include <cstddef>
#include <cstdint>
#include <cstdio>
#include <string>

#include "../../include/kvarn.h"

namespace kvarn_host {

constexpr int kMaxGroup = 8;           // query heads per KV head the decode and prefill kernels hold
constexpr int kMaxSplitsPerPair = 64;  // the decode kernel's merge holds at most this many splits
constexpr long kMaxPagesPerSplit = 32;
constexpr int kWorkgroupsPerCu = 3;    // decode workgroups (4 waves each) per CU in one pass, three waves per SIMD
constexpr int kPrefetchWorkgroupsPerCu = 2;  // the same for the prefetching decode (two waves per SIMD)
constexpr int kPrefetchMaxPagesPerSplit = 16;  // longer splits stream better with the third wave than with prefetch
constexpr int kDefaultCus = 256;       // used when the device cannot be asked

// Scratch memory of the allocation-free decode: counters first, split partials after them.
constexpr size_t kScratchBytes = static_cast<size_t>(64) << 20;
constexpr size_t kScratchCounterBytes = static_cast<size_t>(1) << 20;

inline thread_local std::string last_error;

inline kvarn_status fail(kvarn_status s, const char* msg) {
  last_error = msg;
  return s;
}

inline bool misaligned(const void* p, uintptr_t align) { return (reinterpret_cast<uintptr_t>(p) & (align - 1)) != 0; }

// kvarn_k{4,8}v{2,4}_g{128,64} with head_dim 64, 128 or 256 and 128-token blocks
inline bool config_ok(const kvarn_config* c) {
  return c && (c->head_dim == 64 || c->head_dim == 128 || c->head_dim == 256) && c->block_tokens == 128 &&
         (c->k_bits == 4 || c->k_bits == 8) && (c->v_bits == 2 || c->v_bits == 4) &&
         (c->group_size == 128 || c->group_size == 64) && c->norm_iters == 4 && std::fabs(c->eps - 1e-6f) <= 1e-12f;
}

inline kvarn_status check_config(const kvarn_config* c) {
  if (!c) return fail(KVARN_ERR_NULL, "config is NULL");
  if (!config_ok(c))
    return fail(KVARN_ERR_UNSUPPORTED,
                "supported formats: kvarn_k{4,8}v{2,4}_g{128,64} (head_dim 64, 128 or 256; block 128)");
  return KVARN_OK;
}

// Entry points built for 128-channel heads only (decode with an fp16 tail, the fp16 baseline, prefill).
inline kvarn_status check_config_128(const kvarn_config* c) {
  kvarn_status s = check_config(c);
  if (s == KVARN_OK && c->head_dim != 128) return fail(KVARN_ERR_UNSUPPORTED, "this entry point needs head_dim 128");
  return s;
}

inline kvarn_status parse_config(const char* name, kvarn_config* out) {
  if (!name || !out) return fail(KVARN_ERR_NULL, "name or out is NULL");
  int kb = 0, vb = 0, gs = 0, used = 0;
  if (std::sscanf(name, "kvarn_k%dv%d_g%d%n", &kb, &vb, &gs, &used) != 3 || name[used] != '\0')
    return fail(KVARN_ERR_UNSUPPORTED, "cache dtype name is not of the form kvarn_k<K>v<V>_g<G>");
  out->head_dim = 128;
  out->block_tokens = 128;
  out->k_bits = kb;
  out->v_bits = vb;
  out->group_size = gs;
  out->norm_iters = 4;
  out->eps = 1e-6f;
  if (!config_ok(out)) return fail(KVARN_ERR_UNSUPPORTED, "implemented formats: kvarn_k{4,8}v{2,4}_g{128,64}");
  return KVARN_OK;
}

// codes plus scale and zero fp16 per group, rho fp32[128 tokens] and gamma fp32[head_dim]: key groups are
// one channel over `group` tokens, value groups one token over min(group, head_dim) channels
inline size_t page_bytes_of(int bits, int group, int head_dim, bool is_v) {
  const int vgc = group < head_dim ? group : head_dim;
  const size_t groups = is_v ? static_cast<size_t>(head_dim / vgc) * 128 : static_cast<size_t>(128 / group) * head_dim;
  return static_cast<size_t>(128) * head_dim * bits / 8 + 4 * groups + 4 * 128 + 4 * static_cast<size_t>(head_dim);
}

inline size_t page_bytes(const kvarn_config* cfg, bool is_v) {
  if (!config_ok(cfg)) return 0;
  return page_bytes_of(is_v ? cfg->v_bits : cfg->k_bits, cfg->group_size, cfg->head_dim, is_v);
}

struct DecodePlan {
  int blocks_per_split;
  int max_splits;
};

// Pages per split (a multiple of the 4 waves of a workgroup): about one pass of workgroups over the
// device's CUs (wgs_per_cu each), at most 32 pages per split so mixed lengths balance, and at most 64
// splits per (sequence, KV head) so the final merge stays short (63 page splits when an fp16 tail adds
// one).  Callers bound batch, num_kv_heads (65535) and max_blocks (2^24 - 1), so `units` fits in a long.
inline DecodePlan plan_decode(int batch, int hkv, int max_blocks, int cus, bool tail = false,
                              int wgs_per_cu = kWorkgroupsPerCu) {
  const long target = static_cast<long>(cus > 0 ? cus : kDefaultCus) * wgs_per_cu;
  const long units = static_cast<long>(batch) * hkv * max_blocks;
  long bps = (units + target - 1) / target;
  if (bps > kMaxPagesPerSplit) bps = kMaxPagesPerSplit;
  const long page_splits = tail ? kMaxSplitsPerPair - 1 : kMaxSplitsPerPair;
  const long min_bps = (static_cast<long>(max_blocks) + page_splits - 1) / page_splits;
  if (bps < min_bps) bps = min_bps;
  bps = (bps + 3) / 4 * 4;
  DecodePlan p;
  p.blocks_per_split = static_cast<int>(bps);
  p.max_splits = static_cast<int>((max_blocks + bps - 1) / bps);
  if (p.max_splits < 1) p.max_splits = 1;
  if (tail) p.max_splits += 1;  // the tail split
  return p;
}

inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

inline size_t counter_bytes(int batch, int hkv) { return align256(static_cast<size_t>(batch) * hkv * sizeof(uint32_t)); }

// Floats of one split partial of one query head: o[head_dim], m, l.
inline size_t part_floats(int head_dim) { return static_cast<size_t>(head_dim) + 2; }

// Partials of one decode call (split results of every (sequence, KV head) under the plan).
inline size_t partial_bytes(int batch, int hkv, int max_splits, int head_dim) {
  return static_cast<size_t>(batch) * hkv * max_splits * kMaxGroup * part_floats(head_dim) * sizeof(float);
}

// Shape limits shared by decode and prefill: the grid's y/z extents and 32-bit token positions.
inline bool decode_sizes_in_range(int batch, int hkv, int max_blocks) {
  return batch <= 65535 && hkv <= 65535 && static_cast<long>(max_blocks) * 128 + 127 <= 0x7FFFFFFFL;
}

// The plan a packed decode launches with, and whether it runs the prefetching kernel: formats that
// have one first try two workgroups per CU and take them when the splits stay short (a wave then has
// at most four pages, whose loads the prefetch hides); otherwise three workgroups per CU without it.
struct DecodeChoice {
  DecodePlan plan;
  bool prefetch;
};
inline DecodeChoice choose_decode(int batch, int hkv, int max_blocks, int cus, bool tail, bool can_prefetch) {
  if (can_prefetch) {
    const DecodePlan p = plan_decode(batch, hkv, max_blocks, cus, tail, kPrefetchWorkgroupsPerCu);
    if (p.blocks_per_split <= kPrefetchMaxPagesPerSplit) return DecodeChoice{p, true};
  }
  return DecodeChoice{plan_decode(batch, hkv, max_blocks, cus, tail), false};
}

// Room for the partials of every plan a decode of these sizes may choose (with or without an fp16
// tail split, with or without prefetch).
inline size_t workspace_bytes(int batch, int hkv, int max_blocks, int head_dim, int cus) {
  int splits = 0;
  for (int tail = 0; tail < 2; ++tail)
    for (int wpc : {kWorkgroupsPerCu, kPrefetchWorkgroupsPerCu}) {
      const int m = plan_decode(batch, hkv, max_blocks, cus, tail != 0, wpc).max_splits;
      splits = m > splits ? m : splits;
    }
  return counter_bytes(batch, hkv) + partial_bytes(batch, hkv, splits, head_dim);
}

// kvarn_decode_workspace_bytes: 0 for an unsupported config, a bad or out-of-range shape, or batch 0.
inline size_t decode_workspace_bytes(const kvarn_config* cfg, int batch, int nq, int hkv, int max_blocks, int cus) {
  if (!config_ok(cfg) || batch <= 0 || hkv <= 0 || nq <= 0 || max_blocks < 0) return 0;
  if (!decode_sizes_in_range(batch, hkv, max_blocks)) return 0;
  return workspace_bytes(batch, hkv, max_blocks > 0 ? max_blocks : 1, cfg->head_dim, cus);
}

inline kvarn_status validate_quantize(const kvarn_config* cfg, const void* k, const void* v, int n_blocks, int hkv,
                                      const int32_t* dst_pages, const void* k_pool, const void* v_pool, int num_pages,
                                      bool* run) {
  *run = false;
  kvarn_status s = check_config(cfg);
  if (s != KVARN_OK) return s;
  if (n_blocks < 0 || hkv <= 0 || num_pages < 0) return fail(KVARN_ERR_SHAPE, "negative or zero size");
  if (n_blocks == 0) return KVARN_OK;
  if (!k || !v || !dst_pages || !k_pool || !v_pool) return fail(KVARN_ERR_NULL, "a tensor pointer is NULL");
  if (num_pages == 0) return fail(KVARN_ERR_SHAPE, "num_pages is 0");
  // one tile per (block, KV head, K or V): the kernels' tile index is 32-bit
  if (static_cast<long>(n_blocks) * hkv * 2 > 0x7FFFFFFFL) return fail(KVARN_ERR_SHAPE, "too many tiles");
  if (misaligned(k, 16) || misaligned(v, 16)) return fail(KVARN_ERR_SHAPE, "k and v must be 16-byte aligned");
  if (misaligned(k_pool, 16) || misaligned(v_pool, 16)) return fail(KVARN_ERR_SHAPE, "pools must be 16-byte aligned");
  *run = true;
  return KVARN_OK;
}

inline kvarn_status validate_dequantize(const kvarn_config* cfg, const void* k_pool, const void* v_pool, int num_pages,
                                        const int32_t* pages, int n_blocks, int hkv, const float* k_out,
                                        const float* v_out, bool* run) {
  *run = false;
  kvarn_status s = check_config(cfg);
  if (s != KVARN_OK) return s;
  if (n_blocks < 0 || hkv <= 0 || num_pages < 0) return fail(KVARN_ERR_SHAPE, "negative or zero size");
  if (n_blocks == 0 || (!k_out && !v_out)) return KVARN_OK;
  if (!pages || (k_out && !k_pool) || (v_out && !v_pool)) return fail(KVARN_ERR_NULL, "a tensor pointer is NULL");
  if (num_pages == 0) return fail(KVARN_ERR_SHAPE, "num_pages is 0");
  // one workgroup per (block, KV head, K or V): the grid and the kernel's tile index are 32-bit
  if (static_cast<long>(n_blocks) * hkv * 2 > 0x7FFFFFFFL) return fail(KVARN_ERR_SHAPE, "too many tiles");
  *run = true;
  return KVARN_OK;
}

enum class DecodeKind { packed, packed_tail, fp16 };

struct DecodeArgs {
  DecodeKind kind;
  const kvarn_config* cfg;
  const void* q;
  const void* k_pool;
  const void* v_pool;
  int num_pages;
  const int32_t* block_table;
  int max_blocks;
  const int32_t* seq_lens;
  const void* k_tail;
  const void* v_tail;
  int batch, num_q_heads, num_kv_heads;
  const float* out;
  const void* workspace;
  size_t ws_bytes;
  bool use_scratch;  // the allocation-free variant: partials and counters in the fixed scratch memory
  int cus;           // compute units of the device the call runs on
};

// Validation of the packed decode (with or without an fp16 tail), its allocation-free variant and the
// fp16 baseline; on success with *run, *choice is the split plan to launch and the kernel to run it.
inline kvarn_status validate_decode(const DecodeArgs& a, bool* run, DecodeChoice* choice) {
  *run = false;
  kvarn_status s = a.kind == DecodeKind::packed ? check_config(a.cfg) : check_config_128(a.cfg);
  if (s != KVARN_OK) return s;
  if (a.batch < 0 || a.num_q_heads <= 0 || a.num_kv_heads <= 0 || a.max_blocks < 0 || a.num_pages < 0)
    return fail(KVARN_ERR_SHAPE, "negative or zero size");
  if (a.num_q_heads % a.num_kv_heads != 0)
    return fail(KVARN_ERR_SHAPE, "num_q_heads must be a multiple of num_kv_heads");
  if (a.num_q_heads / a.num_kv_heads > kMaxGroup)
    return fail(KVARN_ERR_UNSUPPORTED, "more than 8 query heads per KV head is not supported");
  if (a.batch == 0) return KVARN_OK;
  if (!a.q || !a.seq_lens || !a.out) return fail(KVARN_ERR_NULL, "q, seq_lens or out is NULL");
  if (a.max_blocks > 0 && (!a.block_table || !a.k_pool || !a.v_pool))
    return fail(KVARN_ERR_NULL, "block_table or a pool is NULL");
  if (static_cast<long>(a.max_blocks) * 128 + 127 > 0x7FFFFFFFL) return fail(KVARN_ERR_SHAPE, "max_blocks too large");
  if (!decode_sizes_in_range(a.batch, a.num_kv_heads, a.max_blocks))
    return fail(KVARN_ERR_SHAPE, "batch or num_kv_heads above 65535");
  const int mb = a.max_blocks > 0 ? a.max_blocks : 1;
  const int D = a.cfg->head_dim;
  if (!a.use_scratch) {
    const size_t need = workspace_bytes(a.batch, a.num_kv_heads, mb, D, a.cus);
    if (!a.workspace || a.ws_bytes < need) return fail(KVARN_ERR_WORKSPACE, "workspace missing or smaller than required");
    if (misaligned(a.workspace, 256)) return fail(KVARN_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  }
  if (misaligned(a.k_pool, 16) || misaligned(a.v_pool, 16)) return fail(KVARN_ERR_SHAPE, "pools must be 16-byte aligned");
  if (misaligned(a.q, 16) || misaligned(a.out, 16)) return fail(KVARN_ERR_SHAPE, "q and out must be 16-byte aligned");
  if (a.max_blocks > 0 && a.num_pages == 0) return fail(KVARN_ERR_SHAPE, "num_pages is 0");
  const bool tail = a.kind == DecodeKind::packed_tail;
  if (tail) {
    if (!a.k_tail || !a.v_tail) return fail(KVARN_ERR_NULL, "k_tail or v_tail is NULL");
    if (misaligned(a.k_tail, 16) || misaligned(a.v_tail, 16))
      return fail(KVARN_ERR_SHAPE, "tails must be 16-byte aligned");
  }
  // a prefetching kernel exists for 128-channel heads with 4-bit keys and group size 128
  const bool can_prefetch = a.kind != DecodeKind::fp16 && D == 128 && a.cfg->k_bits == 4 && a.cfg->group_size == 128;
  // the 64-channel decode (a page per wave, two waves per SIMD) plans two workgroups per CU
  const DecodeChoice c = D == 64 ? DecodeChoice{plan_decode(a.batch, a.num_kv_heads, mb, a.cus, tail,
                                                            kPrefetchWorkgroupsPerCu), false}
                                 : choose_decode(a.batch, a.num_kv_heads, mb, a.cus, tail, can_prefetch);
  const DecodePlan& p = c.plan;
  if (a.use_scratch) {
    if (static_cast<size_t>(a.batch) * a.num_kv_heads * sizeof(uint32_t) > kScratchCounterBytes)
      return fail(KVARN_ERR_WORKSPACE, "batch * num_kv_heads above the 262,144 counters of the fixed scratch memory");
    if (partial_bytes(a.batch, a.num_kv_heads, p.max_splits, D) > kScratchBytes - kScratchCounterBytes)
      return fail(KVARN_ERR_WORKSPACE,
                  "the split partials of this call exceed the 63 MiB of fixed scratch memory; use "
                  "kvarn_decode_attention with a workspace");
  }
  *choice = c;
  *run = true;
  return KVARN_OK;
}

inline kvarn_status validate_prefill(const kvarn_config* cfg, const void* q, int max_q, const void* k_pool,
                                     const void* v_pool, int num_pages, const int32_t* block_table, int max_blocks,
                                     const int32_t* prefix_lens, const void* k_new, const void* v_new, int max_new,
                                     const int32_t* new_lens, const int32_t* q_lens, int batch, int nq, int hkv,
                                     const float* out, bool* run) {
  *run = false;
  kvarn_status s = check_config_128(cfg);
  if (s != KVARN_OK) return s;
  if (batch < 0 || max_q < 0 || max_new < 0 || nq <= 0 || hkv <= 0 || max_blocks < 0 || num_pages < 0)
    return fail(KVARN_ERR_SHAPE, "negative or zero size");
  if (nq % hkv != 0) return fail(KVARN_ERR_SHAPE, "num_q_heads must be a multiple of num_kv_heads");
  if (nq / hkv > kMaxGroup) return fail(KVARN_ERR_UNSUPPORTED, "more than 8 query heads per KV head is not supported");
  if (batch == 0 || max_q == 0) return KVARN_OK;
  if (!q || !prefix_lens || !new_lens || !q_lens || !out) return fail(KVARN_ERR_NULL, "q, a length array or out is NULL");
  if (max_new > 0 && (!k_new || !v_new)) return fail(KVARN_ERR_NULL, "k_new or v_new is NULL");
  if (max_blocks > 0 && (!block_table || !k_pool || !v_pool)) return fail(KVARN_ERR_NULL, "block_table or a pool is NULL");
  if (static_cast<long>(max_blocks) * 128 + 127 > 0x7FFFFFFFL) return fail(KVARN_ERR_SHAPE, "max_blocks too large");
  if (!decode_sizes_in_range(batch, hkv, max_blocks)) return fail(KVARN_ERR_SHAPE, "batch or num_kv_heads above 65535");
  if (max_blocks > 0 && num_pages == 0) return fail(KVARN_ERR_SHAPE, "num_pages is 0");
  if (misaligned(k_pool, 16) || misaligned(v_pool, 16)) return fail(KVARN_ERR_SHAPE, "pools must be 16-byte aligned");
  if (misaligned(q, 16) || misaligned(out, 16) || misaligned(k_new, 16) || misaligned(v_new, 16))
    return fail(KVARN_ERR_SHAPE, "q, out, k_new and v_new must be 16-byte aligned");
  *run = true;
  return KVARN_OK;
}

}  // namespace kvarn_host
