// C ABI of libkvarn: argument validation, launch planning and error reporting.
// The declarations and their contracts are in include/kvarn.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/kvarn.h"

namespace kvarn {
hipError_t launch_quantize(const void* k, const void* v, int n_blocks, int hkv, const int32_t* dst_pages,
                           void* k_pool, void* v_pool, int num_pages, int kbits, int vbits, int group,
                           uint32_t* flags, hipStream_t stream);
hipError_t launch_dequantize(const void* k_pool, const void* v_pool, int num_pages, const int32_t* pages,
                             int n_blocks, int hkv, int kbits, int vbits, int group, float* k_out, float* v_out,
                             uint32_t* flags, hipStream_t stream);
hipError_t launch_decode(const void* q, const void* k_pool, const void* v_pool, int num_pages,
                         const int32_t* block_table, int max_blocks, const int32_t* seq_lens, const void* k_tail,
                         const void* v_tail, int batch, int hq, int hkv, int kbits, int vbits, int group,
                         int blocks_per_split, int max_splits, float scale_log2, float* out, float* part,
                         uint32_t* counters, uint32_t* flags, hipStream_t stream);
hipError_t launch_fp16_decode(const void* q, const void* k_cache, const void* v_cache, int num_pages,
                              const int32_t* block_table, int max_blocks, const int32_t* seq_lens, int batch, int hq,
                              int hkv, int blocks_per_split, int max_splits, float scale_log2, float* out, float* part,
                              uint32_t* counters, uint32_t* flags, hipStream_t stream);
hipError_t launch_quantize_hd(const void* k, const void* v, int n_blocks, int hkv, int head_dim,
                              const int32_t* dst_pages, void* k_pool, void* v_pool, int num_pages, int kbits,
                              int vbits, int group, uint32_t* flags, hipStream_t stream);
hipError_t launch_dequantize_hd(const void* k_pool, const void* v_pool, int num_pages, const int32_t* pages,
                                int n_blocks, int hkv, int head_dim, int kbits, int vbits, int group, float* k_out,
                                float* v_out, uint32_t* flags, hipStream_t stream);
hipError_t launch_decode_hd(const void* q, const void* k_pool, const void* v_pool, int num_pages,
                            const int32_t* block_table, int max_blocks, const int32_t* seq_lens, int batch, int hq,
                            int hkv, int head_dim, int kbits, int vbits, int group, int blocks_per_split,
                            int max_splits, float scale_log2, float* out, float* part, uint32_t* counters,
                            uint32_t* flags, hipStream_t stream);
hipError_t launch_prefill(const void* q, int max_q, const void* k_pool, const void* v_pool, int num_pages,
                          const int32_t* block_table, int max_blocks, const int32_t* prefix_lens, const void* k_new,
                          const void* v_new, int max_new, const int32_t* new_lens, const int32_t* q_lens, int batch,
                          int hq, int hkv, int kbits, int vbits, int group, float scale_log2, float* out,
                          uint32_t* flags, hipStream_t stream);
}  // namespace kvarn

// Scratch memory of the allocation-free decode entry point (kvarn_decode_attention_noalloc): the
// arrival counters in the first kScratchCounterBytes, the split partials after them.  Each GPU the
// library runs on holds its own copy for the life of the process.  Host code never uses this name as
// an address: the per-device address comes from hipGetSymbolAddress (scratch_address below).
constexpr size_t kScratchBytes = static_cast<size_t>(64) << 20;
constexpr size_t kScratchCounterBytes = static_cast<size_t>(1) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Sets n words to zero (a kernel, not a memset, so that a caller may capture it in a HIP graph).
__global__ void zero_words(uint32_t* __restrict__ p, size_t n) {
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    p[i] = 0u;
}

namespace {

constexpr int kMaxGroup = 8;
constexpr int kMaxSplitsPerPair = 64;  // the decode kernel's merge holds at most this many splits
constexpr long kTargetGroups = 768;    // workgroups (4 waves each): one pass over 256 CUs at 3 workgroups per CU
constexpr long kMaxPagesPerSplit = 32;

thread_local std::string g_last_error;

kvarn_status fail(kvarn_status s, const char* msg) {
  g_last_error = msg;
  return s;
}

// kvarn_k{4,8}v{2,4}_g{128,64} with head_dim 64, 128 or 256 and 128-token blocks
bool config_ok(const kvarn_config* c) {
  return c && (c->head_dim == 64 || c->head_dim == 128 || c->head_dim == 256) && c->block_tokens == 128 &&
         (c->k_bits == 4 || c->k_bits == 8) &&
         (c->v_bits == 2 || c->v_bits == 4) && (c->group_size == 128 || c->group_size == 64) &&
         c->norm_iters == 4 && std::fabs(c->eps - 1e-6f) <= 1e-12f;
}

kvarn_status check_config(const kvarn_config* c) {
  if (!c) return fail(KVARN_ERR_NULL, "config is NULL");
  if (!config_ok(c))
    return fail(KVARN_ERR_UNSUPPORTED,
                "supported formats: kvarn_k{4,8}v{2,4}_g{128,64} (head_dim 64, 128 or 256; block 128)");
  return KVARN_OK;
}

// Entry points built for 128-channel heads only (decode with an fp16 tail, the fp16 baseline, prefill).
kvarn_status check_config_128(const kvarn_config* c) {
  kvarn_status s = check_config(c);
  if (s == KVARN_OK && c->head_dim != 128) return fail(KVARN_ERR_UNSUPPORTED, "this entry point needs head_dim 128");
  return s;
}

// codes plus scale and zero fp16 per group, rho fp32[128 tokens] and gamma fp32[head_dim]: key groups are
// one channel over `group` tokens, value groups one token over min(group, head_dim) channels
size_t page_bytes_of(int bits, int group, int head_dim, bool is_v) {
  const int vgc = group < head_dim ? group : head_dim;
  const size_t groups = is_v ? static_cast<size_t>(head_dim / vgc) * 128 : static_cast<size_t>(128 / group) * head_dim;
  return static_cast<size_t>(128) * head_dim * bits / 8 + 4 * groups + 4 * 128 + 4 * static_cast<size_t>(head_dim);
}

struct DecodePlan {
  int blocks_per_split;
  int max_splits;
};

// Pages per split (a multiple of the 4 waves of a workgroup): about one pass of workgroups over the
// chip, at most 32 pages per split so mixed lengths balance, and at most 64 splits per
// (sequence, KV head) so the final merge stays short (63 page splits when an fp16 tail adds one).
DecodePlan plan_decode(int batch, int hkv, int max_blocks, bool tail = false) {
  const long units = static_cast<long>(batch) * hkv * max_blocks;
  long bps = (units + kTargetGroups - 1) / kTargetGroups;
  if (bps > kMaxPagesPerSplit) bps = kMaxPagesPerSplit;
  const long page_splits = tail ? kMaxSplitsPerPair - 1 : kMaxSplitsPerPair;
  const long min_bps = (max_blocks + page_splits - 1) / page_splits;
  if (bps < min_bps) bps = min_bps;
  bps = (bps + 3) / 4 * 4;
  DecodePlan p;
  p.blocks_per_split = static_cast<int>(bps);
  p.max_splits = static_cast<int>((max_blocks + bps - 1) / bps);
  if (p.max_splits < 1) p.max_splits = 1;
  if (tail) p.max_splits += 1;  // the tail split
  return p;
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

size_t counter_bytes(int batch, int hkv) { return align256(static_cast<size_t>(batch) * hkv * sizeof(uint32_t)); }

// Floats of one split partial of one query head: o[head_dim], m, l.
size_t part_floats(int head_dim) { return static_cast<size_t>(head_dim) + 2; }

// Room for the partials of either plan (with or without an fp16 tail split).
size_t workspace_bytes(int batch, int hkv, int max_blocks, int head_dim) {
  const int a = plan_decode(batch, hkv, max_blocks).max_splits;
  const int b = plan_decode(batch, hkv, max_blocks, true).max_splits;
  return counter_bytes(batch, hkv) +
         static_cast<size_t>(batch) * hkv * (a > b ? a : b) * kMaxGroup * part_floats(head_dim) * sizeof(float);
}

kvarn_status launch_status(hipError_t e) {
  if (e == hipSuccess) return KVARN_OK;
  g_last_error = std::string("HIP launch failed: ") + hipGetErrorString(e);
  return KVARN_ERR_LAUNCH;
}

// Device address of `scratch` on the current device, looked up once per device.  The first lookup on a
// device also clears the counter region with a fill kernel on `stream` (every decode call leaves the
// counters it used at zero again, so later calls need no clearing).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

kvarn_status scratch_address(hipStream_t stream, unsigned char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return launch_status(e);
  if (dev < 0 || dev >= kMaxDevices) return fail(KVARN_ERR_UNSUPPORTED, "device index above 63");
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      g_last_error = std::string("hipGetSymbolAddress(scratch) failed: ") + hipGetErrorString(e);
      return KVARN_ERR_LAUNCH;
    }
    hipLaunchKernelGGL(zero_words, dim3(256), dim3(256), 0, stream, static_cast<uint32_t*>(p),
                       kScratchCounterBytes / sizeof(uint32_t));
    e = hipGetLastError();
    if (e != hipSuccess) return launch_status(e);
    g_scratch_ptr[dev] = p;
  }
  *out = static_cast<unsigned char*>(g_scratch_ptr[dev]);
  return KVARN_OK;
}

enum class DecodeKind { packed, packed_tail, fp16 };

// Partials of one decode call (split results of every (sequence, KV head) under the plan).
size_t partial_bytes(int batch, int hkv, int max_splits, int head_dim) {
  return static_cast<size_t>(batch) * hkv * max_splits * kMaxGroup * part_floats(head_dim) * sizeof(float);
}

// Validation and launch shared by the packed decode (with or without an fp16 tail) and the fp16
// baseline (same plan, workspace, partials and error model; the pools and the kernel differ).
kvarn_status decode_common(DecodeKind kind, const kvarn_config* cfg, const void* q, const void* k_pool,
                           const void* v_pool, int32_t num_pages, const int32_t* block_table,
                           int32_t max_blocks_per_seq, const int32_t* seq_lens, const void* k_tail,
                           const void* v_tail, int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                           float softmax_scale, float* out, void* workspace, size_t ws_bytes, uint32_t* dev_flags,
                           void* stream, bool use_scratch = false) {
  kvarn_status s = kind == DecodeKind::packed ? check_config(cfg) : check_config_128(cfg);
  if (s != KVARN_OK) return s;
  const int D = cfg->head_dim;
  if (batch < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_blocks_per_seq < 0 || num_pages < 0)
    return fail(KVARN_ERR_SHAPE, "negative or zero size");
  if (num_q_heads % num_kv_heads != 0) return fail(KVARN_ERR_SHAPE, "num_q_heads must be a multiple of num_kv_heads");
  if (num_q_heads / num_kv_heads > kMaxGroup)
    return fail(KVARN_ERR_UNSUPPORTED, "more than 8 query heads per KV head is not supported");
  if (batch == 0) return KVARN_OK;
  if (!q || !seq_lens || !out) return fail(KVARN_ERR_NULL, "q, seq_lens or out is NULL");
  if (max_blocks_per_seq > 0 && (!block_table || !k_pool || !v_pool))
    return fail(KVARN_ERR_NULL, "block_table or a pool is NULL");
  if (static_cast<long>(max_blocks_per_seq) * 128 + 127 > 0x7FFFFFFFL) return fail(KVARN_ERR_SHAPE, "max_blocks too large");
  if (batch > 65535 || num_kv_heads > 65535) return fail(KVARN_ERR_SHAPE, "batch or num_kv_heads above 65535");
  const int mb = max_blocks_per_seq > 0 ? max_blocks_per_seq : 1;
  if (!use_scratch) {
    const size_t need = workspace_bytes(batch, num_kv_heads, mb, D);
    if (!workspace || ws_bytes < need) return fail(KVARN_ERR_WORKSPACE, "workspace missing or smaller than required");
    if (reinterpret_cast<uintptr_t>(workspace) & 255) return fail(KVARN_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  }
  if ((reinterpret_cast<uintptr_t>(k_pool) | reinterpret_cast<uintptr_t>(v_pool)) & 15)
    return fail(KVARN_ERR_SHAPE, "pools must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(out)) & 15)
    return fail(KVARN_ERR_SHAPE, "q and out must be 16-byte aligned");
  if (max_blocks_per_seq > 0 && num_pages == 0) return fail(KVARN_ERR_SHAPE, "num_pages is 0");
  const bool tail = kind == DecodeKind::packed_tail;
  if (tail) {
    if (!k_tail || !v_tail) return fail(KVARN_ERR_NULL, "k_tail or v_tail is NULL");
    if ((reinterpret_cast<uintptr_t>(k_tail) | reinterpret_cast<uintptr_t>(v_tail)) & 15)
      return fail(KVARN_ERR_SHAPE, "tails must be 16-byte aligned");
  }
  const DecodePlan p = plan_decode(batch, num_kv_heads, mb, tail);
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt(static_cast<float>(D));
  const float scale_log2 = scale * 1.4426950408889634f;
  uint32_t* counters;
  float* part;
  if (use_scratch) {
    if (static_cast<size_t>(batch) * num_kv_heads * sizeof(uint32_t) > kScratchCounterBytes)
      return fail(KVARN_ERR_WORKSPACE, "batch * num_kv_heads above the 262,144 counters of the fixed scratch memory");
    if (partial_bytes(batch, num_kv_heads, p.max_splits, D) > kScratchBytes - kScratchCounterBytes)
      return fail(KVARN_ERR_WORKSPACE,
                  "the split partials of this call exceed the 63 MiB of fixed scratch memory; use "
                  "kvarn_decode_attention with a workspace");
    unsigned char* base = nullptr;
    s = scratch_address(static_cast<hipStream_t>(stream), &base);
    if (s != KVARN_OK) return s;
    counters = reinterpret_cast<uint32_t*>(base);
    part = reinterpret_cast<float*>(base + kScratchCounterBytes);
  } else {
    counters = static_cast<uint32_t*>(workspace);
    part = reinterpret_cast<float*>(static_cast<char*>(workspace) + counter_bytes(batch, num_kv_heads));
  }
  // An empty block table is passed as a harmless non-null pointer; no page is read when max_blocks is 0.
  const int32_t* bt = max_blocks_per_seq > 0 ? block_table : seq_lens;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (kind == DecodeKind::fp16)
    return launch_status(kvarn::launch_fp16_decode(q, k_pool, v_pool, num_pages, bt, max_blocks_per_seq, seq_lens,
                                                   batch, num_q_heads, num_kv_heads, p.blocks_per_split, p.max_splits,
                                                   scale_log2, out, part, counters, dev_flags, st));
  if (D != 128)
    return launch_status(kvarn::launch_decode_hd(q, k_pool, v_pool, num_pages, bt, max_blocks_per_seq, seq_lens, batch,
                                                 num_q_heads, num_kv_heads, D, cfg->k_bits, cfg->v_bits,
                                                 cfg->group_size, p.blocks_per_split, p.max_splits, scale_log2, out,
                                                 part, counters, dev_flags, st));
  return launch_status(kvarn::launch_decode(q, k_pool, v_pool, num_pages, bt, max_blocks_per_seq, seq_lens,
                                            tail ? k_tail : nullptr, tail ? v_tail : nullptr, batch, num_q_heads,
                                            num_kv_heads, cfg->k_bits, cfg->v_bits, cfg->group_size,
                                            p.blocks_per_split, p.max_splits, scale_log2, out, part, counters,
                                            dev_flags, st));
}

}  // namespace

extern "C" {

kvarn_status kvarn_config_parse(const char* name, kvarn_config* out) {
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

size_t kvarn_page_bytes(const kvarn_config* cfg, int is_v) {
  if (!config_ok(cfg)) return 0;
  return page_bytes_of(is_v ? cfg->v_bits : cfg->k_bits, cfg->group_size, cfg->head_dim, is_v != 0);
}

kvarn_status kvarn_quantize_blocks(const kvarn_config* cfg, const void* k, const void* v, int32_t n_blocks,
                                   int32_t num_kv_heads, const int32_t* dst_pages, void* k_pool, void* v_pool,
                                   int32_t num_pages, uint32_t* dev_flags, void* stream) {
  kvarn_status s = check_config(cfg);
  if (s != KVARN_OK) return s;
  if (n_blocks < 0 || num_kv_heads <= 0 || num_pages < 0) return fail(KVARN_ERR_SHAPE, "negative or zero size");
  if (n_blocks == 0) return KVARN_OK;
  if (!k || !v || !dst_pages || !k_pool || !v_pool) return fail(KVARN_ERR_NULL, "a tensor pointer is NULL");
  if (num_pages == 0) return fail(KVARN_ERR_SHAPE, "num_pages is 0");
  if (static_cast<long>(n_blocks) * num_kv_heads * 2 > 0x7FFFFFFFL) return fail(KVARN_ERR_SHAPE, "too many tiles");
  if ((reinterpret_cast<uintptr_t>(k) | reinterpret_cast<uintptr_t>(v)) & 15)
    return fail(KVARN_ERR_SHAPE, "k and v must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(k_pool) | reinterpret_cast<uintptr_t>(v_pool)) & 15)
    return fail(KVARN_ERR_SHAPE, "pools must be 16-byte aligned");
  if (cfg->head_dim != 128)
    return launch_status(kvarn::launch_quantize_hd(k, v, n_blocks, num_kv_heads, cfg->head_dim, dst_pages, k_pool,
                                                   v_pool, num_pages, cfg->k_bits, cfg->v_bits, cfg->group_size,
                                                   dev_flags, static_cast<hipStream_t>(stream)));
  return launch_status(kvarn::launch_quantize(k, v, n_blocks, num_kv_heads, dst_pages, k_pool, v_pool, num_pages,
                                              cfg->k_bits, cfg->v_bits, cfg->group_size, dev_flags,
                                              static_cast<hipStream_t>(stream)));
}

kvarn_status kvarn_dequantize_blocks(const kvarn_config* cfg, const void* k_pool, const void* v_pool,
                                     int32_t num_pages, const int32_t* pages, int32_t n_blocks,
                                     int32_t num_kv_heads, float* k_out, float* v_out, uint32_t* dev_flags,
                                     void* stream) {
  kvarn_status s = check_config(cfg);
  if (s != KVARN_OK) return s;
  if (n_blocks < 0 || num_kv_heads <= 0 || num_pages < 0) return fail(KVARN_ERR_SHAPE, "negative or zero size");
  if (n_blocks == 0 || (!k_out && !v_out)) return KVARN_OK;
  if (!pages || (k_out && !k_pool) || (v_out && !v_pool)) return fail(KVARN_ERR_NULL, "a tensor pointer is NULL");
  if (num_pages == 0) return fail(KVARN_ERR_SHAPE, "num_pages is 0");
  // one workgroup per (block, KV head, K or V): the grid and the kernel's tile index are 32-bit
  if (static_cast<long>(n_blocks) * num_kv_heads * 2 > 0x7FFFFFFFL) return fail(KVARN_ERR_SHAPE, "too many tiles");
  if (cfg->head_dim != 128)
    return launch_status(kvarn::launch_dequantize_hd(k_pool, v_pool, num_pages, pages, n_blocks, num_kv_heads,
                                                     cfg->head_dim, cfg->k_bits, cfg->v_bits, cfg->group_size, k_out,
                                                     v_out, dev_flags, static_cast<hipStream_t>(stream)));
  return launch_status(kvarn::launch_dequantize(k_pool, v_pool, num_pages, pages, n_blocks, num_kv_heads, cfg->k_bits,
                                                cfg->v_bits, cfg->group_size, k_out, v_out, dev_flags,
                                                static_cast<hipStream_t>(stream)));
}

size_t kvarn_decode_workspace_bytes(const kvarn_config* cfg, int32_t batch, int32_t num_q_heads,
                                    int32_t num_kv_heads, int32_t max_blocks_per_seq) {
  if (!config_ok(cfg) || batch < 0 || num_kv_heads <= 0 || num_q_heads <= 0 || max_blocks_per_seq < 0) return 0;
  if (batch == 0) return 0;
  return workspace_bytes(batch, num_kv_heads, max_blocks_per_seq > 0 ? max_blocks_per_seq : 1, cfg->head_dim);
}

kvarn_status kvarn_decode_attention(const kvarn_config* cfg, const void* q, const void* k_pool,
                                    const void* v_pool, int32_t num_pages, const int32_t* block_table,
                                    int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t batch,
                                    int32_t num_q_heads, int32_t num_kv_heads, float softmax_scale, float* out,
                                    void* workspace, size_t ws_bytes, uint32_t* dev_flags, void* stream) {
  return decode_common(DecodeKind::packed, cfg, q, k_pool, v_pool, num_pages, block_table, max_blocks_per_seq,
                       seq_lens, nullptr, nullptr, batch, num_q_heads, num_kv_heads, softmax_scale, out, workspace,
                       ws_bytes, dev_flags, stream);
}

kvarn_status kvarn_decode_attention_tail(const kvarn_config* cfg, const void* q, const void* k_pool,
                                         const void* v_pool, int32_t num_pages, const int32_t* block_table,
                                         int32_t max_blocks_per_seq, const int32_t* seq_lens, const void* k_tail,
                                         const void* v_tail, int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                         float softmax_scale, float* out, void* workspace, size_t ws_bytes,
                                         uint32_t* dev_flags, void* stream) {
  return decode_common(DecodeKind::packed_tail, cfg, q, k_pool, v_pool, num_pages, block_table, max_blocks_per_seq,
                       seq_lens, k_tail, v_tail, batch, num_q_heads, num_kv_heads, softmax_scale, out, workspace,
                       ws_bytes, dev_flags, stream);
}

kvarn_status kvarn_decode_attention_noalloc(const kvarn_config* cfg, const void* q, const void* k_pool,
                                            const void* v_pool, int32_t num_pages, const int32_t* block_table,
                                            int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t batch,
                                            int32_t num_q_heads, int32_t num_kv_heads, float softmax_scale,
                                            float* out, uint32_t* dev_flags, void* stream) {
  return decode_common(DecodeKind::packed, cfg, q, k_pool, v_pool, num_pages, block_table, max_blocks_per_seq,
                       seq_lens, nullptr, nullptr, batch, num_q_heads, num_kv_heads, softmax_scale, out, nullptr, 0,
                       dev_flags, stream, true);
}

size_t kvarn_fp16_page_bytes(const kvarn_config* cfg) {
  return config_ok(cfg) && cfg->head_dim == 128 ? static_cast<size_t>(128) * 128 * sizeof(uint16_t) : 0;
}

kvarn_status kvarn_fp16_decode_attention(const kvarn_config* cfg, const void* q, const void* k_cache,
                                         const void* v_cache, int32_t num_pages, const int32_t* block_table,
                                         int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t batch,
                                         int32_t num_q_heads, int32_t num_kv_heads, float softmax_scale, float* out,
                                         void* workspace, size_t ws_bytes, uint32_t* dev_flags, void* stream) {
  return decode_common(DecodeKind::fp16, cfg, q, k_cache, v_cache, num_pages, block_table, max_blocks_per_seq,
                       seq_lens, nullptr, nullptr, batch, num_q_heads, num_kv_heads, softmax_scale, out, workspace,
                       ws_bytes, dev_flags, stream);
}

kvarn_status kvarn_prefill_attention(const kvarn_config* cfg, const void* q, int32_t max_q, const void* k_pool,
                                     const void* v_pool, int32_t num_pages, const int32_t* block_table,
                                     int32_t max_blocks_per_seq, const int32_t* prefix_lens, const void* k_new,
                                     const void* v_new, int32_t max_new, const int32_t* new_lens,
                                     const int32_t* q_lens, int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                     float softmax_scale, float* out, uint32_t* dev_flags, void* stream) {
  kvarn_status s = check_config_128(cfg);
  if (s != KVARN_OK) return s;
  if (batch < 0 || max_q < 0 || max_new < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_blocks_per_seq < 0 ||
      num_pages < 0)
    return fail(KVARN_ERR_SHAPE, "negative or zero size");
  if (num_q_heads % num_kv_heads != 0) return fail(KVARN_ERR_SHAPE, "num_q_heads must be a multiple of num_kv_heads");
  if (num_q_heads / num_kv_heads > kMaxGroup)
    return fail(KVARN_ERR_UNSUPPORTED, "more than 8 query heads per KV head is not supported");
  if (batch == 0 || max_q == 0) return KVARN_OK;
  if (!q || !prefix_lens || !new_lens || !q_lens || !out) return fail(KVARN_ERR_NULL, "q, a length array or out is NULL");
  if (max_new > 0 && (!k_new || !v_new)) return fail(KVARN_ERR_NULL, "k_new or v_new is NULL");
  if (max_blocks_per_seq > 0 && (!block_table || !k_pool || !v_pool))
    return fail(KVARN_ERR_NULL, "block_table or a pool is NULL");
  if (static_cast<long>(max_blocks_per_seq) * 128 + 127 > 0x7FFFFFFFL) return fail(KVARN_ERR_SHAPE, "max_blocks too large");
  if (batch > 65535 || num_kv_heads > 65535) return fail(KVARN_ERR_SHAPE, "batch or num_kv_heads above 65535");
  if (max_blocks_per_seq > 0 && num_pages == 0) return fail(KVARN_ERR_SHAPE, "num_pages is 0");
  if ((reinterpret_cast<uintptr_t>(k_pool) | reinterpret_cast<uintptr_t>(v_pool)) & 15)
    return fail(KVARN_ERR_SHAPE, "pools must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(out) | reinterpret_cast<uintptr_t>(k_new) |
       reinterpret_cast<uintptr_t>(v_new)) & 15)
    return fail(KVARN_ERR_SHAPE, "q, out, k_new and v_new must be 16-byte aligned");
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt(128.0f);
  const float scale_log2 = scale * 1.4426950408889634f;
  // an empty block table / fp16 region is passed as a harmless non-null pointer; nothing is read from it
  const int32_t* bt = max_blocks_per_seq > 0 ? block_table : prefix_lens;
  const void* kn = max_new > 0 ? k_new : q;
  const void* vn = max_new > 0 ? v_new : q;
  return launch_status(kvarn::launch_prefill(q, max_q, k_pool, v_pool, num_pages, bt, max_blocks_per_seq, prefix_lens,
                                             kn, vn, max_new, new_lens, q_lens, batch, num_q_heads, num_kv_heads,
                                             cfg->k_bits, cfg->v_bits, cfg->group_size, scale_log2, out, dev_flags,
                                             static_cast<hipStream_t>(stream)));
}

kvarn_status kvarn_read_flags(const uint32_t* dev_flags, uint32_t* host_out, void* stream) {
  if (!dev_flags || !host_out) return fail(KVARN_ERR_NULL, "dev_flags or host_out is NULL");
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(host_out, dev_flags, sizeof(uint32_t), hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  return launch_status(e);
}

const char* kvarn_status_string(kvarn_status s) {
  switch (s) {
    case KVARN_OK: return "ok";
    case KVARN_ERR_NULL: return "null pointer";
    case KVARN_ERR_SHAPE: return "bad shape";
    case KVARN_ERR_UNSUPPORTED: return "unsupported configuration";
    case KVARN_ERR_WORKSPACE: return "workspace missing or too small";
    case KVARN_ERR_LAUNCH: return "launch failed";
  }
  return "unknown status";
}

const char* kvarn_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
