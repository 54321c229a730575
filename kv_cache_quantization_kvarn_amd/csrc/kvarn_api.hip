// C ABI of libkvarn: launches, device bookkeeping and error reporting.  Argument validation and launch
// planning are plain host code in kvarn_host.h.  The declarations and their contracts are in include/kvarn.h.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "kvarn_host.h"

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
                         uint32_t* counters, uint32_t* flags, bool prefetch, hipStream_t stream);
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

using kvarn_host::DecodeArgs;
using kvarn_host::DecodeChoice;
using kvarn_host::DecodeKind;
using kvarn_host::DecodePlan;
using kvarn_host::fail;
using kvarn_host::kScratchBytes;
using kvarn_host::kScratchCounterBytes;

// Scratch memory of the allocation-free decode entry point (kvarn_decode_attention_noalloc): the
// arrival counters in the first kScratchCounterBytes, the split partials after them.  Each GPU the
// library runs on holds its own copy for the life of the process.  Host code never uses this name as
// an address: the per-device address comes from hipGetSymbolAddress (scratch_address below).
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Sets n words to zero (a kernel, not a memset, so that a caller may capture it in a HIP graph).
__global__ void zero_words(uint32_t* __restrict__ p, size_t n) {
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    p[i] = 0u;
}

// Debug check of a quantise call's destination pages: marks each in-range page in a bitmap of
// num_pages bits and raises *dup when a page is marked twice.  Entries outside [0, num_pages) are left to
// the quantise kernels, which skip them and raise KVARN_FLAG_BAD_PAGE.
__global__ void mark_pages(const int32_t* __restrict__ pages, int n, int num_pages, uint32_t* __restrict__ bitmap,
                           uint32_t* __restrict__ dup) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) {
    const int p = pages[i];
    if (p < 0 || p >= num_pages) continue;
    const uint32_t bit = 1u << (p & 31);
    if (atomicOr(bitmap + (p >> 5), bit) & bit) atomicOr(dup, 1u);
  }
}

namespace {

kvarn_status launch_status(hipError_t e) {
  if (e == hipSuccess) return KVARN_OK;
  kvarn_host::last_error = std::string("HIP launch failed: ") + hipGetErrorString(e);
  return KVARN_ERR_LAUNCH;
}

constexpr int kMaxDevices = 64;

// Compute units of the current device, asked once per device (the decode plan spreads its splits over
// them; a partitioned GPU shows fewer).  Without a device the plan assumes kDefaultCus.
std::atomic<int> g_cus[kMaxDevices];

int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return kvarn_host::kDefaultCus;
  }
  int n = g_cus[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    return kvarn_host::kDefaultCus;
  }
  g_cus[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Device address of `scratch` on the current device, looked up once per device.  The first lookup on a
// device also clears the counter region with a fill kernel on `stream` (every decode call leaves the
// counters it used at zero again, so later calls need no clearing).
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
      kvarn_host::last_error = std::string("hipGetSymbolAddress(scratch) failed: ") + hipGetErrorString(e);
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

#ifdef KVARN_DEBUG
std::atomic<int> g_debug_checks{1};
#else
std::atomic<int> g_debug_checks{0};
#endif

// With debug checks on: fail with KVARN_ERR_SHAPE, before anything is written, when two entries of
// dst_pages name the same page.  Allocates a bitmap and waits for the stream (not for graph capture).
kvarn_status check_distinct_pages(const int32_t* dst_pages, int n, int num_pages, hipStream_t st) {
  const size_t words = (static_cast<size_t>(num_pages) + 31) / 32 + 1;  // bitmap, then the duplicate word
  uint32_t* buf = nullptr;
  hipError_t e = hipMalloc(&buf, words * sizeof(uint32_t));
  if (e != hipSuccess) return launch_status(e);
  uint32_t dup = 0;
  hipLaunchKernelGGL(zero_words, dim3(256), dim3(256), 0, st, buf, words);
  e = hipGetLastError();
  if (e == hipSuccess) {
    const int grid = static_cast<int>(n / 256 + 1 < 4096 ? n / 256 + 1 : 4096);
    hipLaunchKernelGGL(mark_pages, dim3(grid), dim3(256), 0, st, dst_pages, n, num_pages, buf, buf + words - 1);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipMemcpyAsync(&dup, buf + words - 1, sizeof(uint32_t), hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  const hipError_t ef = hipFree(buf);
  if (e == hipSuccess) e = ef;
  if (e != hipSuccess) return launch_status(e);
  if (dup) return fail(KVARN_ERR_SHAPE, "dst_pages entries are not distinct (debug check)");
  return KVARN_OK;
}

// Validation and launch shared by the packed decode (with or without an fp16 tail), its allocation-free
// variant and the fp16 baseline (same plan, workspace, partials and error model; the pools and the
// kernel differ).
kvarn_status decode_common(DecodeArgs a, uint32_t* dev_flags, float softmax_scale, float* out, void* workspace,
                           void* stream) {
  a.cus = device_cus();
  bool run = false;
  DecodeChoice choice{};
  kvarn_status s = kvarn_host::validate_decode(a, &run, &choice);
  if (s != KVARN_OK || !run) return s;
  const DecodePlan& p = choice.plan;
  const int D = a.cfg->head_dim;
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt(static_cast<float>(D));
  const float scale_log2 = scale * 1.4426950408889634f;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  uint32_t* counters;
  float* part;
  if (a.use_scratch) {
    unsigned char* base = nullptr;
    s = scratch_address(st, &base);
    if (s != KVARN_OK) return s;
    counters = reinterpret_cast<uint32_t*>(base);
    part = reinterpret_cast<float*>(base + kScratchCounterBytes);
  } else {
    counters = static_cast<uint32_t*>(workspace);
    part = reinterpret_cast<float*>(static_cast<char*>(workspace) + kvarn_host::counter_bytes(a.batch, a.num_kv_heads));
  }
  // An empty block table is passed as a harmless non-null pointer; no page is read when max_blocks is 0.
  const int32_t* bt = a.max_blocks > 0 ? a.block_table : a.seq_lens;
  if (a.kind == DecodeKind::fp16)
    return launch_status(kvarn::launch_fp16_decode(a.q, a.k_pool, a.v_pool, a.num_pages, bt, a.max_blocks, a.seq_lens,
                                                   a.batch, a.num_q_heads, a.num_kv_heads, p.blocks_per_split,
                                                   p.max_splits, scale_log2, out, part, counters, dev_flags, st));
  if (D != 128)
    return launch_status(kvarn::launch_decode_hd(a.q, a.k_pool, a.v_pool, a.num_pages, bt, a.max_blocks, a.seq_lens,
                                                 a.batch, a.num_q_heads, a.num_kv_heads, D, a.cfg->k_bits,
                                                 a.cfg->v_bits, a.cfg->group_size, p.blocks_per_split, p.max_splits,
                                                 scale_log2, out, part, counters, dev_flags, st));
  const bool tail = a.kind == DecodeKind::packed_tail;
  return launch_status(kvarn::launch_decode(a.q, a.k_pool, a.v_pool, a.num_pages, bt, a.max_blocks, a.seq_lens,
                                            tail ? a.k_tail : nullptr, tail ? a.v_tail : nullptr, a.batch,
                                            a.num_q_heads, a.num_kv_heads, a.cfg->k_bits, a.cfg->v_bits,
                                            a.cfg->group_size, p.blocks_per_split, p.max_splits, scale_log2, out, part,
                                            counters, dev_flags, choice.prefetch, st));
}

DecodeArgs decode_args(DecodeKind kind, const kvarn_config* cfg, const void* q, const void* k_pool, const void* v_pool,
                       int32_t num_pages, const int32_t* block_table, int32_t max_blocks, const int32_t* seq_lens,
                       const void* k_tail, const void* v_tail, int32_t batch, int32_t nq, int32_t hkv, const float* out,
                       const void* workspace, size_t ws_bytes, bool use_scratch) {
  DecodeArgs a;
  a.kind = kind;
  a.cfg = cfg;
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.num_pages = num_pages;
  a.block_table = block_table;
  a.max_blocks = max_blocks;
  a.seq_lens = seq_lens;
  a.k_tail = k_tail;
  a.v_tail = v_tail;
  a.batch = batch;
  a.num_q_heads = nq;
  a.num_kv_heads = hkv;
  a.out = out;
  a.workspace = workspace;
  a.ws_bytes = ws_bytes;
  a.use_scratch = use_scratch;
  a.cus = kvarn_host::kDefaultCus;
  return a;
}

}  // namespace

extern "C" {

kvarn_status kvarn_config_parse(const char* name, kvarn_config* out) { return kvarn_host::parse_config(name, out); }

size_t kvarn_page_bytes(const kvarn_config* cfg, int is_v) { return kvarn_host::page_bytes(cfg, is_v != 0); }

kvarn_status kvarn_quantize_blocks(const kvarn_config* cfg, const void* k, const void* v, int32_t n_blocks,
                                   int32_t num_kv_heads, const int32_t* dst_pages, void* k_pool, void* v_pool,
                                   int32_t num_pages, uint32_t* dev_flags, void* stream) {
  bool run = false;
  kvarn_status s = kvarn_host::validate_quantize(cfg, k, v, n_blocks, num_kv_heads, dst_pages, k_pool, v_pool,
                                                 num_pages, &run);
  if (s != KVARN_OK || !run) return s;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (g_debug_checks.load(std::memory_order_relaxed)) {
    s = check_distinct_pages(dst_pages, n_blocks, num_pages, st);
    if (s != KVARN_OK) return s;
  }
  if (cfg->head_dim != 128)
    return launch_status(kvarn::launch_quantize_hd(k, v, n_blocks, num_kv_heads, cfg->head_dim, dst_pages, k_pool,
                                                   v_pool, num_pages, cfg->k_bits, cfg->v_bits, cfg->group_size,
                                                   dev_flags, st));
  return launch_status(kvarn::launch_quantize(k, v, n_blocks, num_kv_heads, dst_pages, k_pool, v_pool, num_pages,
                                              cfg->k_bits, cfg->v_bits, cfg->group_size, dev_flags, st));
}

kvarn_status kvarn_dequantize_blocks(const kvarn_config* cfg, const void* k_pool, const void* v_pool,
                                     int32_t num_pages, const int32_t* pages, int32_t n_blocks,
                                     int32_t num_kv_heads, float* k_out, float* v_out, uint32_t* dev_flags,
                                     void* stream) {
  bool run = false;
  kvarn_status s = kvarn_host::validate_dequantize(cfg, k_pool, v_pool, num_pages, pages, n_blocks, num_kv_heads,
                                                   k_out, v_out, &run);
  if (s != KVARN_OK || !run) return s;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (cfg->head_dim != 128)
    return launch_status(kvarn::launch_dequantize_hd(k_pool, v_pool, num_pages, pages, n_blocks, num_kv_heads,
                                                     cfg->head_dim, cfg->k_bits, cfg->v_bits, cfg->group_size, k_out,
                                                     v_out, dev_flags, st));
  return launch_status(kvarn::launch_dequantize(k_pool, v_pool, num_pages, pages, n_blocks, num_kv_heads, cfg->k_bits,
                                                cfg->v_bits, cfg->group_size, k_out, v_out, dev_flags, st));
}

size_t kvarn_decode_workspace_bytes(const kvarn_config* cfg, int32_t batch, int32_t num_q_heads,
                                    int32_t num_kv_heads, int32_t max_blocks_per_seq) {
  return kvarn_host::decode_workspace_bytes(cfg, batch, num_q_heads, num_kv_heads, max_blocks_per_seq, device_cus());
}

kvarn_status kvarn_decode_attention(const kvarn_config* cfg, const void* q, const void* k_pool,
                                    const void* v_pool, int32_t num_pages, const int32_t* block_table,
                                    int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t batch,
                                    int32_t num_q_heads, int32_t num_kv_heads, float softmax_scale, float* out,
                                    void* workspace, size_t ws_bytes, uint32_t* dev_flags, void* stream) {
  return decode_common(decode_args(DecodeKind::packed, cfg, q, k_pool, v_pool, num_pages, block_table,
                                   max_blocks_per_seq, seq_lens, nullptr, nullptr, batch, num_q_heads, num_kv_heads,
                                   out, workspace, ws_bytes, false),
                       dev_flags, softmax_scale, out, workspace, stream);
}

kvarn_status kvarn_decode_attention_tail(const kvarn_config* cfg, const void* q, const void* k_pool,
                                         const void* v_pool, int32_t num_pages, const int32_t* block_table,
                                         int32_t max_blocks_per_seq, const int32_t* seq_lens, const void* k_tail,
                                         const void* v_tail, int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                         float softmax_scale, float* out, void* workspace, size_t ws_bytes,
                                         uint32_t* dev_flags, void* stream) {
  return decode_common(decode_args(DecodeKind::packed_tail, cfg, q, k_pool, v_pool, num_pages, block_table,
                                   max_blocks_per_seq, seq_lens, k_tail, v_tail, batch, num_q_heads, num_kv_heads, out,
                                   workspace, ws_bytes, false),
                       dev_flags, softmax_scale, out, workspace, stream);
}

kvarn_status kvarn_decode_attention_noalloc(const kvarn_config* cfg, const void* q, const void* k_pool,
                                            const void* v_pool, int32_t num_pages, const int32_t* block_table,
                                            int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t batch,
                                            int32_t num_q_heads, int32_t num_kv_heads, float softmax_scale,
                                            float* out, uint32_t* dev_flags, void* stream) {
  return decode_common(decode_args(DecodeKind::packed, cfg, q, k_pool, v_pool, num_pages, block_table,
                                   max_blocks_per_seq, seq_lens, nullptr, nullptr, batch, num_q_heads, num_kv_heads,
                                   out, nullptr, 0, true),
                       dev_flags, softmax_scale, out, nullptr, stream);
}

size_t kvarn_fp16_page_bytes(const kvarn_config* cfg) {
  return kvarn_host::config_ok(cfg) && cfg->head_dim == 128 ? static_cast<size_t>(128) * 128 * sizeof(uint16_t) : 0;
}

kvarn_status kvarn_fp16_decode_attention(const kvarn_config* cfg, const void* q, const void* k_cache,
                                         const void* v_cache, int32_t num_pages, const int32_t* block_table,
                                         int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t batch,
                                         int32_t num_q_heads, int32_t num_kv_heads, float softmax_scale, float* out,
                                         void* workspace, size_t ws_bytes, uint32_t* dev_flags, void* stream) {
  return decode_common(decode_args(DecodeKind::fp16, cfg, q, k_cache, v_cache, num_pages, block_table,
                                   max_blocks_per_seq, seq_lens, nullptr, nullptr, batch, num_q_heads, num_kv_heads,
                                   out, workspace, ws_bytes, false),
                       dev_flags, softmax_scale, out, workspace, stream);
}

kvarn_status kvarn_prefill_attention(const kvarn_config* cfg, const void* q, int32_t max_q, const void* k_pool,
                                     const void* v_pool, int32_t num_pages, const int32_t* block_table,
                                     int32_t max_blocks_per_seq, const int32_t* prefix_lens, const void* k_new,
                                     const void* v_new, int32_t max_new, const int32_t* new_lens,
                                     const int32_t* q_lens, int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                     float softmax_scale, float* out, uint32_t* dev_flags, void* stream) {
  bool run = false;
  kvarn_status s = kvarn_host::validate_prefill(cfg, q, max_q, k_pool, v_pool, num_pages, block_table,
                                                max_blocks_per_seq, prefix_lens, k_new, v_new, max_new, new_lens,
                                                q_lens, batch, num_q_heads, num_kv_heads, out, &run);
  if (s != KVARN_OK || !run) return s;
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

void kvarn_set_debug_checks(int on) { g_debug_checks.store(on != 0, std::memory_order_relaxed); }

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

const char* kvarn_last_error(void) { return kvarn_host::last_error.c_str(); }

}  // extern "C"
