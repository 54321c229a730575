// Host self-test of the C ABI's validation and planning (kvarn_host.h), built with g++ and
// AddressSanitizer + UndefinedBehaviorSanitizer (no recovery) and run by the CPU tests.  It drives every
// validate_* function over extreme sizes, NULL and misaligned pointers and every format, checking the
// documented status for chosen cases and, whenever a call would launch, that its sizes and split plan
// are ones the kernels accept.  Any overflow or out-of-bounds access aborts the run.
#include <climits>
#include <cstdio>
#include <cstring>
#include <vector>

#include "kvarn_host.h"

namespace {

long g_checks = 0, g_failures = 0;

void check(bool ok, const char* what, long a = 0, long b = 0, long c = 0) {
  ++g_checks;
  if (!ok) {
    ++g_failures;
    if (g_failures <= 20) std::printf("FAILED: %s (%ld, %ld, %ld) last_error=%s\n", what, a, b, c, kvarn_host::last_error.c_str());
  }
}

bool valid_status(kvarn_status s) { return s <= KVARN_OK && s >= KVARN_ERR_LAUNCH; }

// fake device addresses: only their values are inspected
const void* const kAligned = reinterpret_cast<const void*>(static_cast<uintptr_t>(1) << 20);
const void* const kOdd = reinterpret_cast<const void*>((static_cast<uintptr_t>(1) << 20) + 4);
const int32_t* const kTable = reinterpret_cast<const int32_t*>(static_cast<uintptr_t>(1) << 21);

const int kSizes[] = {INT_MIN, -1, 0, 1, 2, 7, 64, 65535, 65536, 16777215, 16777216, INT_MAX};

std::vector<kvarn_config> all_configs() {
  std::vector<kvarn_config> v;
  for (int d : {64, 128, 256})
    for (int kb : {4, 8})
      for (int vb : {2, 4})
        for (int g : {64, 128}) v.push_back(kvarn_config{d, 128, kb, vb, g, 4, 1e-6f});
  return v;
}

void test_parse() {
  const char* good[] = {"kvarn_k4v2_g128", "kvarn_k4v2_g64", "kvarn_k8v4_g128", "kvarn_k8v2_g64", "kvarn_k4v4_g128"};
  for (const char* n : good) {
    kvarn_config c{};
    check(kvarn_host::parse_config(n, &c) == KVARN_OK && c.head_dim == 128 && c.block_tokens == 128 &&
              c.norm_iters == 4,
          "parse good name");
  }
  const char* bad[] = {"", "kvarn", "kvarn_k4v2_g128 ", "kvarn_k4v2_g128x", "kvarn_k3v2_g128", "kvarn_k4v3_g128",
                       "kvarn_k4v2_g32", "kvarn_k-4v2_g128", "kvarn_k4v2_g", "KVARN_K4V2_G128", "fp8"};
  for (const char* n : bad) {
    kvarn_config c{};
    check(kvarn_host::parse_config(n, &c) == KVARN_ERR_UNSUPPORTED, "parse bad name");
  }
  std::string longname(4096, 'k');
  kvarn_config c{};
  check(kvarn_host::parse_config(longname.c_str(), &c) == KVARN_ERR_UNSUPPORTED, "parse long name");
  check(kvarn_host::parse_config(nullptr, &c) == KVARN_ERR_NULL, "parse NULL name");
  check(kvarn_host::parse_config("kvarn_k4v2_g128", nullptr) == KVARN_ERR_NULL, "parse NULL out");
}

void test_configs_and_pages() {
  // bytes of the page layouts: codes, fp16 scale + zero per group, rho fp32[128], gamma fp32[D]
  kvarn_config c{128, 128, 4, 2, 128, 4, 1e-6f};
  check(kvarn_host::page_bytes(&c, false) == 8192 + 512 + 512 + 512, "K page k4 g128 D128");
  check(kvarn_host::page_bytes(&c, true) == 4096 + 512 + 512 + 512, "V page v2 g128 D128");
  c.group_size = 64;
  check(kvarn_host::page_bytes(&c, false) == 8192 + 1024 + 512 + 512, "K page k4 g64 D128");
  c = kvarn_config{64, 128, 4, 2, 128, 4, 1e-6f};
  check(kvarn_host::page_bytes(&c, true) == 2048 + 512 + 512 + 256, "V page v2 g128 D64 (64-channel groups)");
  c = kvarn_config{256, 128, 8, 4, 64, 4, 1e-6f};
  check(kvarn_host::page_bytes(&c, false) == 32768 + 2 * 256 * 4 + 512 + 1024, "K page k8 g64 D256");
  check(kvarn_host::page_bytes(&c, true) == 16384 + 4 * 128 * 4 + 512 + 1024, "V page v4 g64 D256");
  for (const kvarn_config& g : all_configs()) {
    check(kvarn_host::check_config(&g) == KVARN_OK, "config ok");
    check((kvarn_host::check_config_128(&g) == KVARN_OK) == (g.head_dim == 128), "config 128");
    check(kvarn_host::page_bytes(&g, false) % 16 == 0 && kvarn_host::page_bytes(&g, true) % 16 == 0,
          "pages keep 16-byte alignment");
  }
  kvarn_config bad[] = {{96, 128, 4, 2, 128, 4, 1e-6f}, {128, 64, 4, 2, 128, 4, 1e-6f}, {128, 128, 2, 2, 128, 4, 1e-6f},
                        {128, 128, 4, 8, 128, 4, 1e-6f}, {128, 128, 4, 2, 32, 4, 1e-6f}, {128, 128, 4, 2, 128, 3, 1e-6f},
                        {128, 128, 4, 2, 128, 4, 1e-5f}, {INT_MIN, INT_MIN, INT_MIN, INT_MIN, INT_MIN, INT_MIN, -1.f}};
  for (const kvarn_config& g : bad) {
    check(kvarn_host::check_config(&g) == KVARN_ERR_UNSUPPORTED, "bad config rejected");
    check(kvarn_host::page_bytes(&g, false) == 0 && kvarn_host::page_bytes(&g, true) == 0, "bad config: 0 bytes");
  }
  check(kvarn_host::check_config(nullptr) == KVARN_ERR_NULL, "NULL config");
  check(kvarn_host::page_bytes(nullptr, true) == 0, "NULL config bytes");
}

// The plan's promises to the decode kernels, for one shape.
void check_plan(int batch, int hkv, int mb, int cus, bool tail) {
  const kvarn_host::DecodePlan p = kvarn_host::plan_decode(batch, hkv, mb, cus, tail);
  const int page_splits = p.max_splits - (tail ? 1 : 0);
  check(p.blocks_per_split >= 4 && p.blocks_per_split % 4 == 0, "plan: pages per split a multiple of 4", batch, hkv, mb);
  check(p.max_splits >= 1 && p.max_splits <= kvarn_host::kMaxSplitsPerPair, "plan: at most 64 splits", batch, hkv, mb);
  check(static_cast<long>(page_splits) * p.blocks_per_split >= mb, "plan: splits cover every page", batch, hkv, mb);
  check(page_splits <= 1 || static_cast<long>(page_splits - 1) * p.blocks_per_split < mb, "plan: no empty split",
        batch, hkv, mb);
  const long cap = (static_cast<long>(mb) + 62) / 63;  // pages per split forced by the split cap
  check(p.blocks_per_split <= 32 || p.blocks_per_split <= (cap + 3) / 4 * 4, "plan: at most 32 pages per split "
        "unless the split cap needs more", batch, hkv, mb);
  const size_t ws = kvarn_host::workspace_bytes(batch, hkv, mb, 128, cus);
  check(ws >= kvarn_host::counter_bytes(batch, hkv) + kvarn_host::partial_bytes(batch, hkv, p.max_splits, 128),
        "plan: workspace holds the plan's partials", batch, hkv, mb);
}

void test_plans() {
  for (int cus : {1, 32, 80, 256, 304, 100000})
    for (int batch : {1, 2, 3, 16, 64, 128, 1000})
      for (int hkv : {1, 2, 8, 64})
        for (int mb = 1; mb <= 1100; mb += (mb < 80 ? 1 : 37))
          for (bool tail : {false, true}) check_plan(batch, hkv, mb, cus, tail);
  // the largest shapes validation lets through
  for (bool tail : {false, true}) {
    check_plan(65535, 65535, 16777215, 256, tail);
    check_plan(1, 1, 16777215, 256, tail);
    check_plan(65535, 1, 1, 1, tail);
  }
  // 16 sequences x 8 KV heads x 64 pages: 768 workgroups; 64 x 2 x 32: 512 (256 CUs); 32 CUs: 128
  kvarn_host::DecodePlan p = kvarn_host::plan_decode(16, 8, 64, 256);
  check(p.blocks_per_split == 12 && p.max_splits == 6, "plan: 16 x 8 heads x 64 pages");
  p = kvarn_host::plan_decode(64, 2, 32, 256);
  check(p.blocks_per_split == 8 && p.max_splits == 4, "plan: 64 x 2 heads x 32 pages");
  p = kvarn_host::plan_decode(64, 2, 32, 32);
  check(p.blocks_per_split == 32 && p.max_splits == 1, "plan: 32 CUs");
  // the kernel choice: two workgroups per CU with prefetch while splits stay at 16 pages or fewer
  kvarn_host::DecodeChoice c = kvarn_host::choose_decode(64, 2, 32, 256, false, true);
  check(c.prefetch && c.plan.blocks_per_split == 8 && c.plan.max_splits == 4, "choice: 64 x 2 x 32 prefetches");
  c = kvarn_host::choose_decode(128, 8, 256, 256, false, true);
  check(!c.prefetch && c.plan.blocks_per_split == 32 && c.plan.max_splits == 8, "choice: long splits stream");
  c = kvarn_host::choose_decode(16, 8, 64, 256, false, false);
  check(!c.prefetch && c.plan.blocks_per_split == 12, "choice: format without a prefetching kernel");
  // one 131,072-token sequence: 64 splits of 16 pages; with an fp16 tail the 63-split cap makes them 20
  c = kvarn_host::choose_decode(1, 8, 1024, 256, false, true);
  check(c.prefetch && c.plan.blocks_per_split == 16 && c.plan.max_splits == 64, "choice: one long sequence");
  c = kvarn_host::choose_decode(1, 8, 1024, 256, true, true);
  check(!c.prefetch && c.plan.blocks_per_split == 20 && c.plan.max_splits == 53, "choice: one long sequence, tail");
  // every choice fits the workspace
  for (int cus : {32, 256, 304})
    for (int batch : {1, 3, 64, 1000})
      for (int mb = 1; mb <= 700; mb += 23)
        for (bool tail : {false, true})
          for (bool can : {false, true}) {
            c = kvarn_host::choose_decode(batch, 8, mb, cus, tail, can);
            check(kvarn_host::workspace_bytes(batch, 8, mb, 128, cus) >=
                      kvarn_host::counter_bytes(batch, 8) + kvarn_host::partial_bytes(batch, 8, c.plan.max_splits, 128),
                  "choice fits the workspace", batch, mb, cus);
          }
}

void test_quantize() {
  const kvarn_config cfg{128, 128, 4, 2, 128, 4, 1e-6f};
  bool run = true;
  check(kvarn_host::validate_quantize(&cfg, kAligned, kAligned, 4, 8, kTable, kAligned, kAligned, 10, &run) ==
            KVARN_OK && run, "quantize ok");
  check(kvarn_host::validate_quantize(&cfg, kAligned, kAligned, 0, 8, nullptr, nullptr, nullptr, 0, &run) ==
            KVARN_OK && !run, "quantize zero blocks is a no-op");
  check(kvarn_host::validate_quantize(&cfg, nullptr, kAligned, 4, 8, kTable, kAligned, kAligned, 10, &run) ==
            KVARN_ERR_NULL, "quantize NULL k");
  check(kvarn_host::validate_quantize(&cfg, kAligned, kAligned, 4, 8, kTable, kOdd, kAligned, 10, &run) ==
            KVARN_ERR_SHAPE, "quantize misaligned pool");
  check(kvarn_host::validate_quantize(&cfg, kOdd, kAligned, 4, 8, kTable, kAligned, kAligned, 10, &run) ==
            KVARN_ERR_SHAPE, "quantize misaligned k");
  check(kvarn_host::validate_quantize(&cfg, kAligned, kAligned, INT_MAX, INT_MAX, kTable, kAligned, kAligned, 10,
                                      &run) == KVARN_ERR_SHAPE, "quantize too many tiles");
  check(kvarn_host::validate_quantize(&cfg, kAligned, kAligned, 4, 8, kTable, kAligned, kAligned, 0, &run) ==
            KVARN_ERR_SHAPE, "quantize no pages");
  check(kvarn_host::validate_quantize(nullptr, kAligned, kAligned, 4, 8, kTable, kAligned, kAligned, 10, &run) ==
            KVARN_ERR_NULL, "quantize NULL config");
  for (const kvarn_config& c : all_configs())
    for (int n : kSizes)
      for (int h : kSizes)
        for (int np : kSizes)
          for (const void* pk : {kAligned, kOdd, static_cast<const void*>(nullptr)}) {
            run = false;
            const kvarn_status s = kvarn_host::validate_quantize(&c, pk, kAligned, n, h, kTable, kAligned, kAligned, np,
                                                                 &run);
            check(valid_status(s), "quantize status", n, h, np);
            if (run)
              check(s == KVARN_OK && n > 0 && h > 0 && np > 0 && static_cast<long>(n) * h * 2 <= INT_MAX &&
                        pk == kAligned,
                    "quantize launches only valid shapes", n, h, np);
          }
}

void test_dequantize() {
  const kvarn_config cfg{64, 128, 4, 2, 128, 4, 1e-6f};
  const float* fo = static_cast<const float*>(kAligned);
  bool run = true;
  check(kvarn_host::validate_dequantize(&cfg, kAligned, kAligned, 5, kTable, 3, 2, fo, nullptr, &run) == KVARN_OK &&
            run, "dequantize K only");
  check(kvarn_host::validate_dequantize(&cfg, nullptr, kAligned, 5, kTable, 3, 2, nullptr, fo, &run) == KVARN_OK && run,
        "dequantize V only needs no K pool");
  check(kvarn_host::validate_dequantize(&cfg, kAligned, kAligned, 5, kTable, 3, 2, nullptr, nullptr, &run) ==
            KVARN_OK && !run, "dequantize with no output is a no-op");
  check(kvarn_host::validate_dequantize(&cfg, nullptr, kAligned, 5, kTable, 3, 2, fo, nullptr, &run) == KVARN_ERR_NULL,
        "dequantize K without K pool");
  for (int n : kSizes)
    for (int h : kSizes)
      for (int np : kSizes) {
        run = false;
        const kvarn_status s = kvarn_host::validate_dequantize(&cfg, kAligned, kAligned, np, kTable, n, h, fo, fo, &run);
        check(valid_status(s), "dequantize status", n, h, np);
        if (run)
          check(n > 0 && h > 0 && np > 0 && static_cast<long>(n) * h * 2 <= INT_MAX, "dequantize launches only valid "
                "shapes", n, h, np);
      }
}

void test_decode() {
  const float* fo = static_cast<const float*>(kAligned);
  const kvarn_config c128{128, 128, 4, 2, 128, 4, 1e-6f};
  const kvarn_config c64{64, 128, 4, 2, 128, 4, 1e-6f};
  auto args = [&](kvarn_host::DecodeKind kind, const kvarn_config* cfg, int batch, int nq, int hkv, int mb) {
    kvarn_host::DecodeArgs a{};
    a.kind = kind;
    a.cfg = cfg;
    a.q = kAligned;
    a.k_pool = kAligned;
    a.v_pool = kAligned;
    a.num_pages = 100;
    a.block_table = kTable;
    a.max_blocks = mb;
    a.seq_lens = kTable;
    a.k_tail = kAligned;
    a.v_tail = kAligned;
    a.batch = batch;
    a.num_q_heads = nq;
    a.num_kv_heads = hkv;
    a.out = fo;
    a.workspace = kAligned;
    a.ws_bytes = SIZE_MAX;
    a.use_scratch = false;
    a.cus = 256;
    return a;
  };
  bool run = false;
  kvarn_host::DecodeChoice p{};
  using K = kvarn_host::DecodeKind;
  kvarn_host::DecodeArgs a = args(K::packed, &c128, 16, 32, 8, 64);
  // 16 x 8 heads x 64 pages at two workgroups per CU: 16 pages per split, short enough to prefetch
  check(kvarn_host::validate_decode(a, &run, &p) == KVARN_OK && run && p.prefetch && p.plan.blocks_per_split == 16 &&
            p.plan.max_splits == 4,
        "decode ok");
  a.ws_bytes = kvarn_host::workspace_bytes(16, 8, 64, 128, 256);
  check(kvarn_host::validate_decode(a, &run, &p) == KVARN_OK && run, "decode with the exact workspace");
  a.ws_bytes -= 1;
  check(kvarn_host::validate_decode(a, &run, &p) == KVARN_ERR_WORKSPACE, "decode workspace one byte short");
  a = args(K::packed, &c128, 16, 32, 8, 64);
  a.workspace = kOdd;
  check(kvarn_host::validate_decode(a, &run, &p) == KVARN_ERR_WORKSPACE, "decode misaligned workspace");
  a = args(K::packed, &c128, 16, 36, 4, 64);
  check(kvarn_host::validate_decode(a, &run, &p) == KVARN_ERR_UNSUPPORTED, "decode 9 query heads per KV head");
  a = args(K::packed, &c128, 16, 30, 4, 64);
  check(kvarn_host::validate_decode(a, &run, &p) == KVARN_ERR_SHAPE, "decode heads not a multiple");
  a = args(K::packed_tail, &c64, 16, 32, 8, 64);
  check(kvarn_host::validate_decode(a, &run, &p) == KVARN_ERR_UNSUPPORTED, "tail decode needs head_dim 128");
  // 64-channel heads: two workgroups per CU (512 on 256 CUs: 16 pages per split for 16 x 8 x 64)
  a = args(K::packed, &c64, 16, 32, 8, 64);
  check(kvarn_host::validate_decode(a, &run, &p) == KVARN_OK && run && !p.prefetch && p.plan.blocks_per_split == 16 &&
            p.plan.max_splits == 4,
        "decode plan at 64 channels");
  a = args(K::packed_tail, &c128, 16, 32, 8, 64);
  a.v_tail = nullptr;
  check(kvarn_host::validate_decode(a, &run, &p) == KVARN_ERR_NULL, "tail decode without v_tail");
  a = args(K::packed, &c128, 0, 32, 8, 64);
  a.q = nullptr;
  check(kvarn_host::validate_decode(a, &run, &p) == KVARN_OK && !run, "decode of an empty batch is a no-op");
  a = args(K::packed, &c128, 16, 32, 8, 0);
  a.block_table = nullptr;
  a.k_pool = a.v_pool = nullptr;
  a.num_pages = 0;
  check(kvarn_host::validate_decode(a, &run, &p) == KVARN_OK && run, "decode with no pages at all");
  // the allocation-free variant's fixed limits
  a = args(K::packed, &c128, 65535, 8, 8, 8);
  a.use_scratch = true;
  a.workspace = nullptr;
  a.ws_bytes = 0;
  check(kvarn_host::validate_decode(a, &run, &p) == KVARN_ERR_WORKSPACE, "no-alloc: too many counters");
  a = args(K::packed, &c128, 64, 16, 2, 32);
  a.use_scratch = true;
  a.workspace = nullptr;
  check(kvarn_host::validate_decode(a, &run, &p) == KVARN_OK && run, "no-alloc: a 64 x 4096 step fits");
  a = args(K::packed, &c128, 2048, 64, 8, 1024);
  a.use_scratch = true;
  a.workspace = nullptr;
  check(kvarn_host::validate_decode(a, &run, &p) == KVARN_ERR_WORKSPACE, "no-alloc: partials above 63 MiB");

  const int heads[][2] = {{1, 1}, {8, 1}, {9, 1}, {6, 2}, {7, 2}, {32, 8}, {INT_MAX, 1}, {1, INT_MAX}, {INT_MIN, 1},
                          {8, INT_MIN}, {0, 1}, {1, 0}};
  for (K kind : {K::packed, K::packed_tail, K::fp16})
    for (bool scratch : {false, true})
      for (int batch : kSizes)
        for (const auto& hh : heads)
          for (int mb : kSizes)
            for (int cus : {0, 32, 256, INT_MAX}) {
              a = args(kind, &c128, batch, hh[0], hh[1], mb);
              a.use_scratch = scratch;
              a.cus = cus;
              run = false;
              const kvarn_status s = kvarn_host::validate_decode(a, &run, &p);
              check(valid_status(s), "decode status", batch, hh[0], mb);
              if (!run) continue;
              check(s == KVARN_OK && batch > 0 && batch <= 65535 && hh[1] > 0 && hh[1] <= 65535 && mb >= 0 &&
                        static_cast<long>(mb) * 128 + 127 <= INT_MAX && hh[0] % hh[1] == 0 && hh[0] / hh[1] <= 8,
                    "decode launches only valid shapes", batch, hh[0], mb);
              check(p.plan.blocks_per_split % 4 == 0 && p.plan.max_splits >= 1 && p.plan.max_splits <= 64 &&
                        static_cast<long>(p.plan.max_splits - (kind == K::packed_tail ? 1 : 0)) *
                                p.plan.blocks_per_split >= (mb > 0 ? mb : 1),
                    "decode plan", batch, hh[0], mb);
              check(!p.prefetch || (kind != K::fp16 && p.plan.blocks_per_split <= 16), "prefetch only for short "
                    "packed splits", batch, hh[0], mb);
              if (scratch)
                check(kvarn_host::partial_bytes(batch, hh[1], p.plan.max_splits, 128) <=
                          kvarn_host::kScratchBytes - kvarn_host::kScratchCounterBytes,
                      "no-alloc partials fit", batch, hh[0], mb);
            }
  // the workspace query never overflows and is 0 exactly where decode would refuse the sizes
  for (const kvarn_config& c : all_configs())
    for (int batch : kSizes)
      for (const auto& hh : heads)
        for (int mb : kSizes) {
          const size_t ws = kvarn_host::decode_workspace_bytes(&c, batch, hh[0], hh[1], mb, 256);
          const bool in_range = batch > 0 && hh[0] > 0 && hh[1] > 0 && mb >= 0 &&
                                kvarn_host::decode_sizes_in_range(batch, hh[1], mb);
          check((ws > 0) == in_range, "workspace query", batch, hh[1], mb);
        }
}

void test_prefill() {
  const kvarn_config cfg{128, 128, 4, 2, 128, 4, 1e-6f};
  const float* fo = static_cast<const float*>(kAligned);
  bool run = false;
  check(kvarn_host::validate_prefill(&cfg, kAligned, 128, kAligned, kAligned, 10, kTable, 4, kTable, kAligned, kAligned,
                                     128, kTable, kTable, 2, 32, 8, fo, &run) == KVARN_OK && run, "prefill ok");
  check(kvarn_host::validate_prefill(&cfg, kAligned, 128, kAligned, kAligned, 10, kTable, 4, kTable, nullptr, kAligned,
                                     128, kTable, kTable, 2, 32, 8, fo, &run) == KVARN_ERR_NULL, "prefill NULL k_new");
  check(kvarn_host::validate_prefill(&cfg, kAligned, 128, kAligned, kAligned, 10, kTable, 4, kTable, nullptr, nullptr,
                                     0, kTable, kTable, 2, 32, 8, fo, &run) == KVARN_OK && run,
        "prefill over the pages alone");
  const kvarn_config c256{256, 128, 4, 2, 128, 4, 1e-6f};
  check(kvarn_host::validate_prefill(&c256, kAligned, 128, kAligned, kAligned, 10, kTable, 4, kTable, kAligned,
                                     kAligned, 128, kTable, kTable, 2, 32, 8, fo, &run) == KVARN_ERR_UNSUPPORTED,
        "prefill needs head_dim 128");
  for (int batch : kSizes)
    for (int mq : kSizes)
      for (int mb : kSizes)
        for (int mn : {INT_MIN, -1, 0, 1, INT_MAX}) {
          run = false;
          const kvarn_status s = kvarn_host::validate_prefill(&cfg, kAligned, mq, kAligned, kAligned, 10, kTable, mb,
                                                              kTable, kAligned, kAligned, mn, kTable, kTable, batch, 32,
                                                              8, fo, &run);
          check(valid_status(s), "prefill status", batch, mq, mb);
          if (run)
            check(batch > 0 && batch <= 65535 && mq > 0 && mn >= 0 && mb >= 0 &&
                      static_cast<long>(mb) * 128 + 127 <= INT_MAX,
                  "prefill launches only valid shapes", batch, mq, mb);
        }
}

}  // namespace

int main() {
  test_parse();
  test_configs_and_pages();
  test_plans();
  test_quantize();
  test_dequantize();
  test_decode();
  test_prefill();
  std::printf("host self-test: %ld checks, %ld failed\n", g_checks, g_failures);
  return g_failures == 0 ? 0 : 1;
}
