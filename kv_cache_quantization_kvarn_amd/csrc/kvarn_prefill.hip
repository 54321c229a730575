// Chunked-prefill attention over the packed KVarN cache for gfx950.
//
// A sequence holds prefix_len / 128 packed blocks (pages of its block-table row) and then new_len
// fp16 rows: the chunk being prefilled, whose blocks are quantised only once whole (KVarN blog
// post, section "KVarN Nasıl Çalışır?").  Its queries are the last q_len of those rows: query i sits
// at fp16 row new_len - q_len + i and attends to every packed token and, causally, to the fp16 rows
// up to its own.
//
// A workgroup of eight waves takes 128 (query token, head) rows of one (sequence, KV head): 128 / G
// query tokens times the G heads that share the KV head.  Wave w owns rows 16w .. 16w + 15, one
// 16-column tile of v_mfma_f32_16x16x32_f16.  The KV blocks stream through LDS once per workgroup:
//
//   * a packed page is loaded by all 512 lanes (the next page's loads are in flight while the
//     current one is attended) and its codes are written to LDS as exact fp16 integers (up to 255
//     for 8-bit keys: normal numbers or zero, which the matrix cores multiply exactly, so no offset
//     has to be removed), keys as [token][channel] rows and values as [channel][token] rows, the
//     16-byte chunks of a row XOR-swizzled so that the 16 lanes of a fragment read hit distinct
//     banks;
//   * the page metadata becomes per-channel and per-token factors, and both products run with the
//     codes as the A operand and the fp32 coefficients as an fp16 hi + lo pair of B operands (two
//     products into one fp32 accumulator):
//
//       score_rt = 2^rho_t ( sum_j a_rj c_tj + b_r ), a_rj = q~_rj 2^gamma_j s_j, b_r = sum_j q~_rj 2^gamma_j z_j
//       o_rj    += 2^gamma_j ( sum_t w_rt c_tj + u_r ), w_rt = p_rt 2^rho_t s_t, u_r = sum_t p_rt 2^rho_t z_t
//
//     in the rotated basis (q~ = H q; the rotation is orthonormal and keeps scores, same section);
//     b_r and u_r enter as the accumulator input of each product chain;
//   * after the packed pages o is rotated back to the original basis in registers, and the fp16
//     rows follow in blocks of 128 through the same LDS layout (keys copied, values transposed),
//     with unit factors, the raw query and the causal mask.
//
// Online softmax in log2 units over all blocks; the output is fp32 in the original basis.  The kernel
// is instantiated per code widths and group size; with group size 64 the scale and zero differ between
// the token halves of a key group and the channel halves of a value group, so the score products run
// once per token half (a lane keeps the half its rows belong to) and each channel half of the value
// products takes its own weights.
#include "kvarn_common.h"

namespace kvarn {

namespace {

constexpr int kPfWaves = 8;
constexpr int kPfThreads = 64 * kPfWaves;
constexpr int kCt = 1;                          // 16-column MFMA tiles (16 rows each) per wave
constexpr int kPfRows = 16 * kCt * kPfWaves;    // (query token, head) rows per workgroup
constexpr int kMetaWords = MetaLayout<64>::kBytes / 4;  // room for either group size

// Page geometry of a format (key / value code widths, group size).
template <int KB, int VB, int GS>
struct PfFormat {
  using Meta = MetaLayout<GS>;
  static constexpr int kHalves = Meta::kHalves;
  static constexpr int kKCode = kBlockTokens * kHeadDim * KB / 8;  // key code bytes
  static constexpr int kVCode = kBlockTokens * kHeadDim * VB / 8;  // value code bytes
  static constexpr int kKPage = kKCode + Meta::kBytes, kVPage = kVCode + Meta::kBytes;
  static constexpr int kKCodeChunks = kKCode / 16, kVCodeChunks = kVCode / 16;
  static constexpr int kKChunks = kKPage / 16;                  // key page, 16-byte chunks
  static constexpr int kChunks = (kKPage + kVPage) / 16;        // both pages
  static constexpr int kRawPerThread = (kChunks + kPfThreads - 1) / kPfThreads;
};
constexpr int kF16Chunks = kBlockTokens * kHeadDim / 8;                         // 2048 per fp16 block
constexpr int kF16PerThread = (kF16Chunks + kPfThreads - 1) / kPfThreads;
static_assert(kPfThreads >= 2 * kHeadDim, "the factor step gives every channel and token a thread");

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

struct __align__(16) PfLds {
  u32x4 kf[kBlockTokens * 16];  // keys: token row t, chunk c (8 channel slots) at 16t + (c ^ kkey(t))
  u32x4 vf[kHeadDim * 16];      // values: channel row j, chunk c (8 token slots) at 16j + (c ^ (j & 15))
  uint32_t kmeta[kMetaWords];   // the page's raw key / value metadata
  uint32_t vmeta[kMetaWords];
  // [0] only for group size 128; [h] of group size 64: the key groups over token half h, the value
  // groups over channel half h
  float ep[2][kHeadDim];        // per channel: key 2^gamma s * sa
  float fz[2][kHeadDim];        // per channel: key 2^gamma z
  float gs[kHeadDim];           // per channel: value 2^gamma / sw
  float pk[kBlockTokens];       // per token: key 2^rho / sa
  float fv[2][kBlockTokens];    // per token: value 2^rho s * sw
  float zv[2][kBlockTokens];    // per token: value 2^rho z
  float sa, sw;                 // the block's power-of-two coefficient scales
  float qmax[kPfWaves];         // per wave: max |query coefficient| of the current phase
};

// Swizzle key of a key row: the 16 lanes of a score fragment read tokens 32(n/4) + 4mt + n%4, whose
// keys are exactly n = 0..15.
__device__ __forceinline__ int kkey(int t) { return (t & 3) | ((t >> 3) & 12); }

// Slot order inside a key chunk (channels 8c .. 8c+7): slot s holds channel 8c + kslot(s).
//   kslot = 0, 4, 1, 5, 2, 6, 3, 7
// Slot order inside a value chunk c (tokens of 16-token word c/2, half c%2):
//   slot s holds token 16(c/2) + 4(c%2) + {0, 8, 1, 9, 2, 10, 3, 11}[s].

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// Two codes placed at bits 0.. and 16.. of a dword under the fp16 pattern of 1024 (where the ulp is
// 1) read 1024 + c exactly; subtracting 1024 in packed fp16 leaves the exact integers.
__device__ __forceinline__ uint32_t code_pair(uint32_t x, uint32_t mask) {
  const uint32_t biased = (x & mask) | 0x64006400u;
  const f16x2 c = __builtin_bit_cast(f16x2, biased) - f16x2{static_cast<_Float16>(1024.0f), static_cast<_Float16>(1024.0f)};
  return __builtin_bit_cast(uint32_t, c);
}

// hi = nearest fp16 of x0*y0 and x1*y1 (round to nearest even, subnormals kept), lo = nearest fp16
// of the exact residual; hi is pinned so that the stored and the subtracted value are one value.
__device__ __forceinline__ void split2(float x0, float y0, float x1, float y1, uint32_t& hi, uint32_t& lo) {
  f16x2 h = {static_cast<_Float16>(x0 * y0), static_cast<_Float16>(x1 * y1)};
  asm("" : "+v"(h));
  const f16x2 l = {static_cast<_Float16>(__builtin_fmaf(x0, y0, -static_cast<float>(h[0]))),
                   static_cast<_Float16>(__builtin_fmaf(x1, y1, -static_cast<float>(h[1])))};
  hi = __builtin_bit_cast(uint32_t, h);
  lo = __builtin_bit_cast(uint32_t, l);
}

// Lanes l and l ^ 16 (l ^ 32): v_permlane16_swap / v_permlane32_swap on two copies return the pair
// (lower lane's value, upper lane's value) in both lanes.
__device__ __forceinline__ float sum16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// 128-point Sylvester transform (unnormalised) of rows held 32 values per lane, a row in lanes
// n, n + 16, n + 32, n + 48: five bits of the channel index are bits of the array index, the other
// two are lane bits 4 and 5.  Every stage maps a pair differing in one bit to (sum, difference).
__device__ __forceinline__ void fwht_rows(float (&v)[32], int lane) {
#pragma unroll
  for (int bit = 1; bit < 32; bit <<= 1)
#pragma unroll
    for (int i = 0; i < 32; ++i)
      if (!(i & bit)) {
        const float a = v[i], c = v[i | bit];
        v[i] = a + c;
        v[i | bit] = a - c;
      }
  const float s16 = (lane & 16) ? -1.f : 1.f, s32 = (lane & 32) ? -1.f : 1.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[i]), __float_as_uint(v[i]), false, false);
    v[i] = fmaf(s16, __uint_as_float(r[1]), __uint_as_float(r[0]));
  }
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[i]), __float_as_uint(v[i]), false, false);
    v[i] = fmaf(s32, __uint_as_float(r[1]), __uint_as_float(r[0]));
  }
}

// Scale 2^(14 - e) that brings values of magnitude < x (x = f 2^e, f in [0.5, 1)) below 2^14, and
// its inverse; unit scale when x is 0 (all coefficients are then zero, the constants are not).
__device__ __forceinline__ void page_scale(float x, float& s, float& inv) {
  int e;
  frexpf(x, &e);
  e = min(max(e, -100), 100);
  const bool live = x > 0.f;
  s = live ? pow2i(14 - e) : 1.f;
  inv = live ? pow2i(e - 14) : 1.f;
}

// Per-wave state: the lane's rows (column n of each of the wave's tiles).
struct PfState {
  float qv[kCt][32];  // query coefficient of channel 32(i/8) + 8g + i%8 (scaled; rotated in the packed phase)
  float o[kCt][32];   // output accumulator of channel 16(i/4) + 4g + i%4
  float m[kCt];       // running maximum (log2 units), identical in the row's four lanes
  float l[kCt];       // this lane's share of the running sum
};

// ---------------------------------------------------------------------------------------------
// Staging of one block into LDS
// ---------------------------------------------------------------------------------------------

// The 16-byte chunks of a key page and a value page (960 for k4v2): thread tid takes chunks tid,
// tid + T, tid + 2T, ... (T threads per workgroup); key-page chunks come first.
template <class F>
struct PageRaw {
  u32x4 c[F::kRawPerThread];
};

template <class F>
__device__ __forceinline__ void load_page_raw(PageRaw<F>& R, const uint8_t* __restrict__ kp,
                                              const uint8_t* __restrict__ vp, int tid) {
  asm volatile("" : "+v"(tid));
#pragma unroll
  for (int k = 0; k < F::kRawPerThread; ++k) {
    const int id = tid + kPfThreads * k;
    if (id < F::kKChunks) {
      R.c[k] = *reinterpret_cast<const u32x4*>(kp + 16 * id);
    } else if (id < F::kChunks) {
      R.c[k] = *reinterpret_cast<const u32x4*>(vp + 16 * (id - F::kKChunks));
    }
  }
}

// A pair of 8-bit codes (bytes at bits 0..7 and 16..23 of x) as exact fp16 integers.
__device__ __forceinline__ uint32_t byte_pair(uint32_t x) {
  const uint32_t biased = (x & 0x00FF00FFu) | 0x64006400u;
  const f16x2 c = __builtin_bit_cast(f16x2, biased) - f16x2{static_cast<_Float16>(1024.0f), static_cast<_Float16>(1024.0f)};
  return __builtin_bit_cast(uint32_t, c);
}

template <class F>
__device__ __forceinline__ void store_page(PfLds& L, const PageRaw<F>& R, int tid) {
  // the store addresses are recomputed for every page (a few integer operations) rather than kept
  // live across the page loop, where registers are short
  asm volatile("" : "+v"(tid));
#pragma unroll
  for (int k = 0; k < F::kRawPerThread; ++k) {
    const int id = tid + kPfThreads * k;
    const u32x4 x = R.c[k];
    constexpr int kc = F::kKCodeChunks, km = F::kKChunks, vc = F::kKChunks + F::kVCodeChunks;
    if (id < kc) {
      if constexpr (F::kKCode == kBlockTokens * kHeadDim / 2) {
        // 4-bit key codes of token t, channels 32q .. 32q + 31 (dword m: channels 8(4q + m) + i at bits 4i)
        const int t = id >> 2, q = id & 3;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          u32x4 p;
          p[0] = code_pair(x[m], 0x000F000Fu);        // channels 0, 4
          p[1] = code_pair(x[m] >> 4, 0x000F000Fu);   // 1, 5
          p[2] = code_pair(x[m] >> 8, 0x000F000Fu);   // 2, 6
          p[3] = code_pair(x[m] >> 12, 0x000F000Fu);  // 3, 7
          L.kf[16 * t + ((4 * q + m) ^ kkey(t))] = p;
        }
      } else {
        // 8-bit key codes of token t, channels 16q .. 16q + 15 (dword m: channels 16q + 4m + i at bits 8i)
        const int t = id >> 3, q = id & 7;
#pragma unroll
        for (int hc = 0; hc < 2; ++hc) {  // chunk 2q + hc: channels 8(2q + hc) + (0, 4, 1, 5, 2, 6, 3, 7)
          const uint32_t lo = x[2 * hc], hi = x[2 * hc + 1];
          u32x4 p;
          p[0] = byte_pair((lo & 0xFFu) | ((hi & 0xFFu) << 16));                 // channels 0, 4
          p[1] = byte_pair(((lo >> 8) & 0xFFu) | (((hi >> 8) & 0xFFu) << 16));   // 1, 5
          p[2] = byte_pair(((lo >> 16) & 0xFFu) | (((hi >> 16) & 0xFFu) << 16)); // 2, 6
          p[3] = byte_pair((lo >> 24) | ((hi >> 24) << 16));                     // 3, 7
          L.kf[16 * t + ((2 * q + hc) ^ kkey(t))] = p;
        }
      }
    } else if (id < km) {
      *reinterpret_cast<u32x4*>(&L.kmeta[4 * (id - kc)]) = x;
    } else if (id < vc) {
      if constexpr (F::kVCode == kBlockTokens * kHeadDim / 4) {
        // 2-bit value codes of channel j, tokens 64h .. 64h + 63 (dword k: token 64h + 16k + m at bits 2m)
        const int v = id - km, j = v >> 1, h = v & 1;
#pragma unroll
        for (int k2 = 0; k2 < 4; ++k2) {
          const uint32_t w = x[k2];
          u32x4 a, b;
#pragma unroll
          for (int pr = 0; pr < 4; ++pr) {
            a[pr] = code_pair(w >> (2 * pr), 0x00030003u);        // tokens pr, pr + 8
            b[pr] = code_pair(w >> (2 * pr + 8), 0x00030003u);    // tokens 4 + pr, 12 + pr
          }
          const int c0 = 2 * (4 * h + k2);
          L.vf[16 * j + (c0 ^ (j & 15))] = a;
          L.vf[16 * j + ((c0 + 1) ^ (j & 15))] = b;
        }
      } else {
        // 4-bit value codes of channel j, tokens 32h .. 32h + 31 (dwords 2u, 2u + 1: tokens 32h + 16u + m
        // at bits 4m of the pair, m = 0..7 in the first dword, 8..15 in the second)
        const int v = id - km, j = v >> 2, h = v & 3;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const uint32_t y0 = x[2 * u], y1 = x[2 * u + 1];
          u32x4 a, b;
#pragma unroll
          for (int pr = 0; pr < 4; ++pr) {
            a[pr] = code_pair(((y0 >> (4 * pr)) & 0xFu) | (((y1 >> (4 * pr)) & 0xFu) << 16), 0x000F000Fu);
            b[pr] = code_pair(((y0 >> (4 * pr + 16)) & 0xFu) | (((y1 >> (4 * pr + 16)) & 0xFu) << 16), 0x000F000Fu);
          }
          const int c0 = 2 * (2 * h + u);
          L.vf[16 * j + (c0 ^ (j & 15))] = a;
          L.vf[16 * j + ((c0 + 1) ^ (j & 15))] = b;
        }
      }
    } else if (id < F::kChunks) {
      *reinterpret_cast<u32x4*>(&L.vmeta[4 * (id - vc)]) = x;
    }
  }
}

// Factors of a packed page (every wave finds the maxima itself; threads 0-127 write the per-channel
// arrays, 128-255 the per-token ones).  Group entries are half-major (entry 128*h + j).
template <int GS>
__device__ __forceinline__ void page_factors(PfLds& L, int tid, int lane) {
  using Meta = MetaLayout<GS>;
  constexpr int NH = Meta::kHalves;
  asm volatile("" : "+v"(tid), "+v"(lane));
  const uint16_t* ksc = reinterpret_cast<const uint16_t*>(L.kmeta) + Meta::kScale / 2;
  const uint16_t* kzr = reinterpret_cast<const uint16_t*>(L.kmeta) + Meta::kZero / 2;
  const float* krho = reinterpret_cast<const float*>(L.kmeta) + Meta::kRho / 4;
  const float* kgam = reinterpret_cast<const float*>(L.kmeta) + Meta::kGamma / 4;
  const uint16_t* vsc = reinterpret_cast<const uint16_t*>(L.vmeta) + Meta::kScale / 2;
  const uint16_t* vzr = reinterpret_cast<const uint16_t*>(L.vmeta) + Meta::kZero / 2;
  const float* vrho = reinterpret_cast<const float*>(L.vmeta) + Meta::kRho / 4;
  const float* vgam = reinterpret_cast<const float*>(L.vmeta) + Meta::kGamma / 4;
  const int i0 = 2 * lane, i1 = 2 * lane + 1;
  float e = 0.f, f = 0.f;
#pragma unroll
  for (int hh = 0; hh < NH; ++hh) {
    e = fmaxf(e, fmaxf(ex2(kgam[i0]) * half_bits_to_float(ksc[128 * hh + i0]),
                       ex2(kgam[i1]) * half_bits_to_float(ksc[128 * hh + i1])));
    f = fmaxf(f, fmaxf(ex2(vrho[i0]) * half_bits_to_float(vsc[128 * hh + i0]),
                       ex2(vrho[i1]) * half_bits_to_float(vsc[128 * hh + i1])));
  }
  const float emax = wave_max(e), fmax = wave_max(f);
  float qmax = 0.f;
#pragma unroll
  for (int x = 0; x < kPfWaves; ++x) qmax = fmaxf(qmax, L.qmax[x]);
  float sa, inv_sa, sw, inv_sw;
  page_scale(qmax * emax, sa, inv_sa);
  page_scale(fmax, sw, inv_sw);
  if (tid < kHeadDim) {
    const int j = tid;
    const float eg = ex2(kgam[j]);
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
      L.ep[hh][j] = eg * half_bits_to_float(ksc[128 * hh + j]) * sa;
      L.fz[hh][j] = eg * half_bits_to_float(kzr[128 * hh + j]);
    }
    L.gs[j] = ex2(vgam[j]) * inv_sw;
  } else if (tid < 2 * kHeadDim) {
    const int t = tid - kHeadDim;
    const float ev = ex2(vrho[t]);
    L.pk[t] = ex2(krho[t]) * inv_sa;
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
      L.fv[hh][t] = ev * half_bits_to_float(vsc[128 * hh + t]) * sw;
      L.zv[hh][t] = ev * half_bits_to_float(vzr[128 * hh + t]);
    }
  }
  if (tid == 0) {
    L.sa = sa;
    L.sw = sw;
  }
}

// fp16 rows r0 .. r0 + 127 of one (sequence, KV head) (row r at base + r * rstride halves); rows at
// or past nrows are stored as zeros.  Keys are copied into the key layout (channel slots reordered),
// values transposed into the value layout.
__device__ __forceinline__ void store_fp16_block(PfLds& L, const uint16_t* __restrict__ kbase,
                                                 const uint16_t* __restrict__ vbase, size_t rstride, int r0,
                                                 int nrows, int tid) {
  asm volatile("" : "+v"(tid));
  _Float16* vh = reinterpret_cast<_Float16*>(L.vf);
#pragma unroll 2
  for (int k = 0; k < kF16PerThread; ++k) {
    const int id = tid + kPfThreads * k;
    if (id >= kF16Chunks) break;
    const int t = id >> 4, c = id & 15;  // token t, channels 8c .. 8c + 7
    const bool live = r0 + t < nrows;
    const size_t off = static_cast<size_t>(live ? r0 + t : 0) * rstride + 8 * c;
    const u32x4 zero = {0u, 0u, 0u, 0u};
    const u32x4 kx = live ? *reinterpret_cast<const u32x4*>(kbase + off) : zero;
    const u32x4 vx = live ? *reinterpret_cast<const u32x4*>(vbase + off) : zero;
    u32x4 p;
    p[0] = (kx[0] & 0xFFFFu) | (kx[2] << 16);          // channels 0, 4
    p[1] = (kx[0] >> 16) | (kx[2] & 0xFFFF0000u);      // 1, 5
    p[2] = (kx[1] & 0xFFFFu) | (kx[3] << 16);          // 2, 6
    p[3] = (kx[1] >> 16) | (kx[3] & 0xFFFF0000u);      // 3, 7
    L.kf[16 * t + (c ^ kkey(t))] = p;
    // token t's slot in every value row: word t/16, pair j = t%8 (second of the pair if t%16 >= 8)
    const int m = t & 15, jp = m & 7;
    const int chunk = 2 * (t >> 4) + (jp >> 2);
    const int slot = 2 * (jp & 3) + (m >> 3);
    const f16x8 vv = __builtin_bit_cast(f16x8, vx);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int j = 8 * c + i;
      vh[8 * (16 * j + (chunk ^ (j & 15))) + slot] = vv[i];
    }
  }
}

// Unit factors of an fp16 block under the scale of the raw query.
__device__ __forceinline__ void fp16_factors(PfLds& L, int tid) {
  float qmax = 0.f;
#pragma unroll
  for (int x = 0; x < kPfWaves; ++x) qmax = fmaxf(qmax, L.qmax[x]);
  float sa, inv_sa, sw, inv_sw;
  page_scale(qmax, sa, inv_sa);
  page_scale(1.0f, sw, inv_sw);
  if (tid < kHeadDim) {
    L.ep[0][tid] = sa;
    L.fz[0][tid] = 0.f;
    L.gs[tid] = inv_sw;
  } else if (tid < 2 * kHeadDim) {
    const int t = tid - kHeadDim;
    L.pk[t] = inv_sa;
    L.fv[0][t] = sw;
    L.zv[0][t] = 0.f;
  }
  if (tid == 0) {
    L.sa = sa;
    L.sw = sw;
  }
}

// ---------------------------------------------------------------------------------------------
// One block against the wave's 16 rows
// ---------------------------------------------------------------------------------------------
static_assert(kCt == 1, "the pipelined block step holds one 16-row tile per wave");

// Online-softmax step over one half of a block: the lane's 16 products sc[lt][r] of tokens
// 32g + 16h + 4lt + r, scaled here by 2^rho / sa and masked past `lim`.  Updates m and the lane's
// share of l; returns the factor that rescales everything accumulated before, the row's value
// offset term (u, times sw) and the value-product B operands of token pairs (lt, lt + 2).
// NH = 2 (group size 64): one B operand and offset term per channel half of the value groups.
template <int NH>
struct HalfOut {
  f16x8 whi[NH][2], wlo[NH][2];
  float alpha, vinit[NH];
};

template <bool kMasked, int NH>
__device__ __forceinline__ HalfOut<NH> softmax_half(PfState& S, const PfLds& L, f32x4 (&sc)[4], int h, int g,
                                                    int lim) {
  HalfOut<NH> R;
  const int t0 = 32 * g + 16 * h;
  float mloc = -INFINITY;
#pragma unroll
  for (int lt = 0; lt < 4; ++lt) {
    const float4 p4 = *reinterpret_cast<const float4*>(&L.pk[t0 + 4 * lt]);
    const float pkv[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float s = sc[lt][r] * pkv[r];
      sc[lt][r] = kMasked && t0 + 4 * lt + r > lim ? -INFINITY : s;
      mloc = fmaxf(mloc, sc[lt][r]);
    }
  }
  mloc = max32(max16(mloc));
  const float m_new = fmaxf(S.m[0], mloc);
  const float m_use = m_new == -INFINITY ? 0.f : m_new;  // nothing visible yet: every weight stays 0
  R.alpha = ex2(S.m[0] - m_use);
  S.m[0] = m_new;
  float lsum = 0.f, usum[NH];
#pragma unroll
  for (int vh = 0; vh < NH; ++vh) usum[vh] = 0.f;
#pragma unroll
  for (int lt = 0; lt < 4; ++lt) {
    float zvv[NH][4];
#pragma unroll
    for (int vh = 0; vh < NH; ++vh) {
      const float4 z4 = *reinterpret_cast<const float4*>(&L.zv[vh][t0 + 4 * lt]);
      zvv[vh][0] = z4.x; zvv[vh][1] = z4.y; zvv[vh][2] = z4.z; zvv[vh][3] = z4.w;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float p = ex2(sc[lt][r] - m_use);
      lsum += p;
#pragma unroll
      for (int vh = 0; vh < NH; ++vh) usum[vh] = fmaf(p, zvv[vh][r], usum[vh]);
      sc[lt][r] = p;
    }
  }
  S.l[0] = fmaf(S.l[0], R.alpha, lsum);
#pragma unroll
  for (int vh = 0; vh < NH; ++vh) {
    R.vinit[vh] = L.sw * sum32(sum16(usum[vh]));
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const float4 fa = *reinterpret_cast<const float4*>(&L.fv[vh][t0 + 4 * hf]);
      const float4 fb = *reinterpret_cast<const float4*>(&L.fv[vh][t0 + 4 * hf + 8]);
      const float fva[4] = {fa.x, fa.y, fa.z, fa.w}, fvb[4] = {fb.x, fb.y, fb.z, fb.w};
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) split2(sc[hf][j], fva[j], sc[hf + 2][j], fvb[j], hi[j], lo[j]);
      R.whi[vh][hf] = __builtin_bit_cast(f16x8, u32x4{hi[0], hi[1], hi[2], hi[3]});
      R.wlo[vh][hf] = __builtin_bit_cast(f16x8, u32x4{lo[0], lo[1], lo[2], lo[3]});
    }
  }
  return R;
}

// The block runs as two halves of 64 tokens (lane g: tokens 32g .. 32g + 15, then 32g + 16 ..
// 32g + 31), each its own online-softmax step, so that matrix products and vector arithmetic of
// different halves interleave in one wave: the half-1 scores run under the half-0 softmax, the
// half-0 value products under the half-1 softmax.  lim: block-relative index of the last key row the
// lane's row may see; kMasked false: every row sees the whole block (packed pages), no mask.
template <bool kMasked, int NH>
__device__ __forceinline__ void attend_block(PfState& S, const PfLds& L, int lane, const int (&lim)[kCt]) {
  asm volatile("" : "+v"(lane));  // fragment addresses are recomputed per block, not kept live
  const int n = lane & 15, g = lane >> 4;
  const float sa = L.sa;

  // ---- b_r over this lane's 32 channels, then over the row's four lanes (per key token half) -------
  float kinit[NH];
#pragma unroll
  for (int hh = 0; hh < NH; ++hh) {
    float b = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const float4 f0 = *reinterpret_cast<const float4*>(&L.fz[hh][32 * ks + 8 * g]);
      const float4 f1 = *reinterpret_cast<const float4*>(&L.fz[hh][32 * ks + 8 * g + 4]);
      const float fz8[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
#pragma unroll
      for (int s = 0; s < 8; ++s) b = fmaf(S.qv[0][8 * ks + s], fz8[s], b);
    }
    kinit[hh] = sa * sum32(sum16(b));
  }

  // ---- coefficient B operands of the four channel steps (slots 2s2, 2s2 + 1: channels s2, s2 + 4) --
  auto coef_ops = [&](int hh, f16x8 (&bhi)[4], f16x8 (&blo)[4]) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const float4 e0 = *reinterpret_cast<const float4*>(&L.ep[hh][32 * ks + 8 * g]);
      const float4 e1 = *reinterpret_cast<const float4*>(&L.ep[hh][32 * ks + 8 * g + 4]);
      const float ep8[8] = {e0.x, e0.y, e0.z, e0.w, e1.x, e1.y, e1.z, e1.w};
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2)
        split2(S.qv[0][8 * ks + s2], ep8[s2], S.qv[0][8 * ks + s2 + 4], ep8[s2 + 4], hi[s2], lo[s2]);
      bhi[ks] = __builtin_bit_cast(f16x8, u32x4{hi[0], hi[1], hi[2], hi[3]});
      blo[ks] = __builtin_bit_cast(f16x8, u32x4{lo[0], lo[1], lo[2], lo[3]});
    }
  };

  // score tile mt: D[token][row], A = key row 32(n/4) + 4mt + n%4; lane (n, g) gets tokens 32g + 4mt + r
  auto key_frag = [&](int mt, int ks) {
    const int t = 32 * (n >> 2) + 4 * mt + (n & 3);
    return __builtin_bit_cast(f16x8, L.kf[16 * t + ((4 * ks + g) ^ n)]);
  };
  // value tile mt: D[channel][row], A = value row 16mt + n, token chunk 4g + c (c = 2 * half + hf)
  auto val_frag = [&](int mt, int c) {
    const int j = 16 * mt + n;
    return __builtin_bit_cast(f16x8, L.vf[16 * j + ((4 * g + c) ^ n)]);
  };

  f32x4 s0[4], s1[4], d[8];
  if constexpr (NH == 1) {
    f16x8 bhi[4], blo[4];
    coef_ops(0, bhi, blo);
    // ---- half 0 scores ---------------------------------------------------------------------------
#pragma unroll
    for (int lt = 0; lt < 4; ++lt) {
      s0[lt] = f32x4{kinit[0], kinit[0], kinit[0], kinit[0]};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const f16x8 a = key_frag(lt, ks);
        s0[lt] = mfma16x16x32(a, bhi[ks], s0[lt]);
        s0[lt] = mfma16x16x32(a, blo[ks], s0[lt]);
      }
    }
    // ---- half 1 scores, with the half-0 softmax -----------------------------------------------------
#pragma unroll
    for (int lt = 0; lt < 4; ++lt) {
      s1[lt] = f32x4{kinit[0], kinit[0], kinit[0], kinit[0]};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const f16x8 a = key_frag(4 + lt, ks);
        s1[lt] = mfma16x16x32(a, bhi[ks], s1[lt]);
        s1[lt] = mfma16x16x32(a, blo[ks], s1[lt]);
      }
    }
  } else {
    // Two key token halves: lane group g holds tokens of quarter g, i.e. of half g / 2.  Every score
    // tile is computed with each half's coefficients; groups 2 and 3 keep the second result.
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
      f16x8 bhi[4], blo[4];
      coef_ops(hh, bhi, blo);
#pragma unroll
      for (int lt = 0; lt < 8; ++lt) {
        f32x4 t = {kinit[hh], kinit[hh], kinit[hh], kinit[hh]};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const f16x8 a = key_frag(lt, ks);
          t = mfma16x16x32(a, bhi[ks], t);
          t = mfma16x16x32(a, blo[ks], t);
        }
        f32x4& dst = lt < 4 ? s0[lt & 3] : s1[lt & 3];
        if (hh == 0) {
          dst = t;
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) dst[r] = g >= 2 ? t[r] : dst[r];
        }
      }
    }
  }
  const HalfOut<NH> h0 = softmax_half<kMasked, NH>(S, L, s0, 0, g, lim[0]);

  // ---- half 0 value products, with the half-1 softmax (value M-tiles 4-7 are channel half 1) -------
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) {
    const int vh = NH == 1 ? 0 : (mt >> 2);
    d[mt] = f32x4{h0.vinit[vh], h0.vinit[vh], h0.vinit[vh], h0.vinit[vh]};
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const f16x8 a = val_frag(mt, hf);
      d[mt] = mfma16x16x32(a, h0.whi[vh][hf], d[mt]);
      d[mt] = mfma16x16x32(a, h0.wlo[vh][hf], d[mt]);
    }
  }
  const HalfOut<NH> h1 = softmax_half<kMasked, NH>(S, L, s1, 1, g, lim[0]);

  // ---- half 1 value products on the rescaled half-0 partial --------------------------------------
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) {
    const int vh = NH == 1 ? 0 : (mt >> 2);
#pragma unroll
    for (int r = 0; r < 4; ++r) d[mt][r] = fmaf(d[mt][r], h1.alpha, h1.vinit[vh]);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const f16x8 a = val_frag(mt, 2 + hf);
      d[mt] = mfma16x16x32(a, h1.whi[vh][hf], d[mt]);
      d[mt] = mfma16x16x32(a, h1.wlo[vh][hf], d[mt]);
    }
  }

  // ---- o = alpha o + 2^gamma d --------------------------------------------------------------------
  const float alpha = h0.alpha * h1.alpha;
  if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {
#pragma unroll
    for (int i = 0; i < 32; ++i) S.o[0][i] *= alpha;
  }
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) {
    const float4 g4 = *reinterpret_cast<const float4*>(&L.gs[16 * mt + 4 * g]);
    const float gsv[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
    for (int r = 0; r < 4; ++r) S.o[0][4 * mt + r] = fmaf(d[mt][r], gsv[r], S.o[0][4 * mt + r]);
  }
}

// The lane's query coefficients of one row in channel order 32(i/8) + 8g + i%8, times `scale`; with
// `rotate` the row is first transformed by H (the unnormalised transform; scale carries 2^-3.5).
__device__ __forceinline__ float load_query(float (&qv)[32], const uint16_t* __restrict__ row, bool live, int g,
                                            int lane, bool rotate, float scale) {
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const u32x4 zero = {0u, 0u, 0u, 0u};
    const u32x4 x = live ? *reinterpret_cast<const u32x4*>(row + 32 * ks + 8 * g) : zero;
    const f16x8 h = __builtin_bit_cast(f16x8, x);
#pragma unroll
    for (int s = 0; s < 8; ++s) qv[8 * ks + s] = static_cast<float>(h[s]);
  }
  if (rotate) fwht_rows(qv, lane);
  float mx = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    qv[i] *= scale;
    mx = fmaxf(mx, fabsf(qv[i]));
  }
  return mx;
}

}  // namespace

// One workgroup per (sequence, KV head, tile of qt queries): query i of a sequence sits at fp16 row
// new_len - q_len + i and sees every packed token and the fp16 rows up to its own.
template <int KB, int VB, int GS>
__global__ __launch_bounds__(kPfThreads, 2) void prefill_kernel(
    const uint16_t* __restrict__ q, int max_q, const uint8_t* __restrict__ k_pool, const uint8_t* __restrict__ v_pool,
    int num_pages, const int32_t* __restrict__ block_table, int max_blocks, const int32_t* __restrict__ prefix_lens,
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new, int max_new,
    const int32_t* __restrict__ new_lens, const int32_t* __restrict__ q_lens, int batch, int hq, int hkv, int qt,
    int ntile, float scale_log2, float* __restrict__ out, uint32_t* __restrict__ flags) {
  using F = PfFormat<KB, VB, GS>;
  __shared__ PfLds L;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, n = lane & 15, g = lane >> 4;

  // Workgroups reach the eight XCDs round-robin by linear id: all query tiles of one (sequence, KV
  // head) go to one XCD, consecutively, so its pages are fetched into that XCD's L2 once.
  const int lin = blockIdx.x;
  const int jlin = lin >> 3;
  const int pair = (jlin / ntile) * 8 + (lin & 7);
  const int tile = jlin % ntile;
  if (pair >= batch * hkv) return;
  const int b = pair / hkv, kvh = pair - b * hkv;
  const int G = hq / hkv;
  const int i0 = tile * qt;

  const int prefix = prefix_lens[b], nnew = new_lens[b], nq = q_lens[b];
  const bool bad = prefix < 0 || (prefix & 127) || prefix > kBlockTokens * max_blocks || nnew < 0 ||
                   nnew > max_new || nq < 0 || nq > nnew || nq > max_q;

  // the lane's two rows
  int ri[kCt], rh[kCt];
  bool inrange[kCt], valid[kCt];
#pragma unroll
  for (int ct = 0; ct < kCt; ++ct) {
    const int r = 16 * (kCt * w + ct) + n;
    ri[ct] = r / G;
    rh[ct] = r - ri[ct] * G;
    inrange[ct] = r < qt * G && i0 + ri[ct] < max_q;
    valid[ct] = !bad && inrange[ct] && i0 + ri[ct] < nq;
  }
  auto out_row = [&](int ct) {
    return out + ((static_cast<size_t>(b) * max_q + i0 + ri[ct]) * hq + static_cast<size_t>(kvh) * G + rh[ct]) *
                     kHeadDim;
  };
  auto q_row = [&](int ct) {
    const int i = valid[ct] ? i0 + ri[ct] : 0;
    return q + ((static_cast<size_t>(b) * max_q + i) * hq + static_cast<size_t>(kvh) * G + (valid[ct] ? rh[ct] : 0)) *
                   kHeadDim;
  };

  if (bad || i0 >= nq) {
    // no query of this tile: zero rows (and flag a bad length)
#pragma unroll
    for (int ct = 0; ct < kCt; ++ct)
      if (inrange[ct]) {
        float* o = out_row(ct);
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) *reinterpret_cast<float4*>(o + 16 * mt + 4 * g) = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    if (bad && tid == 0 && flags) atomicOr(flags, kFlagBadSeqLen);
    return;
  }

  // a wave whose rows are all padding (the tail of the last tile) stages blocks with the others but
  // skips the products
  const bool wave_live = __builtin_amdgcn_ballot_w64(valid[0]) != 0;
  PfState S;
#pragma unroll
  for (int ct = 0; ct < kCt; ++ct) {
    S.m[ct] = -INFINITY;
    S.l[ct] = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) S.o[ct][i] = 0.f;
  }
  const int nblk = prefix >> 7;

  // ---- packed prefix (rotated basis) ----------------------------------------------------------------
  if (nblk > 0) {
    float mx = 0.f;
#pragma unroll
    for (int ct = 0; ct < kCt; ++ct)
      mx = fmaxf(mx, load_query(S.qv[ct], q_row(ct), valid[ct], g, lane, true, scale_log2 * kInvSqrt128));
    mx = wave_max(mx);
    if (lane == 0) L.qmax[w] = mx;
    const int32_t* bt = block_table + static_cast<size_t>(b) * max_blocks;
    const size_t kstride = static_cast<size_t>(F::kKPage), vstride = static_cast<size_t>(F::kVPage);
    bool bad_page = false;
    // page p + 1 is requested before page p is attended; a page id out of range reads page 0 and
    // is skipped (the caller guarantees num_pages > 0)
    auto request = [&](PageRaw<F>& R, int page) {
      const size_t unit = static_cast<size_t>(page >= 0 && page < num_pages ? page : 0) * hkv + kvh;
      load_page_raw(R, k_pool + unit * kstride, v_pool + unit * vstride, tid);
    };
    PageRaw<F> R;
    int cur = bt[0];
    request(R, cur);
    for (int p = 0; p < nblk; ++p) {
      const bool ok = cur >= 0 && cur < num_pages;
      __syncthreads();  // every wave is done with the previous block
      if (ok) store_page(L, R, tid);
      const int nxt = p + 1 < nblk ? bt[p + 1] : 0;
      __syncthreads();
      if (p + 1 < nblk) request(R, nxt);
      if (ok) page_factors<GS>(L, tid, lane);
      __syncthreads();
      if (ok) {
        int nolim[kCt];
#pragma unroll
        for (int ct = 0; ct < kCt; ++ct) nolim[ct] = 0x7FFFFFFF;
        if (wave_live) attend_block<false, F::kHalves>(S, L, lane, nolim);
      } else {
        bad_page = true;
      }
      cur = nxt;
    }
    if (bad_page && tid == 0 && flags) atomicOr(flags, kFlagBadPage);
    // back to the original basis
#pragma unroll
    for (int ct = 0; ct < kCt; ++ct) {
      fwht_rows(S.o[ct], lane);
#pragma unroll
      for (int i = 0; i < 32; ++i) S.o[ct][i] *= kInvSqrt128;
    }
  }

  // ---- fp16 rows (original basis, causal) ---------------------------------------------------------
  {
    float mx = 0.f;
#pragma unroll
    for (int ct = 0; ct < kCt; ++ct)
      mx = fmaxf(mx, load_query(S.qv[ct], q_row(ct), valid[ct], g, lane, false, scale_log2));
    mx = wave_max(mx);
    // the previous phase read qmax before its last barrier
    if (lane == 0) L.qmax[w] = mx;
  }
  const int off = nnew - nq;                                  // fp16 row of query 0
  const int last = off + min(i0 + qt, nq) - 1;                // last fp16 row any query of the tile sees
  const size_t rstride = static_cast<size_t>(hkv) * kHeadDim;
  const uint16_t* kb = k_new + (static_cast<size_t>(b) * max_new * hkv + kvh) * kHeadDim;
  const uint16_t* vb = v_new + (static_cast<size_t>(b) * max_new * hkv + kvh) * kHeadDim;
  int lim_abs[kCt];
#pragma unroll
  for (int ct = 0; ct < kCt; ++ct) lim_abs[ct] = valid[ct] ? off + i0 + ri[ct] : 0x7FFFFFFF;
  for (int fb = 0; fb * kBlockTokens <= last; ++fb) {
    __syncthreads();
    store_fp16_block(L, kb, vb, rstride, fb * kBlockTokens, nnew, tid);
    __syncthreads();
    fp16_factors(L, tid);
    __syncthreads();
    const int base = fb * kBlockTokens;
    int lim[kCt];
#pragma unroll
    for (int ct = 0; ct < kCt; ++ct) lim[ct] = lim_abs[ct] == 0x7FFFFFFF ? 0x7FFFFFFF : lim_abs[ct] - base;
    if (wave_live) attend_block<true, 1>(S, L, lane, lim);
  }

  // ---- normalise and store ---------------------------------------------------------------------------
#pragma unroll
  for (int ct = 0; ct < kCt; ++ct) {
    const float l = sum32(sum16(S.l[ct]));
    const float inv = valid[ct] ? 1.0f / l : 0.f;
    if (inrange[ct]) {
      float* o = out_row(ct);
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
        *reinterpret_cast<float4*>(o + 16 * mt + 4 * g) =
            make_float4(S.o[ct][4 * mt] * inv, S.o[ct][4 * mt + 1] * inv, S.o[ct][4 * mt + 2] * inv,
                        S.o[ct][4 * mt + 3] * inv);
    }
  }
}

hipError_t launch_prefill(const void* q, int max_q, const void* k_pool, const void* v_pool, int num_pages,
                          const int32_t* block_table, int max_blocks, const int32_t* prefix_lens, const void* k_new,
                          const void* v_new, int max_new, const int32_t* new_lens, const int32_t* q_lens, int batch,
                          int hq, int hkv, int kbits, int vbits, int group, float scale_log2, float* out,
                          uint32_t* flags, hipStream_t stream) {
  const int G = hq / hkv;
  const int qt = kPfRows / G;
  const int ntile = (max_q + qt - 1) / qt;
  const long pairs8 = (static_cast<long>(batch) * hkv + 7) / 8;
  const long groups = 8 * pairs8 * ntile;
  if (groups == 0) return hipSuccess;
  if (groups > 0x7FFFFFFFL) return hipErrorInvalidConfiguration;
  auto kernel = group == 64 ? (kbits == 8 ? (vbits == 4 ? prefill_kernel<8, 4, 64> : prefill_kernel<8, 2, 64>)
                                          : (vbits == 4 ? prefill_kernel<4, 4, 64> : prefill_kernel<4, 2, 64>))
                            : (kbits == 8 ? (vbits == 4 ? prefill_kernel<8, 4, 128> : prefill_kernel<8, 2, 128>)
                                          : (vbits == 4 ? prefill_kernel<4, 4, 128> : prefill_kernel<4, 2, 128>));
  hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(groups)), dim3(kPfThreads), 0, stream,
                     static_cast<const uint16_t*>(q), max_q, static_cast<const uint8_t*>(k_pool),
                     static_cast<const uint8_t*>(v_pool), num_pages, block_table, max_blocks, prefix_lens,
                     static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new), max_new, new_lens,
                     q_lens, batch, hq, hkv, qt, ntile, scale_log2, out, flags);
  return hipGetLastError();
}

}  // namespace kvarn
