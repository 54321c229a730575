// Decode attention over the packed KVarN cache for gfx950.
//
// A workgroup of four waves handles one (sequence, KV head, split): the G <= 8
// query heads that share the KV head attend to a run of 128-token pages, wave
// w taking every fourth page of the run.  Nothing is dequantised to memory.
// Because the rotation is orthonormal (KVarN blog post, section "KVarN Nasıl
// Çalışır?": it keeps attention scores), the query is rotated once, q~ = H q,
// and both contractions run in the rotated basis:
//
//   key page:   score_t = 2^rho_t * ( sum_j a_j c_tj + b ),
//               a_j = q~_j 2^gamma_j s_j,   b = sum_j q~_j 2^gamma_j z_j
//   value page: o_j += 2^gamma_j * ( sum_t w_t c_tj + u ),
//               w_t = p_t 2^rho_t s_t,      u = sum_t p_t 2^rho_t z_t
//
// with online softmax over the pages (scores in log2 units).  Both sums over
// codes are dense (G x 128) x (128 x 128) products per page and run on
// v_mfma_f32_16x16x32_f16.  Codes enter as exact fp16 integers off + c: one
// mask-and-or (and for most pairs one shift) places a pair of codes in the
// mantissa under a fixed exponent, which fixes the offset (4-bit keys 16 or 64,
// 8-bit keys 1024; 2-bit values 4 or 16, 4-bit values 64).  The kernel is
// instantiated per code widths and group size; only the page geometry, the
// code loads and these conversions differ, and for group size 64 (two scale /
// zero sets per channel or token) the key products run once per token half and
// the value products take their channel half's weights.  The offsets are
// removed with sums of the very fp16 coefficients the matrix cores multiplied.  (fp16 subnormal operands would
// need no offset, but the matrix cores lose precision on them, biased toward
// zero.)  The fp32 coefficients a_j and w_t enter as an fp16 hi + lo pair (hi in
// matrix columns 0-7, lo in columns 8-15) after a power-of-two page scale keeps
// them in fp16 range; lanes n and n^8 of a 16-lane row then hold the two halves
// of one query head.  The per-head constants (b and u, offsets removed) enter
// as the accumulator input of the first product of each chain.
//
// Latency: three workgroups (twelve waves) share a compute unit with 4-bit keys
// and group size 128 (two otherwise), so one wave's page loads overlap the
// others' arithmetic; a wave's first page is requested
// together with the query, before the query transform, which then runs under
// that page's HBM latency.  Both 128-point transforms (q~ = H q at the start,
// H o at the end) run in registers, two entries per lane, with DPP and
// permlane exchanges: no workgroup barrier.
//
// Each wave keeps (m, l, o[128]) per head; the four waves merge through LDS,
// the workgroup writes one partial per split, and the last workgroup of a
// (sequence, KV head) to arrive merges the splits with log-sum-exp weights,
// applies the inverse rotation H and writes fp32 output.
#include "kvarn_codes.h"

namespace kvarn {

namespace {

constexpr int kWaves = 4;
constexpr int kPartStride = kHeadDim + 2;  // o[128], m, l per (split, query head)
constexpr int kCoefStride = 68;            // dwords per coefficient column (64 slots + pad)
constexpr int kMaxSplits = 64;             // the host plan never exceeds this many splits per (sequence, KV head)
static_assert(kMaxSplits <= 64, "the split merge gives every split its own lane");
constexpr int kQLaneStride = 20;           // floats per lane row of q~ (16 used; 20 keeps float4 reads conflict-free)

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// Split the products x0*y0 and x1*y1 into packed fp16 hi and lo parts.  hi is the nearest fp16
// of the fp32 product (v_cvt_pk_f16_f32 rounds to nearest even and keeps fp16 subnormals; the
// round-toward-zero packing instruction flushes them, and a flushed lo part biases every sum it
// enters); lo is the nearest fp16 of the exact residual x*y - hi (one v_fma_mix each), so
// hi + lo carries about 22 significant bits.  hi is pinned by the empty asm so that the value
// stored and the value subtracted are the same one.
__device__ __forceinline__ void split_prod(float x0, float y0, float x1, float y1, uint32_t& hi, uint32_t& lo) {
  f16x2 h = {static_cast<_Float16>(x0 * y0), static_cast<_Float16>(x1 * y1)};
  asm("" : "+v"(h));
  const f16x2 l = {static_cast<_Float16>(__builtin_fmaf(x0, y0, -static_cast<float>(h[0]))),
                   static_cast<_Float16>(__builtin_fmaf(x1, y1, -static_cast<float>(h[1])))};
  hi = __builtin_bit_cast(uint32_t, h);
  lo = __builtin_bit_cast(uint32_t, l);
}

// Per-lane select without data-dependent indexing: lanes 8-15 of every 16-lane row (DPP banks 2
// and 3) take `lo_lanes`, lanes 0-7 keep `hi_lanes` (a bank-masked identity DPP move).
__device__ __forceinline__ uint32_t sel_lo_u32(uint32_t hi_lanes, uint32_t lo_lanes) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(hi_lanes), static_cast<int>(lo_lanes),
                                                           0xE4, 0xF, 0xC, false));
}
__device__ __forceinline__ float sel_lo(float hi_lanes, float lo_lanes) {
  return __uint_as_float(sel_lo_u32(__float_as_uint(hi_lanes), __float_as_uint(lo_lanes)));
}

__device__ __forceinline__ uint32_t dpp_u32_xor8(uint32_t x) {
  return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(x), kDppXor8, 0xF, 0xF, true));
}

// One bank-masked row_ror:8 move each: lanes 8-15 of every 16-lane row take `src` of lane l ^ 8 and
// lanes 0-7 keep `keep` (take_xor8_hi), or lanes 0-7 take it and lanes 8-15 keep (take_xor8_lo).
__device__ __forceinline__ uint32_t take_xor8_hi(uint32_t keep, uint32_t src) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(static_cast<int>(keep), static_cast<int>(src), kDppXor8, 0xF, 0xC, false));
}
__device__ __forceinline__ uint32_t take_xor8_lo(uint32_t keep, uint32_t src) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(static_cast<int>(keep), static_cast<int>(src), kDppXor8, 0xF, 0x3, false));
}

// x from lane l^16 and l^32 (v_permlane16_swap / v_permlane32_swap on two copies of x).  The
// pair (self, partner) is returned in lane order, so both lanes of a pair combine the same two
// values in the same order and get identical bits.
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Max / sum over the 8 lanes that hold one query head (lanes n, n^8 in each of the 4 rows).
__device__ __forceinline__ float head_max(float x) {
  x = fmaxf(x, dpp<kDppXor8>(x));
  return max_xor32(max_xor16(x));
}
__device__ __forceinline__ float head_sum(float x) {
  x += dpp<kDppXor8>(x);
  return sum_xor32(sum_xor16(x));
}
// Max over the whole wave, identical in every lane.
__device__ __forceinline__ float wave_max_all(float x) { return max_xor32(max_xor16(row16_max(x))); }

// The same for values that are never negative (scales and their products): such floats, with the
// sign bit cleared, order like unsigned integers, and the integer max takes its DPP operand
// directly (a float max would first canonicalise the moved value).
__device__ __forceinline__ float wave_max_nonneg(float x) {
  uint32_t u = __float_as_uint(x) & 0x7FFFFFFFu;
  auto mx = [&](uint32_t v) { u = u > v ? u : v; };
  mx(static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(u), kDppXor1, 0xF, 0xF, true)));
  mx(static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(u), kDppXor2, 0xF, 0xF, true)));
  mx(static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(u), kDppXor7, 0xF, 0xF, true)));
  mx(static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(u), kDppXor8, 0xF, 0xF, true)));
  auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  u = r[0] > r[1] ? r[0] : r[1];
  r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  u = r[0] > r[1] ? r[0] : r[1];
  return __uint_as_float(u);
}

// Sum over all 64 lanes of v[l & 7] (for each lane l): a transpose-reduce that halves the
// number of values per lane at each of the first three stages (partners l^1, l^2 and l+4 mod
// 16, the last one a row rotation), then adds across lanes l^8, l^16, l^32.
__device__ __forceinline__ float head_reduce8(const float (&v)[kMaxGroup], int lane) {
  const bool b0 = lane & 1, b1 = lane & 2, b2 = lane & 4;
  float s4[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float keep = b0 ? v[2 * k + 1] : v[2 * k];
    const float send = b0 ? v[2 * k] : v[2 * k + 1];
    s4[k] = keep + dpp<kDppXor1>(send);
  }
  float s2[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    // s4[k] holds head 2k + b0; keep the two whose bit 1 (= k & 1) matches this lane
    const float keep = b1 ? s4[2 * m + 1] : s4[2 * m];
    const float send = b1 ? s4[2 * m] : s4[2 * m + 1];
    s2[m] = keep + dpp<kDppXor2>(send);
  }
  // s2[k] holds head 4k + 2 b1 + b0; lane (l + 4) mod 16 always has the other value of b2
  const float keep = b2 ? s2[1] : s2[0];
  const float send = b2 ? s2[0] : s2[1];
  float s = keep + dpp<kDppRor4>(send);
  s += dpp<kDppXor8>(s);
  return sum_xor32(sum_xor16(s));
}

// Agent-scope relaxed accesses to the split partials: on gfx950 they bypass the XCD-private L2
// state that other XCDs cannot see.
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// In-register 128-point Walsh-Hadamard transform (natural order, unnormalised) of one vector
// held two entries per lane, x0 = v[2l] and x1 = v[2l + 1].  Index bit 0 is inside the lane;
// index bit s >= 1 is lane bit s - 1, so stage s pairs lane l with l ^ 2^(s-1): the lane whose
// bit is clear keeps the sum, the other the difference (partner minus own).
__device__ __forceinline__ void wave_fwht(float& x0, float& x1, int lane) {
  {
    const float a = x0 + x1, b = x0 - x1;
    x0 = a;
    x1 = b;
  }
  auto dpp_stage = [&](float p0, float p1, int bit) {
    const float sg = (lane & bit) ? -1.f : 1.f;
    x0 = fmaf(sg, x0, p0);
    x1 = fmaf(sg, x1, p1);
  };
  dpp_stage(dpp<kDppXor1>(x0), dpp<kDppXor1>(x1), 1);
  dpp_stage(dpp<kDppXor2>(x0), dpp<kDppXor2>(x1), 2);
  // lane ^ 4 = (lane ^ 7) ^ 3 inside 8 lanes
  dpp_stage(dpp<kDppXor3>(dpp<kDppXor7>(x0)), dpp<kDppXor3>(dpp<kDppXor7>(x1)), 4);
  dpp_stage(dpp<kDppXor8>(x0), dpp<kDppXor8>(x1), 8);
  // the swaps return (value of the lower partner, value of the upper partner): lower + sign * upper
  {
    const float sg = (lane & 16) ? -1.f : 1.f;
    const auto r0 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x0), __float_as_uint(x0), false, false);
    const auto r1 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x1), __float_as_uint(x1), false, false);
    x0 = fmaf(sg, __uint_as_float(r0[1]), __uint_as_float(r0[0]));
    x1 = fmaf(sg, __uint_as_float(r1[1]), __uint_as_float(r1[0]));
  }
  {
    const float sg = (lane & 32) ? -1.f : 1.f;
    const auto r0 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x0), __float_as_uint(x0), false, false);
    const auto r1 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x1), __float_as_uint(x1), false, false);
    x0 = fmaf(sg, __uint_as_float(r0[1]), __uint_as_float(r0[0]));
    x1 = fmaf(sg, __uint_as_float(r1[1]), __uint_as_float(r1[0]));
  }
}

__device__ __forceinline__ float wave_sum_all(float x) { return sum_xor32(sum_xor16(row16_sum(x))); }

// Per-wave page state in shared memory; NH = groups per channel (keys) or token (values): 1 for group
// size 128, 2 for group size 64 (index = the half of the block's tokens / channels).
template <int NH>
struct __align__(16) WaveLds {
  uint32_t coef[NH][16][kCoefStride];  // key-side B operand per token half: [column][slot] packed fp16 pairs
  float pk[kHeadDim];                  // 2^rho (K) / key page scale, per token
  float fv[NH][kHeadDim];              // 2^rho s (V) * value page scale, per channel half and token
  float zv[NH][kHeadDim];              // 2^rho z (V), per channel half and token
  float gs[kHeadDim];                  // 2^gamma (V) / value page scale, per channel
};

// Page geometry of one pair of code widths (4- or 8-bit keys, 2- or 4-bit values) and group size.
template <int KB, int VB, int GS>
struct DecFormat {
  using Meta = MetaLayout<GS>;
  static constexpr int kHalves = Meta::kHalves;
  static constexpr int kKRow = kHeadDim * KB / 8;       // bytes of one token's key codes
  static constexpr int kVRow = kBlockTokens * VB / 8;   // bytes of one channel's value codes
  static constexpr int kKCode = kBlockTokens * kKRow;
  static constexpr int kVCode = kHeadDim * kVRow;
  static constexpr int kKPage = kKCode + Meta::kBytes;
  static constexpr int kVPage = kVCode + Meta::kBytes;
  // second coefficient slot of a lane: channel ch0 + 4 for nibbles (pairs j, j + 4 of a dword),
  // ch0 + 1 for bytes (channel order)
  static constexpr int kCh1 = KB == 8 ? 1 : 4;
  // resident waves per SIMD: byte-wide keys and two groups per channel / token need more registers
  // (4-bit keys with 4-bit values keep three waves at the cost of a two-register spill, which is
  // faster than two waves).  The prefetching kernel (kCanPrefetch formats only) runs at two.
  static constexpr int kMinWaves = KB == 4 && GS == 128 ? 3 : 2;
  // Formats whose next-page registers fit at two waves per SIMD without spills.
  static constexpr bool kCanPrefetch = KB == 4 && GS == 128;
};

// Coefficient slots of a lane: channels ch0 and ch0 + kCh1, ch0 = 32*(lane/16) + 8*((lane/4)%4) +
// (lane%4, or 2*(lane%4) for byte-wide key codes).
template <int KB>
__device__ __forceinline__ int coef_channel(int lane) {
  return 32 * (lane >> 4) + 8 * ((lane >> 2) & 3) + (KB == 8 ? 2 : 1) * (lane & 3);
}

// One page of one KV head as this lane loads it.
template <int KB, int VB, int GS>
struct PageRegs {
  static constexpr int NH = DecFormat<KB, VB, GS>::kHalves;
  u32x4 kc[8][KB / 4];    // key codes: M-tile mt, row n -> token 32*(n/4) + 4*mt + n%4, channels 32g .. 32g+31
  uint32_t vc[8][VB];     // value codes: M-tile mt, row n -> channel 16mt + n, tokens 32g .. 32g+31
  uint32_t ks0[NH], ks1[NH];  // key scale (fp16 bits) of channels ch0, ch1, per token half
  uint32_t kz0[NH], kz1[NH];  // key zero
  float kg0, kg1;             // key gamma
  float2 kr;                  // key rho of tokens 2*lane, 2*lane+1
  uint32_t vs2[NH], vz2[NH];  // value scale / zero (fp16 pairs) of tokens 2*lane, 2*lane+1, per channel half
  float2 vr, vg;              // value rho of those tokens, value gamma of channels 2*lane, 2*lane+1
  bool ok;
};

// Page bases of one (page, KV head).  A bad page id reads page 0 instead (the caller guarantees
// num_pages > 0) and only clears `ok`, so every load is issued without a branch.
struct PagePtrs {
  const uint8_t* kp;
  const uint8_t* vp;
  bool ok;
  bool load;  // false: nothing to prefetch (the wave's last page)
};
template <int KB, int VB, int GS>
__device__ __forceinline__ PagePtrs page_ptrs(int page, int num_pages, int hkv, int kvh,
                                              const uint8_t* __restrict__ k_pool, const uint8_t* __restrict__ v_pool) {
  using F = DecFormat<KB, VB, GS>;
  PagePtrs r;
  r.ok = page >= 0 && page < num_pages;
  const int safe = r.ok ? page : 0;
  r.kp = k_pool + (static_cast<size_t>(safe) * hkv + kvh) * F::kKPage;
  r.vp = v_pool + (static_cast<size_t>(safe) * hkv + kvh) * F::kVPage;
  r.load = true;
  return r;
}

// The three parts of a page a lane loads: metadata (consumed first), key codes, value codes.  Lane
// offsets are recomputed for every page (a few integer operations) rather than kept live across the
// page loop, where registers are short.  They are unsigned 32-bit byte offsets from the wave-uniform
// page base, so each load takes the base from scalar registers, the lane offset from one vector
// register and the per-load constant as its immediate.
template <int KB, int VB, int GS>
__device__ __forceinline__ void load_meta(PageRegs<KB, VB, GS>& P, const PagePtrs& pg, int lane, int ch0) {
  using F = DecFormat<KB, VB, GS>;
  using Meta = typename F::Meta;
  asm volatile("" : "+v"(lane), "+v"(ch0));
  P.ok = pg.ok;
  const uint32_t c2 = 2u * static_cast<uint32_t>(ch0), c4 = 4u * static_cast<uint32_t>(ch0);
  const uint32_t l4 = 4u * static_cast<uint32_t>(lane), l8 = 8u * static_cast<uint32_t>(lane);
  auto u16 = [](const uint8_t* a) { return static_cast<uint32_t>(*reinterpret_cast<const uint16_t*>(a)); };
  auto u32 = [](const uint8_t* a) { return *reinterpret_cast<const uint32_t*>(a); };
  auto f32 = [](const uint8_t* a) { return *reinterpret_cast<const float*>(a); };
  auto f2 = [](const uint8_t* a) { return *reinterpret_cast<const float2*>(a); };
#pragma unroll
  for (int hh = 0; hh < F::kHalves; ++hh) {  // group entry 128*hh + j (half-major)
    P.ks0[hh] = u16(pg.kp + c2 + (F::kKCode + Meta::kScale + 256 * hh));
    P.ks1[hh] = u16(pg.kp + c2 + (F::kKCode + Meta::kScale + 256 * hh + 2 * F::kCh1));
    P.kz0[hh] = u16(pg.kp + c2 + (F::kKCode + Meta::kZero + 256 * hh));
    P.kz1[hh] = u16(pg.kp + c2 + (F::kKCode + Meta::kZero + 256 * hh + 2 * F::kCh1));
    P.vs2[hh] = u32(pg.vp + l4 + (F::kVCode + Meta::kScale + 256 * hh));
    P.vz2[hh] = u32(pg.vp + l4 + (F::kVCode + Meta::kZero + 256 * hh));
  }
  P.kg0 = f32(pg.kp + c4 + (F::kKCode + Meta::kGamma));
  P.kg1 = f32(pg.kp + c4 + (F::kKCode + Meta::kGamma + 4 * F::kCh1));
  P.kr = f2(pg.kp + l8 + (F::kKCode + Meta::kRho));
  P.vr = f2(pg.vp + l8 + (F::kVCode + Meta::kRho));
  P.vg = f2(pg.vp + l8 + (F::kVCode + Meta::kGamma));
}
template <int KB, int VB, int GS>
__device__ __forceinline__ void load_kcodes(PageRegs<KB, VB, GS>& P, const PagePtrs& pg, int n, int g) {
  using F = DecFormat<KB, VB, GS>;
  asm volatile("" : "+v"(n), "+v"(g));
  const uint32_t off = static_cast<uint32_t>((32 * (n >> 2) + (n & 3)) * F::kKRow + (KB / 4) * 16 * g);
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int h = 0; h < KB / 4; ++h)
      P.kc[mt][h] = *reinterpret_cast<const u32x4*>(pg.kp + off + (4 * mt * F::kKRow + 16 * h));
}
template <int KB, int VB, int GS>
__device__ __forceinline__ void load_vcodes(PageRegs<KB, VB, GS>& P, const PagePtrs& pg, int n, int g) {
  using F = DecFormat<KB, VB, GS>;
  asm volatile("" : "+v"(n), "+v"(g));
  const uint32_t off = static_cast<uint32_t>(n * F::kVRow + (VB == 2 ? 8 : 16) * g);
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) {
    if constexpr (VB == 2) {
      const u32x2 x = *reinterpret_cast<const u32x2*>(pg.vp + off + 16 * mt * F::kVRow);
      P.vc[mt][0] = x[0];
      P.vc[mt][1] = x[1];
    } else {
      const u32x4 x = *reinterpret_cast<const u32x4*>(pg.vp + off + 16 * mt * F::kVRow);
#pragma unroll
      for (int k = 0; k < 4; ++k) P.vc[mt][k] = x[k];
    }
  }
}
template <int KB, int VB, int GS>
__device__ __forceinline__ void load_page(PageRegs<KB, VB, GS>& P, const PagePtrs& pg, int lane, int n, int g,
                                          int ch0) {
  load_kcodes(P, pg, n, g);
  load_vcodes(P, pg, n, g);
  load_meta(P, pg, lane, ch0);
}

// Per-wave state carried across pages.
struct WaveState {
  const float* ql;                     // rotated, scaled query at this lane's two slots: [h] and [8 + h]
  float qmax;                          // max over the heads of |q~| at every slot
  float m_run, l_run;                  // online softmax of this lane's head (log2 units)
  float acc[8][4];                     // o (rotated basis, hi or lo column) of channels 16mt + 4g + r
};

// Magic fp16 exponent patterns (each twice, kept in vector registers) that turn codes into fp16 off + c.
struct Mags {
  uint32_t m16, m64, m4, m1024;
};

// One page of the wave.  With PF, the next page's parts are loaded into P as soon as this page's
// copies have been used (metadata after the coefficients, key codes after the scores, value codes at
// the end), so that their HBM latency runs under the rest of this page.
template <int KB, int VB, int GS, bool PF>
__device__ __forceinline__ void process_page(PageRegs<KB, VB, GS>& P, WaveState& S,
                                             WaveLds<DecFormat<KB, VB, GS>::kHalves>& L, int G, int lane, int g,
                                             int lo_col, const Mags& M, const PagePtrs& next, int ch0) {
  // NH = 2 (group size 64): key groups differ between the token halves, value groups between the
  // channel halves.  A lane's score rows are tokens of quarter g, i.e. of half g / 2; value M-tiles
  // 0-3 are channels 0-63 and 4-7 channels 64-127.
  constexpr int NH = DecFormat<KB, VB, GS>::kHalves;
  // ---- key-side coefficients (this lane: slots ch0 and ch1, all heads), per token half -----------
  const float eg0 = ex2(P.kg0), eg1 = ex2(P.kg1);
  float e0[NH], e1[NH], f0[NH], f1[NH];
  float emx = 0.f;
#pragma unroll
  for (int hh = 0; hh < NH; ++hh) {
    e0[hh] = eg0 * half_bits_to_float(P.ks0[hh]);
    e1[hh] = eg1 * half_bits_to_float(P.ks1[hh]);
    f0[hh] = eg0 * half_bits_to_float(P.kz0[hh]);
    f1[hh] = eg1 * half_bits_to_float(P.kz1[hh]);
    emx = fmaxf(emx, fmaxf(e0[hh], e1[hh]));
  }
  // ---- value-side per-token factors (this lane: tokens 2*lane, 2*lane+1), per channel half -------
  const float vr0 = ex2(P.vr.x), vr1 = ex2(P.vr.y);
  float F0[NH], F1[NH];
  float fmx = 0.f;
#pragma unroll
  for (int hh = 0; hh < NH; ++hh) {
    F0[hh] = vr0 * half_bits_to_float(P.vs2[hh] & 0xFFFFu);
    F1[hh] = vr1 * half_bits_to_float(P.vs2[hh] >> 16);
    fmx = fmaxf(fmx, fmaxf(F0[hh], F1[hh]));
  }
  const float emax = wave_max_nonneg(emx);
  const float fmaxv = wave_max_nonneg(fmx);

  int ex;
  const float prod = S.qmax * emax;
  frexpf(prod, &ex);
  ex = min(max(ex, -100), 100);
  const bool live = prod > 0.f;
  const float sa = live ? pow2i(14 - ex) : 1.f;  // |a * sa| < 2^14
  // with no positive key scale the coefficients are all zero but b is not: keep the page at unit scale
  const float inv_sa = live ? pow2i(ex - 14) : 1.f;
  // the key offsets of this lane's two slots: 1024 for bytes; for nibbles 64 for nibbles 1 and 5
  // of a dword, else 16
  const _Float16 off = KB == 8 ? static_cast<_Float16>(1024.0f)
                               : ((lane & 3) == 1 ? static_cast<_Float16>(64.0f) : static_cast<_Float16>(16.0f));
  const f16x2 offp = {off, off};
  float q0[kMaxGroup], q1[kMaxGroup];
  {
    const float4* qv = reinterpret_cast<const float4*>(__builtin_assume_aligned(S.ql, 16));
    const float4 a = qv[0], b = qv[1], c = qv[2], d = qv[3];
    q0[0] = a.x; q0[1] = a.y; q0[2] = a.z; q0[3] = a.w; q0[4] = b.x; q0[5] = b.y; q0[6] = b.z; q0[7] = b.w;
    q1[0] = c.x; q1[1] = c.y; q1[2] = c.z; q1[3] = c.w; q1[4] = d.x; q1[5] = d.y; q1[6] = d.z; q1[7] = d.w;
  }
  float kinit[NH];
#pragma unroll
  for (int hh = 0; hh < NH; ++hh) {
    const float e0s = e0[hh] * sa, e1s = e1[hh] * sa;
    float bp[kMaxGroup];
#pragma unroll
    for (int h = 0; h < kMaxGroup; ++h) {
      if (h < G) {
        uint32_t hi, lo;
        split_prod(q0[h], e0s, q1[h], e1s, hi, lo);
        L.coef[hh][h][lane] = hi;
        L.coef[hh][8 + h][lane] = lo;
        // offset contribution of exactly the fp16 coefficients the matrix cores use
        const float aoff = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, lo), offp,
                                                  __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, hi), offp, 0.f,
                                                                         false),
                                                  false);
        bp[h] = fmaf(-inv_sa, aoff, fmaf(q0[h], f0[hh], q1[h] * f1[hh]));
      } else {
        bp[h] = 0.f;
      }
    }
    // b (offsets removed) of this lane's head, in key-page-scaled units, enters the hi columns
    kinit[hh] = sel_lo(head_reduce8(bp, lane) * sa, 0.f);
  }

  int exf;
  frexpf(fmaxv, &exf);
  exf = min(max(exf, -100), 100);
  const bool livef = fmaxv > 0.f;
  const float sw = livef ? pow2i(14 - exf) : 1.f;  // p <= 1, so |w * sw| < 2^14
  // with no positive value scale the weights are all zero but u is not: unit scale again
  const float inv_sw = livef ? pow2i(exf - 14) : 1.f;
  const int t0 = 2 * lane;
  L.pk[t0] = ex2(P.kr.x) * inv_sa;
  L.pk[t0 + 1] = ex2(P.kr.y) * inv_sa;
#pragma unroll
  for (int hh = 0; hh < NH; ++hh) {
    L.fv[hh][t0] = F0[hh] * sw;
    L.fv[hh][t0 + 1] = F1[hh] * sw;
    L.zv[hh][t0] = vr0 * half_bits_to_float(P.vz2[hh] & 0xFFFFu);
    L.zv[hh][t0 + 1] = vr1 * half_bits_to_float(P.vz2[hh] >> 16);
  }
  L.gs[t0] = ex2(P.vg.x) * inv_sw;
  L.gs[t0 + 1] = ex2(P.vg.y) * inv_sw;
  if constexpr (PF) {
    if (next.load) load_meta(P, next, lane, ch0);
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();

  // ---- key side: scores ---------------------------------------------------
  // M-tiles mt and mt + 4 give this lane's tokens of the hi and lo halves; lanes 0-7 of a row
  // keep tile mt, lanes 8-15 tile mt + 4 (tokens 32g + 16*lo_col + 4mt + r).  With two token
  // halves the products run once per half's coefficients and lanes of quarters 2, 3 keep the second.
  const int n = lane & 15;
  float sm[4][4];
  const float* pkp = &L.pk[32 * g + 16 * lo_col];
#pragma unroll
  for (int hh = 0; hh < NH; ++hh) {
    f16x8 cb[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      cb[ks] = __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4*>(&L.coef[hh][n][16 * g + 4 * ks]));
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      f32x4 da = {kinit[hh], kinit[hh], kinit[hh], kinit[hh]}, db = da;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        if constexpr (KB == 4) {
          da = mfma16x16x32(key_codes(P.kc[mt][0][ks], M.m16, M.m64), cb[ks], da);
          db = mfma16x16x32(key_codes(P.kc[mt + 4][0][ks], M.m16, M.m64), cb[ks], db);
        } else {
          const int h = ks >> 1, d = 2 * (ks & 1);
          da = mfma16x16x32(key_codes8(P.kc[mt][h][d], P.kc[mt][h][d + 1], M.m1024), cb[ks], da);
          db = mfma16x16x32(key_codes8(P.kc[mt + 4][h][d], P.kc[mt + 4][h][d + 1], M.m1024), cb[ks], db);
        }
      }
      const float4 pk4 = *reinterpret_cast<const float4*>(pkp + 4 * mt);
      const float pkv[4] = {pk4.x, pk4.y, pk4.z, pk4.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float xa = da[r] + dpp<kDppXor8>(da[r]);
        const float xb = db[r] + dpp<kDppXor8>(db[r]);
        const float v = pkv[r] * sel_lo(xa, xb);
        sm[mt][r] = hh == 0 ? v : (g >= 2 ? v : sm[mt][r]);
      }
    }
  }
  if constexpr (PF) {
    if (next.load) load_kcodes(P, next, n, g);
  }
  float mloc = -INFINITY;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) mloc = fmaxf(mloc, sm[mt][r]);
  mloc = head_max(mloc);
  const float m_new = fmaxf(S.m_run, mloc);
  const float alpha = ex2(S.m_run - m_new);
  // o needs rescaling only if some head of the wave has a new maximum (alpha is exactly 1 otherwise)
  if (__builtin_amdgcn_ballot_w64(m_new != S.m_run) != 0) {
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) S.acc[mt][r] *= alpha;
  }
  S.m_run = m_new;

  // ---- softmax weights ----------------------------------------------------
  float lsum = 0.f;
  float pv[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float p = ex2(sm[mt][r] - m_new);
      lsum += p;
      pv[mt][r] = p;
    }
  lsum = head_sum(lsum);
  S.l_run = fmaf(S.l_run, alpha, lsum);

  // ---- value side, per channel half: B operand, then o (rotated basis, hi and lo columns apart) --
#pragma unroll
  for (int vh = 0; vh < NH; ++vh) {
    const float* fvp = &L.fv[vh][32 * g + 16 * lo_col];
    const float* zvp = &L.zv[vh][32 * g + 16 * lo_col];
    float usum = 0.f, wev = 0.f, wod = 0.f;
    float fvv[4][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const float4 f4 = *reinterpret_cast<const float4*>(fvp + 4 * mt);
      const float4 z4 = *reinterpret_cast<const float4*>(zvp + 4 * mt);
      fvv[mt][0] = f4.x; fvv[mt][1] = f4.y; fvv[mt][2] = f4.z; fvv[mt][3] = f4.w;
      const float zvv[4] = {z4.x, z4.y, z4.z, z4.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) usum = fmaf(pv[mt][r], zvv[r], usum);
    }
    // w_t = p_t * fv_t; pair (hf, j) = tokens 4hf + j and 4hf + j + 8 of this lane's 16
    uint32_t own_hi[2][4], own_lo[2][4];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        split_prod(pv[hf][j], fvv[hf][j], pv[hf + 2][j], fvv[hf + 2][j], own_hi[hf][j], own_lo[hf][j]);
    // value offsets (2-bit codes: 4 for even tokens, 16 for odd; 4-bit codes: 64) of exactly the fp16
    // weights used
    {
      const f16x2 ones = {static_cast<_Float16>(1.0f), static_cast<_Float16>(1.0f)};
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float& acc = (j & 1) ? wod : wev;
          acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, own_hi[hf][j]), ones, acc, false);
          acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, own_lo[hf][j]), ones, acc, false);
        }
    }
    // u minus the value offsets, in value-page-scaled units, enters the hi columns
    const float voff = VB == 2 ? fmaf(16.f, wod, 4.f * wev) : 64.f * (wev + wod);
    const float ucorr = head_sum(fmaf(usum, sw, -voff));
    const float vinit = sel_lo(ucorr, 0.f);
    f16x8 wb[2][2];  // [u][hf]
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      // u0: the tokens of lanes 0-7, hi parts in columns 0-7 and lo parts (from lane n ^ 8) in 8-15;
      // u1: the tokens of lanes 8-15, hi parts (from lane n ^ 8) in 0-7 and lo parts in 8-15
      u32x4 u0, u1;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u0[j] = take_xor8_hi(own_hi[hf][j], own_lo[hf][j]);
        u1[j] = take_xor8_lo(own_lo[hf][j], own_hi[hf][j]);
      }
      wb[0][hf] = __builtin_bit_cast(f16x8, u0);
      wb[1][hf] = __builtin_bit_cast(f16x8, u1);
    }
#pragma unroll
    for (int mt = (NH == 1 ? 0 : 4 * vh); mt < (NH == 1 ? 8 : 4 * vh + 4); ++mt) {
      f32x4 d = {vinit, vinit, vinit, vinit};
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        f16x8 c0, c1;
        if constexpr (VB == 2) {
          value_codes(P.vc[mt][u], M.m4, M.m16, c0, c1);
        } else {
          value_codes4(P.vc[mt][2 * u], P.vc[mt][2 * u + 1], M.m64, c0, c1);
        }
        d = mfma16x16x32(c0, wb[u][0], d);
        d = mfma16x16x32(c1, wb[u][1], d);
      }
      const float4 gs4 = *reinterpret_cast<const float4*>(&L.gs[16 * mt + 4 * g]);
      const float gsv[4] = {gs4.x, gs4.y, gs4.z, gs4.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) S.acc[mt][r] = fmaf(d[r], gsv[r], S.acc[mt][r]);
    }
  }
  if constexpr (PF) {
    if (next.load) load_vcodes(P, next, lane & 15, g);
  }
}

// The fp16 tail of one (sequence, KV head): the ntail < 128 tokens after the last full block, token
// t of KV head kvh at kt + t * tstride (the layout of the quantiser's input, one block per
// sequence).  Wave 0 computes (m, l, o) of the G heads over the tail exactly as over an fp16 page
// (MFMA scores, masked past ntail; V transposed by a selection-matrix product; p as fp16 hi + lo),
// rotates o by H~ so that it merges with the packed splits (whose o is in the rotated basis), and
// stores the partial at pp.  scratch: 8 x 128 floats of LDS.
__device__ __forceinline__ void tail_partial(const uint16_t* __restrict__ qrow0, const uint16_t* __restrict__ kt,
                                             const uint16_t* __restrict__ vt, size_t tstride, int ntail, int G,
                                             float scale_log2, float* __restrict__ pp, float (*scratch)[kHeadDim],
                                             float* __restrict__ ml, int lane) {
  const int n = lane & 15, g = lane >> 4;
  f16x8 qb[4];
#pragma unroll
  for (int cg = 0; cg < 4; ++cg) {
    const f16x8 v = *reinterpret_cast<const f16x8*>(qrow0 + (n < G ? n : 0) * kHeadDim + 32 * cg + 8 * g);
    const f16x8 zero = {};
    qb[cg] = n < G ? v : zero;
  }
  f16x8 sel[2];
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
    for (int x = 0; x < 8; ++x)
      sel[h2][x] = (8 * g + x == 16 * h2 + n) ? static_cast<_Float16>(1.0f) : static_cast<_Float16>(0.0f);
  const f16x8 zero8 = {};
  // rows past the tail are never read as data: their operands are zero and their scores -inf
  auto row = [&](const uint16_t* base, int t, int cg) {
    const f16x8 v = *reinterpret_cast<const f16x8*>(base + static_cast<size_t>(t < ntail ? t : 0) * tstride +
                                                    32 * cg + 8 * g);
    return t < ntail ? v : zero8;
  };
  float s[8][4];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) {
    f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cg = 0; cg < 4; ++cg) d = mfma16x16x32(row(kt, 16 * mt + n, cg), qb[cg], d);
#pragma unroll
    for (int r = 0; r < 4; ++r) s[mt][r] = 16 * mt + 4 * g + r < ntail ? d[r] * scale_log2 : -INFINITY;
  }
  float m = -INFINITY;
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) m = fmaxf(m, s[mt][r]);
  m = max_xor32(max_xor16(m));  // lanes n, n^16, n^32, n^48 hold the 128 tokens of head n
  float l = 0.f;
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      s[mt][r] = ex2(s[mt][r] - m);  // 0 past the tail
      l += s[mt][r];
    }
  l = sum_xor32(sum_xor16(l));
  f32x4 acc[8];
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    f16x8 hi, lo;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float pv = s[2 * c + (k >> 2)][k & 3];
      hi[k] = static_cast<_Float16>(pv);
      lo[k] = static_cast<_Float16>(pv - static_cast<float>(hi[k]));
    }
    // rows 0-7 take p in fp16, rows 8-15 the remainder of head n - 8 (from lane n ^ 8).  The lane
    // move runs in every lane before the select: under a branch on n, lanes n < 8 would be
    // inactive and the move would read zeros from them.
    f16x8 ap;
    {
      const u32x4 lo_u = __builtin_bit_cast(u32x4, lo), hi_u = __builtin_bit_cast(u32x4, hi);
      u32x4 r;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const uint32_t from8 = dpp_u32_xor8(lo_u[x]);
        r[x] = n < 8 ? hi_u[x] : from8;
      }
      ap = __builtin_bit_cast(f16x8, r);
    }
#pragma unroll
    for (int cg = 0; cg < 4; ++cg) {
      const f16x8 v0 = row(vt, 32 * c + n, cg);
      const f16x8 v1 = row(vt, 32 * c + 16 + n, cg);
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        const f32x4 t0 = mfma16x16x32(v0, sel[h2], z);
        const f32x4 t1 = mfma16x16x32(v1, sel[h2], z);
        f16x8 bv;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          bv[r] = static_cast<_Float16>(t0[r]);
          bv[4 + r] = static_cast<_Float16>(t1[r]);
        }
        acc[2 * cg + h2] = mfma16x16x32(ap, bv, acc[2 * cg + h2]);
      }
    }
  }
  // hi + lo rows; lanes g < 2 then hold o of heads 4g + r for channel 16ct + n
#pragma unroll
  for (int ct = 0; ct < 8; ++ct)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[ct][r] = sum_xor32(acc[ct][r]);
  if (g < 2) {
#pragma unroll
    for (int ct = 0; ct < 8; ++ct)
#pragma unroll
      for (int r = 0; r < 4; ++r) scratch[4 * g + r][16 * ct + n] = acc[ct][r];
  }
  if (g == 0 && n < kMaxGroup) {
    ml[2 * n] = m;
    ml[2 * n + 1] = l;
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  for (int h = 0; h < G; ++h) {
    const float2 ov = reinterpret_cast<const float2*>(scratch[h])[lane];
    float x0 = ov.x, x1 = ov.y;
    wave_fwht(x0, x1, lane);
    float* ph = pp + static_cast<size_t>(h) * kPartStride;
    store_coherent(ph + 2 * lane, x0 * kInvSqrt128);
    store_coherent(ph + 2 * lane + 1, x1 * kInvSqrt128);
    if (lane == 0) {
      store_coherent(ph + kHeadDim, ml[2 * h]);
      store_coherent(ph + kHeadDim + 1, ml[2 * h + 1]);
    }
  }
}

}  // namespace

// PF: the next page of a wave is loaded during the current one (two waves per SIMD); without it
// every page is loaded when its turn comes (three waves per SIMD for 4-bit keys at group size 128).
template <int KB, int VB, int GS, bool PF>
__global__ __launch_bounds__(256, (PF ? 2 : DecFormat<KB, VB, GS>::kMinWaves)) void decode_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ k_pool, const uint8_t* __restrict__ v_pool,
    int num_pages, const int32_t* __restrict__ block_table, int max_blocks, const int32_t* __restrict__ seq_lens,
    const uint16_t* __restrict__ k_tail, const uint16_t* __restrict__ v_tail, int hq, int hkv,
    int blocks_per_split, int max_splits, float scale_log2, float* __restrict__ out, float* __restrict__ part,
    uint32_t* __restrict__ counters, uint32_t* __restrict__ flags) {
  // The per-wave page buffers are live only inside the page loop; before it each wave uses its own
  // buffer as scratch for the query transform, and the four-wave merge after it reuses the memory.
  __shared__ union __align__(16) {
    WaveLds<DecFormat<KB, VB, GS>::kHalves> wl[kWaves];
    struct {
      float wacc[kWaves][kMaxGroup][kHeadDim];   // per-wave o
    } t;
  } U;
  __shared__ __align__(16) float qlane[64][kQLaneStride];  // q~ of each lane's slots, shared by the waves
  __shared__ float wm[kWaves][kMaxGroup], wls[kWaves][kMaxGroup];
  __shared__ int last_flag;
  float (*wacc)[kMaxGroup][kHeadDim] = U.t.wacc;

  // Dispatch order is KV head fastest, then sequence, then split.  Workgroups go to the XCDs
  // round-robin, so consecutive KV heads of one sequence (equal work) land on different XCDs and
  // every XCD gets the same share of each sequence, whatever the mix of lengths; split positions
  // (the high ones empty for all but the longest sequences) vary slowest, so empty splits come last.
  const int kvh = blockIdx.x, b = blockIdx.y, split = blockIdx.z;
  const int G = hq / hkv;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, n = lane & 15, g = lane >> 4;
  const int hd = n & 7;
  const int lo_col = n >> 3;  // this lane's MFMA column carries the lo fp16 part
  const int sl = seq_lens[b];
  float* out_b = out + (static_cast<size_t>(b) * hq + static_cast<size_t>(kvh) * G) * kHeadDim;

  // Without a tail the length must be whole blocks; with one, the tokens past the last full block
  // are in the fp16 tail and form one more split.
  const bool has_tail = k_tail != nullptr;
  const bool bad = sl < 0 || sl > max_blocks * kBlockTokens + (has_tail ? kBlockTokens - 1 : 0) ||
                   (!has_tail && (sl & (kBlockTokens - 1)) != 0);
  const int nblk = bad ? 0 : sl / kBlockTokens;
  const int ntail = bad || !has_tail ? 0 : (sl & (kBlockTokens - 1));
  if (nblk == 0 && ntail == 0) {
    if (split == 0) {
      if (bad && tid == 0 && flags) atomicOr(flags, kFlagBadSeqLen);
      for (int e = tid; e < G * kHeadDim; e += blockDim.x) out_b[e] = 0.f;
    }
    return;
  }
  const int npsplit = (nblk + blocks_per_split - 1) / blocks_per_split;  // splits over packed pages
  const int nsplit = npsplit + (ntail > 0 ? 1 : 0);
  if (split >= nsplit) return;
  const size_t pair = static_cast<size_t>(b) * hkv + kvh;
  float* pbase = part + pair * max_splits * kMaxGroup * kPartStride;
  if (split == npsplit) {
    // ---- the fp16 tail --------------------------------------------------------
    if (w == 0) {
      const uint16_t* qrow0 = q + (static_cast<size_t>(b) * hq + static_cast<size_t>(kvh) * G) * kHeadDim;
      const size_t tstride = static_cast<size_t>(hkv) * kHeadDim;
      const size_t t0 = (static_cast<size_t>(b) * kBlockTokens * hkv + kvh) * kHeadDim;
      tail_partial(qrow0, k_tail + t0, v_tail + t0, tstride, ntail, G, scale_log2,
                   pbase + static_cast<size_t>(split) * kMaxGroup * kPartStride, wacc[0], &wm[0][0], lane);
    }
  } else {
    // ---- packed page splits -------------------------------------------------
    const int blk0 = split * blocks_per_split;
    const int cnt = min(nblk, blk0 + blocks_per_split) - blk0;
    const int32_t* bt = block_table + static_cast<size_t>(b) * max_blocks + blk0;
    const int wu = __builtin_amdgcn_readfirstlane(w);  // wave index, known uniform: page ids load as scalars

    // ---- query loads, then the loads of this wave's first page ----------------
    // Both are issued before the query transform so that the page's HBM latency overlaps it.  Lane
    // l takes channels 2l and 2l + 1 of every head (heads past G re-read head 0 and are zeroed).
    const uint16_t* qb = q + (static_cast<size_t>(b) * hq + static_cast<size_t>(kvh) * G) * kHeadDim;
    uint32_t qraw[kMaxGroup];
  #pragma unroll
    for (int h = 0; h < kMaxGroup; ++h)
      qraw[h] = reinterpret_cast<const uint32_t*>(qb + (h < G ? h : 0) * kHeadDim)[lane];
    __builtin_amdgcn_sched_barrier(0);
    const int ch0 = coef_channel<KB>(lane);
    constexpr int ch1 = DecFormat<KB, VB, GS>::kCh1;
    // The prefetching kernel visits only the valid pages of the wave (w, w + 4, ...): an invalid id
    // is passed over by a scalar search and flagged, so its page loop has no per-page branch and the
    // loads of the next page land in the very registers of the current one (a branch around a bad
    // page would make the two paths hold the page in different registers, and the copies at their
    // join wait on every load).  The other kernels test each page as they load it.
    bool bad_page = false;
    auto next_valid = [&](int i) {  // first index >= i in steps of kWaves with a valid page id, or >= cnt
      for (; i < cnt; i += kWaves) {
        const int pid = bt[i];
        if (pid >= 0 && pid < num_pages) break;
        bad_page = true;
      }
      return i;
    };
    const int i0 = PF ? next_valid(wu) : wu;
    PageRegs<KB, VB, GS> A;
    load_page(A, page_ptrs<KB, VB, GS>(i0 < cnt ? bt[i0] : -1, num_pages, hkv, kvh, k_pool, v_pool), lane, n, g, ch0);
    __builtin_amdgcn_sched_barrier(0);

    // ---- rotated, scaled query ------------------------------------------------
    // Every wave transforms all heads itself (in registers) and writes the same values into the
    // shared per-lane array, so no workgroup barrier is needed; the wave's own page buffer serves as
    // scratch for the change of layout.
    auto& L = U.wl[w];
    float (*qt)[kHeadDim] = reinterpret_cast<float (*)[kHeadDim]>(&L.coef[0][0][0]);  // [kMaxGroup][128]
    const float qscale = kInvSqrt128 * scale_log2;
  #pragma unroll
    for (int h = 0; h < kMaxGroup; ++h) {
      float x0 = h < G ? half_bits_to_float(qraw[h] & 0xFFFFu) : 0.f;
      float x1 = h < G ? half_bits_to_float(qraw[h] >> 16) : 0.f;
      wave_fwht(x0, x1, lane);
      reinterpret_cast<float2*>(qt[h])[lane] = make_float2(x0 * qscale, x1 * qscale);
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    Mags M{0x4C004C00u, 0x54005400u, 0x44004400u, 0x64006400u};  // fp16 16 / 64 / 4 / 1024, twice
    asm volatile("" : "+v"(M.m16), "+v"(M.m64), "+v"(M.m4), "+v"(M.m1024));
    WaveState S;
    float qmax = 0.f;
  #pragma unroll
    for (int h = 0; h < kMaxGroup; ++h) {
      const float a = qt[h][ch0];
      const float c = qt[h][ch0 + ch1];
      qlane[lane][h] = a;
      qlane[lane][kMaxGroup + h] = c;
      qmax = fmaxf(qmax, fmaxf(fabsf(a), fabsf(c)));
    }
    S.qmax = wave_max_all(qmax);
    S.ql = &qlane[lane][0];
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    S.m_run = -INFINITY;
    S.l_run = 0.f;
  #pragma unroll
    for (int mt = 0; mt < 8; ++mt)
  #pragma unroll
      for (int r = 0; r < 4; ++r) S.acc[mt][r] = 0.f;
    // unused coefficient columns stay zero
    for (int e = lane; e < DecFormat<KB, VB, GS>::kHalves * 16 * kCoefStride; e += 64) (&L.coef[0][0][0])[e] = 0u;

    // ---- pages of this wave: w, w + 4, ... ---------------------------------------
    static_assert(!PF || DecFormat<KB, VB, GS>::kCanPrefetch, "format without a prefetching kernel");
    if constexpr (PF) {
      for (int i = i0; i < cnt;) {
        // the wave's next valid page (after its last one: no loads)
        const int nxt = next_valid(i + kWaves);
        PagePtrs nx = page_ptrs<KB, VB, GS>(bt[nxt < cnt ? nxt : i], num_pages, hkv, kvh, k_pool, v_pool);
        nx.load = nxt < cnt;
        process_page<KB, VB, GS, PF>(A, S, L, G, lane, g, lo_col, M, nx, ch0);
        i = nxt;
      }
    } else {
      const PagePtrs none{k_pool, v_pool, false, false};  // no next-page loads in this format
      if (wu < cnt) {
        if (A.ok) {
          process_page<KB, VB, GS, PF>(A, S, L, G, lane, g, lo_col, M, none, ch0);
        } else {
          bad_page = true;
        }
      }
      for (int i = wu + kWaves; i < cnt; i += kWaves) {
        load_page(A, page_ptrs<KB, VB, GS>(bt[i], num_pages, hkv, kvh, k_pool, v_pool), lane, n, g, ch0);
        if (A.ok) {
          process_page<KB, VB, GS, PF>(A, S, L, G, lane, g, lo_col, M, none, ch0);
        } else {
          bad_page = true;
        }
      }
    }
    if (bad_page && lane == 0 && flags) atomicOr(flags, kFlagBadPage);

    // ---- merge the four waves through LDS --------------------------------------
  #pragma unroll
    for (int mt = 0; mt < 8; ++mt)
  #pragma unroll
      for (int r = 0; r < 4; ++r) S.acc[mt][r] += dpp<kDppXor8>(S.acc[mt][r]);
    __syncthreads();  // every wave is out of the page loop: its page buffers may be reused
    if (!lo_col && hd < G) {
  #pragma unroll
      for (int mt = 0; mt < 8; ++mt)
  #pragma unroll
        for (int r = 0; r < 4; ++r) wacc[w][hd][16 * mt + 4 * g + r] = S.acc[mt][r];
      if (g == 0) {
        wm[w][hd] = S.m_run;
        wls[w][hd] = S.l_run;
      }
    }
    __syncthreads();
    for (int e = tid; e < G * kHeadDim; e += blockDim.x) {
      const int h = e >> 7, j = e & 127;
      float mx = -INFINITY;
  #pragma unroll
      for (int x = 0; x < kWaves; ++x) mx = fmaxf(mx, wm[x][h]);
      float o = 0.f, lsum = 0.f;
  #pragma unroll
      for (int x = 0; x < kWaves; ++x) {
        const float wgt = wm[x][h] == -INFINITY ? 0.f : ex2(wm[x][h] - mx);
        o = fmaf(wgt, wacc[x][h][j], o);
        lsum = fmaf(wgt, wls[x][h], lsum);
      }
      float* pp = pbase + (static_cast<size_t>(split) * kMaxGroup + h) * kPartStride;
      store_coherent(pp + j, o);
      if (j == 0) {
        store_coherent(pp + kHeadDim, mx);
        store_coherent(pp + kHeadDim + 1, lsum);
      }
    }
  }
  // Hand-off between workgroups without fences.  Every XCD has its own L2, so an agent-scope
  // fence would write back (release) or invalidate (acquire) this XCD's whole L2.  Instead the
  // partials are written and read with agent-scope atomic accesses, which go through to the
  // device-coherent level, and each wave waits until its stores are acknowledged before the
  // workgroup counts itself in.  Why this orders the hand-off on gfx950:
  //   * an agent-scope relaxed store or load is a global store / load with the sc1 bit (LLVM's
  //     AMDGPU memory model for the GFX940 family), which is performed at the device-coherent level
  //     and never served from, or left in, a non-coherent XCD-private L2 line;
  //   * on this GFX9-family target the vmcnt counter covers stores as well as loads (there is no
  //     separate store counter), so s_waitcnt vmcnt(0) returns only once every partial store of the
  //     wave is acknowledged, i.e. visible at that level; the barrier then covers all four waves;
  //   * the counter add is an agent-scope atomic, issued after that point in program order, and the
  //     last arriver issues its partial loads only after the add has returned (through the barrier
  //     that publishes last_flag), so every load sees every store that preceded an add.
  // Invariant that the argument needs: every access to the partials and counters, here, in the tail
  // split and in the merge, goes through store_coherent / load_coherent / the atomic add; no plain
  // load or store ever touches them.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(counters + pair, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last_flag = (prev == static_cast<uint32_t>(nsplit - 1));
  }
  __syncthreads();
  if (!last_flag) return;
  if (tid == 0) __hip_atomic_store(counters + pair, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // ready for the next call

  // ---- merge the splits (log-sum-exp) and undo the rotation ---------------
  // Wave w takes heads w and w + 4; lane l holds output channels 2l and 2l + 1, and lane s the
  // maximum and sum of split s (nsplit <= 64).
  for (int h = w; h < G; h += kWaves) {
    const float* ph = pbase + static_cast<size_t>(h) * kPartStride;
    constexpr size_t kSplitStride = static_cast<size_t>(kMaxGroup) * kPartStride;
    const int sp = lane < nsplit ? lane : 0;
    const float ms = load_coherent(ph + sp * kSplitStride + kHeadDim);
    const float ls = load_coherent(ph + sp * kSplitStride + kHeadDim + 1);
    const float msv = lane < nsplit ? ms : -INFINITY;
    const float mx = wave_max_all(msv);
    const float wgt = msv == -INFINITY ? 0.f : ex2(msv - mx);
    const float den = wave_sum_all(wgt * (lane < nsplit ? ls : 0.f));
    float n0 = 0.f, n1 = 0.f;
    for (int s0 = 0; s0 < nsplit; s0 += 8) {
      // eight splits at a time, so that their loads are in flight together
      float2 o[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int sk = s0 + k < nsplit ? s0 + k : 0;
        const float* pp = ph + sk * kSplitStride + 2 * lane;
        o[k] = make_float2(load_coherent(pp), load_coherent(pp + 1));
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int src = s0 + k < nsplit ? s0 + k : 0;
        const float wsrc = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wgt), src));
        const float wk = s0 + k < nsplit ? wsrc : 0.f;
        n0 = fmaf(wk, o[k].x, n0);
        n1 = fmaf(wk, o[k].y, n1);
      }
    }
    const float inv = den > 0.f ? 1.0f / den : 0.f;
    float x0 = n0 * inv, x1 = n1 * inv;
    wave_fwht(x0, x1, lane);
    reinterpret_cast<float2*>(out_b + static_cast<size_t>(h) * kHeadDim)[lane] =
        make_float2(x0 * kInvSqrt128, x1 * kInvSqrt128);
  }
}

hipError_t launch_decode(const void* q, const void* k_pool, const void* v_pool, int num_pages,
                         const int32_t* block_table, int max_blocks, const int32_t* seq_lens, const void* k_tail,
                         const void* v_tail, int batch, int hq, int hkv, int kbits, int vbits, int group,
                         int blocks_per_split, int max_splits, float scale_log2, float* out, float* part,
                         uint32_t* counters, uint32_t* flags, bool prefetch, hipStream_t stream) {
  auto kern = group == 64 ? (kbits == 8 ? (vbits == 4 ? decode_kernel<8, 4, 64, false> : decode_kernel<8, 2, 64, false>)
                                        : (vbits == 4 ? decode_kernel<4, 4, 64, false> : decode_kernel<4, 2, 64, false>))
                          : (kbits == 8 ? (vbits == 4 ? decode_kernel<8, 4, 128, false> : decode_kernel<8, 2, 128, false>)
                                        : (vbits == 4 ? decode_kernel<4, 4, 128, false> : decode_kernel<4, 2, 128, false>));
  if (prefetch && kbits == 4 && group == 128)
    kern = vbits == 4 ? decode_kernel<4, 4, 128, true> : decode_kernel<4, 2, 128, true>;
  hipLaunchKernelGGL(kern, dim3(hkv, batch, max_splits), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint8_t*>(k_pool),
                     static_cast<const uint8_t*>(v_pool), num_pages, block_table, max_blocks, seq_lens,
                     static_cast<const uint16_t*>(k_tail), static_cast<const uint16_t*>(v_tail), hq, hkv,
                     blocks_per_split, max_splits, scale_log2, out, part, counters, flags);
  return hipGetLastError();
}

}  // namespace kvarn
