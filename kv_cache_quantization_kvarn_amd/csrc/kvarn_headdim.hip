// KVarN quantisation, dequantisation and decode attention for heads of 64 or 256 channels (gfx950).
//
// The method is the one of the 128-channel kernels (KVarN blog post, section "KVarN Nasıl
// Çalışır?": per 128-token block, a Hadamard rotation along the channels, log2-variance row/column
// normalisation, round to nearest with fp16 scale and zero, packing), with D channels in place of
// 128: the rotation is the D-point Sylvester matrix over sqrt(D), row passes take the variance over
// D channels, key groups are one channel over `group` tokens and value groups one token over
// min(group, D) channels.  Page of one (block, KV head): codes | scale fp16[n] | zero fp16[n] |
// rho fp32[128] | gamma fp32[D]; keys token-major (4 bits: byte (D/2) t + j/2; 8 bits: byte D t + j),
// values channel-major (2 bits: byte 32 j + t/4; 4 bits: byte 64 j + t/2); scale/zero entry D h + j
// for keys (token half h), 128 h + t for values (channel group h).
//
// Quantiser.  One workgroup of D/32 waves per tile, wave w owning 128/(D/32) consecutive tokens.  The
// rotation runs on the matrix cores: H_D = H_{D/32} (x) H_32, so each output chunk of 32 channels is
// a chain of D/32 v_mfma_f32_16x16x32_f16 products of the wave's fp16 tokens with the exact +-1 H32
// block, each input chunk entering with the sign of its H_{D/32} entry (fp32 accumulation of exact
// products; the factor 1/sqrt(D) rides in the row normaliser).  Each lane then holds 4*(TW/16)
// tokens x 2*(D/32) channels, 64 values in every case:
//     token   T(i) = w*TW + 16*(i/4) + 4g + i%4,   channel C(c) = 32*(c/2) + 2n + c%2.
// Row moments reduce inside the wave (the 16 lanes of a DPP row hold every channel of their
// tokens); column moments reduce across the four rows of the wave and then across waves through
// LDS.  Every pass is centred in two sweeps (mean, then the mean square of the deviations), so no
// fp32 cancellation can lose digits, except the first row pass: with every column normaliser 1 its
// moments follow from the input (a token's mean is its first input value, its mean square the square
// sum of its inputs), and it is taken from them when every token of the wave keeps its mean square
// above twice its squared mean (at most one bit lost to cancellation), else centred as the others.
// The page is assembled in LDS (codes, scale/zero, rho, gamma) and written with 16-byte stores.
//
// Decode.  One workgroup of four waves per (sequence, KV head, split), the same split plan, partial
// layout and fence-free hand-off as the 128-channel decode.  With q~ = H q (orthonormal H) the page
// contractions run in the rotated basis,
//     score_t = 2^rho_t * sum_j q~_j 2^gamma_j (s c_tj + z)       (key group of channel j, half of t)
//     o~_j   += 2^gamma_j * sum_t p_t 2^rho_t (s c_tj + z)        (value group of token t, group of j)
// both code sums as dense products on the matrix cores (codes as exact fp16 operands, the fp32
// coefficients as fp16 hi + lo), with online softmax; the last workgroup of a (sequence, KV head)
// merges the splits and applies H.
#include "kvarn_codes.h"

namespace kvarn {

namespace {

template <int D>
struct HdGeom {
  static_assert(D == 64 || D == 128 || D == 256, "head size");
  static constexpr int kWaves = D / 32;                      // waves of a quantising workgroup
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kTokPerWave = kBlockTokens / kWaves;  // 64, 32 or 16
  static constexpr int kMT = kTokPerWave / 16;               // 16-token MFMA tiles per wave
  static constexpr int kNT = 4 * kMT;                        // tokens per lane
  static constexpr int kChunks = D / 32;                     // 32-channel chunks
  static constexpr int kNC = 2 * kChunks;                    // channels per lane
  static constexpr float kInvSqrtD = D == 64 ? 0.125f : (D == 256 ? 0.0625f : 0.08838834764831845f);
};

// Page geometry of one tensor (keys or values) at head size D, code width BITS, group size GS.
template <int D, bool V, int BITS, int GS>
struct HdPage {
  static constexpr int kVGroup = GS < D ? GS : D;  // channels per value group
  static constexpr int kGroups = V ? (D / kVGroup) * kBlockTokens : (kBlockTokens / GS) * D;
  static constexpr int kCode = kBlockTokens * D * BITS / 8;
  static constexpr int kScale = kCode;
  static constexpr int kZero = kCode + 2 * kGroups;
  static constexpr int kRho = kCode + 4 * kGroups;
  static constexpr int kGamma = kRho + 4 * kBlockTokens;
  static constexpr int kBytes = kGamma + 4 * D;
  static_assert(kBytes % 16 == 0, "pages are written in 16-byte pieces");
};

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// Sign patterns of the exact +-1 H32 operand of the rotation (Sylvester: entry (k, o) is
// (-1)^popcount(k & o)).  A lane's 8-long k-chunk k = 8g + i (i = 0..7) of output column o has
// signs (-1)^(popcount(i & (o & 7)) + popcount(g & (o >> 3))), since the two index parts share no
// bits.  Entry o7 + 8p holds the chunk for o & 7 = o7 and second parity p as four fp16 pairs
// (element i in half i % 2 of word i / 2); entry ^ 8 is its negation.
struct H32Signs {
  uint32_t w[16][4];
};
constexpr H32Signs make_h32_signs() {
  H32Signs t{};
  for (int e = 0; e < 16; ++e)
    for (int k = 0; k < 4; ++k) {
      uint32_t word = 0;
      for (int h = 0; h < 2; ++h) {
        const int i = 2 * k + h;
        int par = e >> 3;
        for (int b = 0; b < 3; ++b) par ^= ((i & e) >> b) & 1;
        word |= (0x3C00u | (par ? 0x8000u : 0u)) << (16 * h);
      }
      t.w[e][k] = word;
    }
  return t;
}
__constant__ const H32Signs kH32Signs = make_h32_signs();
__device__ __forceinline__ float lg2(float x) { return __builtin_amdgcn_logf(x); }

// Rounded product the compiler may not fuse into a later add (a constant group must get range 0).
__device__ __forceinline__ float mul_rn(float a, float b) {
  float p = a * b;
  asm("" : "+v"(p));
  return p;
}

// Sum / max over lanes l, l^16, l^32, l^48 (permlane swaps return the pair in lane order, so
// every lane combines the same values in the same order and gets identical bits).
__device__ __forceinline__ float rows_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float rows_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float wave_sump(float x) { return rows_sum(row16_sum(x)); }

// Transposed sum (or min, max) over the four 16-lane rows of a wave of NC values per lane: v[c] is
// combined over lanes l, l^16, l^32, l^48 and lane l of row g keeps the results of c = 4m + g, out[m].  A swap of the
// odd rows of one register with the even rows of another (v_permlane16_swap) pairs v[2k] of the even
// rows with v[2k + 1] of the odd ones, so one swap and one add per pair halve the values a lane holds;
// v_permlane32_swap does the same across the two row pairs.  3 NC / 4 swaps and adds, in place of
// four operations (two swaps, two adds) per value for separate sums.
template <int NC, class Op>
__device__ __forceinline__ void rows_transpose(const float (&v)[NC], float (&out)[NC / 4], Op op) {
  float h[NC / 2];
#pragma unroll
  for (int k = 0; k < NC / 2; ++k) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[2 * k]), __float_as_uint(v[2 * k + 1]),
                                                    false, false);
    h[k] = op(__uint_as_float(r[0]), __uint_as_float(r[1]));  // c = 2k + (row & 1)
  }
#pragma unroll
  for (int m = 0; m < NC / 4; ++m) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(h[2 * m]), __float_as_uint(h[2 * m + 1]),
                                                    false, false);
    out[m] = op(__uint_as_float(r[0]), __uint_as_float(r[1]));  // c = 4m + row
  }
}
template <int NC>
__device__ __forceinline__ void rows_transpose_sum(const float (&v)[NC], float (&out)[NC / 4]) {
  rows_transpose(v, out, [](float a, float b) { return a + b; });
}

// Transposed sum (or min, max) over the 16 lanes of a DPP row: lane n returns the row's total of v[n].  Each stage
// halves the values a lane holds: it keeps the half whose index bit k equals its own lane bit k and
// adds the partner's copy of that half, the partners being lanes n^1, n^2, (n - 4) mod 16 and n^8
// (each differs from n in bit k and agrees in the bits already used).  45 operations for 16 sums, in
// place of 64 for 16 separate reductions.
template <class Op>
__device__ __forceinline__ float row_transpose16(const float (&v)[16], int n, Op op) {
  const bool b0 = n & 1, b1 = n & 2, b2 = n & 4, b3 = n & 8;
  float a[8], b[4], c[2];
#pragma unroll
  for (int j = 0; j < 8; ++j) a[j] = op(b0 ? v[2 * j + 1] : v[2 * j], dpp<kDppXor1>(b0 ? v[2 * j] : v[2 * j + 1]));
#pragma unroll
  for (int j = 0; j < 4; ++j) b[j] = op(b1 ? a[2 * j + 1] : a[2 * j], dpp<kDppXor2>(b1 ? a[2 * j] : a[2 * j + 1]));
#pragma unroll
  for (int j = 0; j < 2; ++j) c[j] = op(b2 ? b[2 * j + 1] : b[2 * j], dpp<kDppRor4>(b2 ? b[2 * j] : b[2 * j + 1]));
  return op(b3 ? c[1] : c[0], dpp<kDppXor8>(b3 ? c[0] : c[1]));
}
// The same over 8 values: after three halving stages (partners n^1, n^2, (n - 4) mod 16) lanes n and
// n^8 hold the combination of v[n & 7] over their halves of the row, and one exchange across them
// completes it: lane n returns the row's total of v[n & 7].
template <class Op>
__device__ __forceinline__ float row_transpose8(const float (&v)[8], int n, Op op) {
  const bool b0 = n & 1, b1 = n & 2, b2 = n & 4;
  float a[4], b[2];
#pragma unroll
  for (int j = 0; j < 4; ++j) a[j] = op(b0 ? v[2 * j + 1] : v[2 * j], dpp<kDppXor1>(b0 ? v[2 * j] : v[2 * j + 1]));
#pragma unroll
  for (int j = 0; j < 2; ++j) b[j] = op(b1 ? a[2 * j + 1] : a[2 * j], dpp<kDppXor2>(b1 ? a[2 * j] : a[2 * j + 1]));
  const float c = op(b2 ? b[1] : b[0], dpp<kDppRor4>(b2 ? b[0] : b[1]));
  return op(c, dpp<kDppXor8>(c));
}
__device__ __forceinline__ float row_transpose_sum16(const float (&v)[16], int n) {
  return row_transpose16(v, n, [](float x, float y) { return x + y; });
}
__device__ __forceinline__ float wave_maxp(float x) { return rows_max(row16_max(x)); }

// code = round-half-even(clamp(x, 0, L)): the low mantissa bits of clamp + 1.5 * 2^23
template <int L>
__device__ __forceinline__ uint32_t rne_code(float x) {
  return __float_as_uint(fminf(fmaxf(x, 0.f), static_cast<float>(L)) + 12582912.0f) & 0xFFu;
}

// Shared memory of one quantising workgroup.
template <int D, int BITS_K, int BITS_V, int GS>
struct QhdLds {
  static constexpr int kPageMax = HdPage<D, false, BITS_K, GS>::kBytes > HdPage<D, true, BITS_V, GS>::kBytes
                                      ? HdPage<D, false, BITS_K, GS>::kBytes
                                      : HdPage<D, true, BITS_V, GS>::kBytes;
  uint8_t page[kPageMax];                          // the page image
  float part_a[HdGeom<D>::kWaves][D];              // per-wave column sums (or minima)
  float part_b[HdGeom<D>::kWaves][D];              // per-wave column maxima
  float col[D];                                    // column means, then 2^-gamma
  float qa[kBlockTokens / GS][D], qb[kBlockTokens / GS][D];  // key rounding factors per token half
  float rowv[D == 64 ? HdGeom<D>::kWaves : 1][64];  // 64 channels: per-wave token means, then 2^-rho / sqrt(D)
  alignas(16) float2 tokm[HdGeom<D>::kWaves][HdGeom<D>::kTokPerWave];  // first row pass: mean, mean square
  // 256 channels: value rounding factors per (token, channel group) of each wave
  alignas(16) float2 vfac[D == 256 ? HdGeom<D>::kWaves : 1][D == 256 ? 2 * HdGeom<D>::kTokPerWave : 1];
};

// Quantise one tile (block blk of head `head`, keys or values) into the page image, then store it.
template <bool kIsV, int D, int BITS, int GS, class Lds>
__device__ __forceinline__ void quantize_hd_tile(const uint16_t* __restrict__ in, int hkv, int blk, int head,
                                                 int page, bool ok, uint8_t* __restrict__ pool, Lds& s) {
  using Gm = HdGeom<D>;
  using Pg = HdPage<D, kIsV, BITS, GS>;
  constexpr int MT = Gm::kMT, NT = Gm::kNT, NC = Gm::kNC, CH = Gm::kChunks, TW = Gm::kTokPerWave, NW = Gm::kWaves;
  constexpr int L = (1 << BITS) - 1;
  constexpr float kInvBlock = 1.0f / kBlockTokens, kInvD = 1.0f / D;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, n = lane & 15, g = lane >> 4;
  auto tok = [&](int i) { return w * TW + 16 * (i >> 2) + 4 * g + (i & 3); };
  auto chan = [&](int c) { return 32 * (c >> 1) + 2 * n + (c & 1); };

  // ---- load: A operands xa[mt][gi] = X[w*TW + 16 mt + n][32 gi + 8 g .. + 7] --------------
  const size_t tstride = static_cast<size_t>(hkv) * D;
  const uint16_t* src = in + (static_cast<size_t>(blk) * kBlockTokens * hkv + head) * D;
  f16x8 xa[MT][CH];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int gi = 0; gi < CH; ++gi)
      xa[mt][gi] = *reinterpret_cast<const f16x8*>(src + static_cast<size_t>(w * TW + 16 * mt + n) * tstride +
                                                    32 * gi + 8 * g);
  // H32 block: B[k][col] = (-1)^popcount(k & o), input index k = 8g + i, output o = 2n + hh
  // (hbn = -hb), from the sign table
  f16x8 hb[2], hbn[2];
  {
    const int par = __popc(g & (n >> 2)) & 1;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int e = ((2 * n + hh) & 7) + 8 * par;
      hb[hh] = __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4*>(kH32Signs.w[e]));
      hbn[hh] = __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4*>(kH32Signs.w[e ^ 8]));
    }
  }
  // ---- rotation R' = sqrt(D) R: output chunk ho = sum_gi H_{D/32}[gi][ho] (X_gi H32) ---------
  float R[NT][NC];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int ho = 0; ho < CH; ++ho) {
        f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int gi = 0; gi < CH; ++gi) d = mfma16x16x32(xa[mt][gi], (__popc(gi & ho) & 1) ? hbn[hh] : hb[hh], d);
#pragma unroll
        for (int r = 0; r < 4; ++r) R[4 * mt + r][2 * ho + hh] = d[r];
      }
  // The first row pass's moments from the input: with every column normaliser still 1, a token's
  // mean over the rotated channels is its first input value (only row 0 of the +-1 matrix sums to
  // D) and its mean square the square sum of its inputs (the matrix times its transpose is D I).
  // Row g = 0 of the wave stores them for token w*TW + 16 mt + n.
  {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      float q = 0.f;
#pragma unroll
      for (int gi = 0; gi < CH; ++gi)
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
          const h2 x = {xa[mt][gi][i], xa[mt][gi][i + 1]};
          q = __builtin_amdgcn_fdot2(x, x, q, false);
        }
      q = rows_sum(q);
      if (g == 0) s.tokm[w][16 * mt + n] = make_float2(static_cast<float>(xa[mt][0][0]), q);
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
  }

  // ---- normalisation: rf = 2^-rho / sqrt(D) per token, cf = 2^-gamma per channel -------------
  float rho[NT], rf[NT], cf[NC];
  float rho_own = 0.f, rf_own = Gm::kInvSqrtD;  // 64 channels: normaliser of token tok(n), kept by lane n
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    rho[i] = 0.f;
    rf[i] = Gm::kInvSqrtD;
  }
#pragma unroll
  for (int c = 0; c < NC; ++c) cf[c] = 1.f;
  float gam_red = 0.f, cf_red = 1.f;  // gamma of channel tid, kept by reducer thread tid < D
#pragma unroll
  for (int it = 0; it < kNormIters; ++it) {
    // row pass: per token, over its D channels (16 lanes of a DPP row)
    if constexpr (NT == 16) {
      // 64 channels: the 16 lanes of a row share their 16 tokens, so a transposed sum leaves lane n
      // with token n's moment, lane n updates that token's normaliser, and the wave's LDS row hands
      // the means and then the factors back to every lane (wave-local: program order suffices)
      float* rv = &s.rowv[w][16 * g];
      float v = 0.f;  // variance of token tok(n)
      bool from_input = false;
      if (it == 0) {
        // one sweep from the input moments, unless a token's mean could cancel digits of its variance
        const float2 me = s.tokm[w][16 * (n >> 2) + 4 * g + (n & 3)];
        v = fmaf(-me.x, me.x, me.y);
        from_input = __builtin_amdgcn_ballot_w64(!(v >= 0.5f * me.y)) == 0;
      }
      if (!from_input) {
        float acc[16];
#pragma unroll
        for (int i = 0; i < NT; ++i) {
          float s1 = 0.f;
#pragma unroll
          for (int c = 0; c < NC; ++c) s1 = fmaf(R[i][c], cf[c], s1);
          acc[i] = s1;
        }
        rv[n] = row_transpose_sum16(acc, n) * kInvD;
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
        float mi[16];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float4 x = *reinterpret_cast<const float4*>(rv + 4 * k);
          mi[4 * k] = x.x; mi[4 * k + 1] = x.y; mi[4 * k + 2] = x.z; mi[4 * k + 3] = x.w;
        }
#pragma unroll
        for (int i = 0; i < NT; ++i) {
          float s2 = 0.f;
#pragma unroll
          for (int c = 0; c < NC; ++c) {
            const float d = fmaf(R[i][c], cf[c], -mi[i]);
            s2 = fmaf(d, d, s2);
          }
          acc[i] = s2;
        }
        v = row_transpose_sum16(acc, n) * kInvD;
      }
      rho_own += 0.5f * lg2(fmaf(v, rf_own * rf_own, kNormEps));
      rf_own = ex2(-rho_own) * Gm::kInvSqrtD;
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
      rv[n] = rf_own;
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float4 x = *reinterpret_cast<const float4*>(rv + 4 * k);
        rf[4 * k] = x.x; rf[4 * k + 1] = x.y; rf[4 * k + 2] = x.z; rf[4 * k + 3] = x.w;
      }
    } else {
      bool from_input = false;
      if (it == 0) {
        // one sweep from the input moments, unless a token's mean could cancel digits of its variance
        float vi[NT];
        bool fine = true;
#pragma unroll
        for (int i = 0; i < NT; ++i) {
          const float2 me = s.tokm[w][16 * (i >> 2) + 4 * g + (i & 3)];
          vi[i] = fmaf(-me.x, me.x, me.y);
          fine = fine && vi[i] >= 0.5f * me.y;
        }
        from_input = __builtin_amdgcn_ballot_w64(!fine) == 0;
        if (from_input) {
#pragma unroll
          for (int i = 0; i < NT; ++i) {
            rho[i] += 0.5f * lg2(fmaf(vi[i], rf[i] * rf[i], kNormEps));
            rf[i] = ex2(-rho[i]) * Gm::kInvSqrtD;
          }
        }
      }
      if (!from_input) {
#pragma unroll
        for (int i = 0; i < NT; ++i) {
          float s1 = 0.f;
#pragma unroll
          for (int c = 0; c < NC; ++c) s1 = fmaf(R[i][c], cf[c], s1);
          const float m = row16_sum(s1) * kInvD;
          float s2 = 0.f;
#pragma unroll
          for (int c = 0; c < NC; ++c) {
            const float d = fmaf(R[i][c], cf[c], -m);
            s2 = fmaf(d, d, s2);
          }
          const float v = row16_sum(s2) * kInvD;
          rho[i] += 0.5f * lg2(fmaf(v, rf[i] * rf[i], kNormEps));
          rf[i] = ex2(-rho[i]) * Gm::kInvSqrtD;
        }
      }
    }
    // column pass: per channel, over the 128 tokens (four rows of the wave, then the waves)
    {
      float s1[NC], t1[NC / 4];
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        s1[c] = 0.f;
#pragma unroll
        for (int i = 0; i < NT; ++i) s1[c] = fmaf(R[i][c], rf[i], s1[c]);
      }
      rows_transpose_sum(s1, t1);
#pragma unroll
      for (int m = 0; m < NC / 4; ++m) s.part_a[w][chan(4 * m + g)] = t1[m];
    }
    __syncthreads();
    if (tid < D) {
      float t = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) t += s.part_a[ww][tid];
      s.col[tid] = t * kInvBlock;
    }
    __syncthreads();
    {
      float s2[NC], t2[NC / 4];
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const float m = s.col[chan(c)];
        s2[c] = 0.f;
#pragma unroll
        for (int i = 0; i < NT; ++i) {
          const float d = fmaf(R[i][c], rf[i], -m);
          s2[c] = fmaf(d, d, s2[c]);
        }
      }
      rows_transpose_sum(s2, t2);
#pragma unroll
      for (int m = 0; m < NC / 4; ++m) s.part_a[w][chan(4 * m + g)] = t2[m];
    }
    __syncthreads();
    if (tid < D) {
      float t = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) t += s.part_a[ww][tid];
      gam_red += 0.5f * lg2(fmaf(t * kInvBlock, cf_red * cf_red, kNormEps));
      cf_red = ex2(-gam_red);
      s.col[tid] = cf_red;
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < NC; ++c) cf[c] = s.col[chan(c)];
  }
  // normalisers into the page image: rho of each token from lane n == 0 of its row, gamma from the reducer
  if constexpr (NT == 16) {
    *reinterpret_cast<float*>(&s.page[Pg::kRho + 4 * tok(n)]) = rho_own;
  } else if (n == 0) {
#pragma unroll
    for (int i = 0; i < NT; ++i) *reinterpret_cast<float*>(&s.page[Pg::kRho + 4 * tok(i)]) = rho[i];
  }
  if (tid < D) *reinterpret_cast<float*>(&s.page[Pg::kGamma + 4 * tid]) = gam_red;

  // ---- groups: min/max, fp16 scale and zero, rounding factors; codes packed as they are made ------
  if constexpr (!kIsV) {
    // key groups: channel j over the GS tokens of half h (a lane's tokens lie in one half)
    constexpr int KH = kBlockTokens / GS;
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
      for (int c = 0; c < NC; ++c) R[i][c] *= rf[i];
    {
      float a[NC], b[NC], ta[NC / 4], tb[NC / 4];
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        a[c] = R[0][c];
        b[c] = R[0][c];
#pragma unroll
        for (int i = 1; i < NT; ++i) {
          a[c] = fminf(a[c], R[i][c]);
          b[c] = fmaxf(b[c], R[i][c]);
        }
      }
      rows_transpose(a, ta, [](float x, float y) { return fminf(x, y); });
      rows_transpose(b, tb, [](float x, float y) { return fmaxf(x, y); });
#pragma unroll
      for (int m = 0; m < NC / 4; ++m) {
        s.part_a[w][chan(4 * m + g)] = ta[m];
        s.part_b[w][chan(4 * m + g)] = tb[m];
      }
    }
    __syncthreads();
    if (tid < KH * D) {
      const int ch = tid % D, h = tid / D;
      constexpr int WPH = NW / KH;  // waves per token half
      float mn = s.part_a[h * WPH][ch], mx = s.part_b[h * WPH][ch];
#pragma unroll
      for (int k = 1; k < WPH; ++k) {
        mn = fminf(mn, s.part_a[h * WPH + k][ch]);
        mx = fmaxf(mx, s.part_b[h * WPH + k][ch]);
      }
      const float cfc = s.col[ch];
      mn = mul_rn(mn, cfc);
      mx = mul_rn(mx, cfc);
      const uint32_t sb = float_to_half_bits((mx - mn) / static_cast<float>(L));
      const uint32_t zb = float_to_half_bits(mn);
      const float sf = half_bits_to_float(sb), zf = half_bits_to_float(zb);
      const float inv = sf > 0.f ? 1.0f / sf : 0.f;
      *reinterpret_cast<uint16_t*>(&s.page[Pg::kScale + 2 * (D * h + ch)]) = static_cast<uint16_t>(sb);
      *reinterpret_cast<uint16_t*>(&s.page[Pg::kZero + 2 * (D * h + ch)]) = static_cast<uint16_t>(zb);
      s.qa[h][ch] = cfc * inv;
      s.qb[h][ch] = -zf * inv;
    }
    __syncthreads();
    const int kh = (w * TW) / GS;
#pragma unroll
    for (int ho = 0; ho < CH; ++ho) {
      // the rounding factors of this lane's channel pair (2 ho, 2 ho + 1): one byte of each token
      const float qa0 = s.qa[kh][chan(2 * ho)], qb0 = s.qb[kh][chan(2 * ho)];
      const float qa1 = s.qa[kh][chan(2 * ho + 1)], qb1 = s.qb[kh][chan(2 * ho + 1)];
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        const uint32_t c0 = rne_code<L>(fmaf(R[i][2 * ho], qa0, qb0));
        const uint32_t c1 = rne_code<L>(fmaf(R[i][2 * ho + 1], qa1, qb1));
        if constexpr (BITS == 4)
          s.page[(D / 2) * tok(i) + 16 * ho + n] = static_cast<uint8_t>(c0 | (c1 << 4));
        else
          *reinterpret_cast<uint16_t*>(&s.page[D * tok(i) + 32 * ho + 2 * n]) = static_cast<uint16_t>(c0 | (c1 << 8));
      }
    }
  } else {
    // value groups: token t over the channels of group vg (a chunk pair's worth or more); a byte of
    // the page holds one channel's codes of four consecutive tokens, those of one 4-token row of a tile
    constexpr int VGC = Pg::kVGroup, NVG = D / VGC, CPG = NC / NVG;  // lane channels per group
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
      for (int c = 0; c < NC; ++c) R[i][c] *= cf[c];
    // 64 channels (one value group per token): lane n finds token tok(n)'s minimum and maximum by
    // transposed reductions, computes its scale, zero and rounding factors once, and the wave's LDS
    // row (the first row pass's moment slots, free by now) hands the factors to every lane
    [[maybe_unused]] float qv[NT][2];
    [[maybe_unused]] float qw[NT][2][2];  // 256 channels: [token][group][qa, qb]
    if constexpr (NT == 4 && NVG == 2) {
      // 256 channels: 4 tokens x 2 channel groups per lane, so the row's 16 lanes reduce the 8 groups
      // transposed, lanes n and n^8 ending with group (token (n & 7) / 2, half n & 1); each such lane
      // computes that group's scale, zero and factors once and the wave's LDS rows hand them back
      float a[8], b[8];
#pragma unroll
      for (int i = 0; i < NT; ++i)
#pragma unroll
        for (int vg = 0; vg < NVG; ++vg) {
          float x = R[i][CPG * vg], y = R[i][CPG * vg];
#pragma unroll
          for (int c = CPG * vg + 1; c < CPG * (vg + 1); ++c) {
            x = fminf(x, R[i][c]);
            y = fmaxf(y, R[i][c]);
          }
          a[2 * i + vg] = x;
          b[2 * i + vg] = y;
        }
      const int io = (n & 7) >> 1, vo = n & 1;  // this lane's (token, group)
      const float rfo = io == 0 ? rf[0] : io == 1 ? rf[1] : io == 2 ? rf[2] : rf[3];
      const float mn = mul_rn(row_transpose8(a, n, [](float x, float y) { return fminf(x, y); }), rfo);
      const float mx = mul_rn(row_transpose8(b, n, [](float x, float y) { return fmaxf(x, y); }), rfo);
      const uint32_t sb = float_to_half_bits((mx - mn) / static_cast<float>(L));
      const uint32_t zb = float_to_half_bits(mn);
      const float sf = half_bits_to_float(sb), zf = half_bits_to_float(zb);
      const float inv = sf > 0.f ? 1.0f / sf : 0.f;
      float2* vf = &s.vfac[w][0];
      if (n < 8) {
        *reinterpret_cast<uint16_t*>(&s.page[Pg::kScale + 2 * (kBlockTokens * vo + tok(io))]) =
            static_cast<uint16_t>(sb);
        *reinterpret_cast<uint16_t*>(&s.page[Pg::kZero + 2 * (kBlockTokens * vo + tok(io))]) =
            static_cast<uint16_t>(zb);
        vf[8 * g + 2 * io + vo] = make_float2(rfo * inv, -zf * inv);
      }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float4 x = *reinterpret_cast<const float4*>(&vf[8 * g + 2 * k]);
        qw[k][0][0] = x.x;
        qw[k][0][1] = x.y;
        qw[k][1][0] = x.z;
        qw[k][1][1] = x.w;
      }
    }
    if constexpr (NT == 16) {
      static_assert(NVG == 1, "one value group per token at 64 channels");
      float a[16], b[16];
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        a[i] = R[i][0];
        b[i] = R[i][0];
#pragma unroll
        for (int c = 1; c < NC; ++c) {
          a[i] = fminf(a[i], R[i][c]);
          b[i] = fmaxf(b[i], R[i][c]);
        }
      }
      const float mn = mul_rn(row_transpose16(a, n, [](float x, float y) { return fminf(x, y); }), rf_own);
      const float mx = mul_rn(row_transpose16(b, n, [](float x, float y) { return fmaxf(x, y); }), rf_own);
      const uint32_t sb = float_to_half_bits((mx - mn) / static_cast<float>(L));
      const uint32_t zb = float_to_half_bits(mn);
      const float sf = half_bits_to_float(sb), zf = half_bits_to_float(zb);
      const float inv = sf > 0.f ? 1.0f / sf : 0.f;
      *reinterpret_cast<uint16_t*>(&s.page[Pg::kScale + 2 * tok(n)]) = static_cast<uint16_t>(sb);
      *reinterpret_cast<uint16_t*>(&s.page[Pg::kZero + 2 * tok(n)]) = static_cast<uint16_t>(zb);
      float2* tq = &s.tokm[w][0];
      tq[16 * (n >> 2) + 4 * g + (n & 3)] = make_float2(rf_own * inv, -zf * inv);
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const float4 x = *reinterpret_cast<const float4*>(&tq[16 * mt + 4 * g + 2 * h2]);
          qv[4 * mt + 2 * h2][0] = x.x;
          qv[4 * mt + 2 * h2][1] = x.y;
          qv[4 * mt + 2 * h2 + 1][0] = x.z;
          qv[4 * mt + 2 * h2 + 1][1] = x.w;
        }
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int t0 = w * TW + 16 * mt + 4 * g;  // the four consecutive tokens of this lane
#pragma unroll
      for (int vg = 0; vg < NVG; ++vg) {
        float qa[4], qb[4];
        if constexpr (NT == 16) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            qa[r] = qv[4 * mt + r][0];
            qb[r] = qv[4 * mt + r][1];
          }
        } else if constexpr (NT == 4 && NVG == 2) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            qa[r] = qw[r][vg][0];
            qb[r] = qw[r][vg][1];
          }
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = 4 * mt + r;
            float a = R[i][CPG * vg], b = R[i][CPG * vg];
#pragma unroll
            for (int c = CPG * vg + 1; c < CPG * (vg + 1); ++c) {
              a = fminf(a, R[i][c]);
              b = fmaxf(b, R[i][c]);
            }
            const float mn = mul_rn(row16_min(a), rf[i]);
            const float mx = mul_rn(row16_max(b), rf[i]);
            const uint32_t sb = float_to_half_bits((mx - mn) / static_cast<float>(L));
            const uint32_t zb = float_to_half_bits(mn);
            const float sf = half_bits_to_float(sb), zf = half_bits_to_float(zb);
            const float inv = sf > 0.f ? 1.0f / sf : 0.f;
            if (n == 0) {
              *reinterpret_cast<uint16_t*>(&s.page[Pg::kScale + 2 * (kBlockTokens * vg + tok(i))]) =
                  static_cast<uint16_t>(sb);
              *reinterpret_cast<uint16_t*>(&s.page[Pg::kZero + 2 * (kBlockTokens * vg + tok(i))]) =
                  static_cast<uint16_t>(zb);
            }
            qa[r] = rf[i] * inv;
            qb[r] = -zf * inv;
          }
        }
#pragma unroll
        for (int c = CPG * vg; c < CPG * (vg + 1); ++c) {
          uint32_t k4[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) k4[r] = rne_code<L>(fmaf(R[4 * mt + r][c], qa[r], qb[r]));
          if constexpr (BITS == 2)
            s.page[32 * chan(c) + t0 / 4] = static_cast<uint8_t>(k4[0] | (k4[1] << 2) | (k4[2] << 4) | (k4[3] << 6));
          else
            *reinterpret_cast<uint16_t*>(&s.page[64 * chan(c) + t0 / 2]) =
                static_cast<uint16_t>(k4[0] | (k4[1] << 4) | (k4[2] << 8) | (k4[3] << 12));
        }
      }
    }
  }
  __syncthreads();
  if (ok) {
    uint8_t* dst = pool + (static_cast<size_t>(page) * hkv + head) * Pg::kBytes;
    for (int e = tid; e < Pg::kBytes / 16; e += Gm::kThreads)
      reinterpret_cast<uint4*>(dst)[e] = reinterpret_cast<const uint4*>(s.page)[e];
  }
}

}  // namespace

// One workgroup per (block, KV head, K or V): tile index 2 (block * hkv + head) + (0 keys, 1 values).
template <int D, int KB, int VB, int GS>
__global__ __launch_bounds__(HdGeom<D>::kThreads, D == 64 ? 3 : 1) void quantize_hd_kernel(
    const uint16_t* __restrict__ kin, const uint16_t* __restrict__ vin, int hkv,
    const int32_t* __restrict__ dst_pages, uint8_t* __restrict__ k_pool, uint8_t* __restrict__ v_pool,
    int num_pages, uint32_t* __restrict__ flags) {
  __shared__ __align__(16) QhdLds<D, KB, VB, GS> lds;
  const int tile = blockIdx.x;
  const bool is_v = tile & 1;
  const int bh = tile >> 1;
  const int blk = bh / hkv, head = bh - blk * hkv;
  const int page = dst_pages[blk];
  const bool ok = page >= 0 && page < num_pages;
  if (!ok && threadIdx.x == 0 && flags && !is_v) atomicOr(flags, kFlagBadPage);
  if (is_v)
    quantize_hd_tile<true, D, VB, GS>(vin, hkv, blk, head, page, ok, v_pool, lds);
  else
    quantize_hd_tile<false, D, KB, GS>(kin, hkv, blk, head, page, ok, k_pool, lds);
}

// Test / inspection export: fp32 K^ or V^ (original basis) of TT tokens of one tile.
template <int D>
__global__ __launch_bounds__(256) void dequantize_hd_kernel(const uint8_t* __restrict__ k_pool,
                                                            const uint8_t* __restrict__ v_pool, int num_pages,
                                                            const int32_t* __restrict__ pages, int hkv, int kbits,
                                                            int vbits, int group, float* __restrict__ k_out,
                                                            float* __restrict__ v_out, uint32_t* __restrict__ flags) {
  constexpr int TT = D >= 256 ? 64 : kBlockTokens;  // tokens per workgroup
  constexpr int NPART = kBlockTokens / TT;
  __shared__ float buf[TT][D + 1];
  const int part = blockIdx.x % NPART, tile = blockIdx.x / NPART;
  const bool is_v = tile & 1;
  const int bh = tile >> 1, blk = bh / hkv, head = bh - blk * hkv;
  float* out = is_v ? v_out : k_out;
  if (out == nullptr) return;
  const int page = pages[blk];
  if (page < 0 || page >= num_pages) {
    if (threadIdx.x == 0 && part == 0 && flags) atomicOr(flags, kFlagBadPage);
    return;
  }
  const int bits = is_v ? vbits : kbits;
  const int vgc = group < D ? group : D;
  const int ngroups = is_v ? (D / vgc) * kBlockTokens : (kBlockTokens / group) * D;
  const int code_bytes = kBlockTokens * D * bits / 8;
  const int page_bytes = code_bytes + 4 * ngroups + 4 * kBlockTokens + 4 * D;
  const uint8_t* pb = (is_v ? v_pool : k_pool) + (static_cast<size_t>(page) * hkv + head) * page_bytes;
  const uint16_t* sc = reinterpret_cast<const uint16_t*>(pb + code_bytes);
  const uint16_t* zr = sc + ngroups;
  const float* rho = reinterpret_cast<const float*>(pb + code_bytes + 4 * ngroups);
  const float* gam = rho + kBlockTokens;
  for (int e = threadIdx.x; e < TT * D; e += blockDim.x) {
    const int tl = e / D, j = e - tl * D, t = part * TT + tl;
    uint32_t c;
    int gi;
    if (is_v) {
      c = bits == 4 ? (pb[64 * j + (t >> 1)] >> (4 * (t & 1))) & 15u : (pb[32 * j + (t >> 2)] >> (2 * (t & 3))) & 3u;
      gi = kBlockTokens * (j / vgc) + t;
    } else {
      c = bits == 8 ? pb[D * t + j] : (pb[(D / 2) * t + (j >> 1)] >> (4 * (j & 1))) & 15u;
      gi = D * (t / group) + j;
    }
    buf[tl][j] = fmaf(half_bits_to_float(sc[gi]), static_cast<float>(c), half_bits_to_float(zr[gi])) *
                 exp2f(rho[t] + gam[j]);
  }
  __syncthreads();
  for (int half = 1; half < D; half <<= 1) {  // fast Walsh-Hadamard transform of every token row
    for (int u = threadIdx.x; u < TT * D / 2; u += blockDim.x) {
      const int tl = u / (D / 2), p = u - tl * (D / 2);
      const int i = (p / half) * 2 * half + (p % half);
      const float a = buf[tl][i], b = buf[tl][i + half];
      buf[tl][i] = a + b;
      buf[tl][i + half] = a - b;
    }
    __syncthreads();
  }
  for (int e = threadIdx.x; e < TT * D; e += blockDim.x) {
    const int tl = e / D, j = e - tl * D, t = part * TT + tl;
    out[(static_cast<size_t>(blk) * kBlockTokens + t) * hkv * D + static_cast<size_t>(head) * D + j] =
        buf[tl][j] * HdGeom<D>::kInvSqrtD;
  }
}

namespace {

constexpr int kDecWaves = 4;
constexpr int kDecThreads = 64 * kDecWaves;

// Agent-scope relaxed accesses to the split partials (they go to the device-coherent level, which
// every XCD sees; see the 128-channel decode for the hand-off argument).
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// In-LDS fast Walsh-Hadamard transform of kMaxGroup rows of D values (unnormalised).
template <int D>
__device__ __forceinline__ void lds_fwht_rows(float (*x)[D], int rows) {
  for (int half = 1; half < D; half <<= 1) {
    for (int u = threadIdx.x; u < rows * D / 2; u += blockDim.x) {
      const int r = u / (D / 2), p = u - r * (D / 2);
      const int i = (p / half) * 2 * half + (p % half);
      const float a = x[r][i], b = x[r][i + half];
      x[r][i] = a + b;
      x[r][i + half] = a - b;
    }
    __syncthreads();
  }
}

// x as fp16 hi + lo: hi the nearest fp16 of x, lo the nearest fp16 of x - hi (exact in fp32), about
// 22 significant bits together.  hi is pinned so that the value stored and the value subtracted agree.
__device__ __forceinline__ void split_hl(float x, _Float16& hi, _Float16& lo) {
  _Float16 h = static_cast<_Float16>(x);
  asm("" : "+v"(h));
  hi = h;
  lo = static_cast<_Float16>(x - static_cast<float>(h));
}

// Slot of channel j in a key coefficient column: 8-channel groups in the element order of key_codes
// (channels 0,4,1,5,2,6,3,7) for 4-bit codes, in channel order for 8-bit codes.
template <int KB>
__device__ __forceinline__ int key_slot(int j) {
  return KB == 4 ? (j & ~7) + 2 * (j & 3) + ((j >> 2) & 1) : j;
}
// Offset the code conversion adds to the code of channel j (kvarn_codes.h).
template <int KB>
__device__ __forceinline__ float key_offset(int j) {
  return KB == 8 ? 1024.f : ((j & 3) == 1 ? 64.f : 16.f);
}
// Slot of token t in a value weight column: 16-token groups in the element order of value_codes and
// value_codes4 (tokens 0,8,1,9,2,10,3,11 then 4,12,5,13,6,14,7,15).
__device__ __forceinline__ int value_slot(int t) {
  const int o = t & 15;
  return (t & ~15) + 8 * ((o & 7) >> 2) + 2 * (o & 3) + (o >> 3);
}
template <int VB>
__device__ __forceinline__ float value_offset(int t) {
  return VB == 4 ? 64.f : ((t & 1) ? 16.f : 4.f);
}

// The end of every split workgroup of the head-size decodes, after its partial (o~, m, l per head) is
// stored: count in, and the last workgroup of the (sequence, KV head) merges the splits (log-sum-exp)
// and writes o = H o~ / sqrt(D).  Hand-off without fences, as in the 128-channel decode: partials go
// through agent-scope (sc1) atomic accesses, vmcnt(0) covers the stores before the workgroup counts in
// with an agent-scope add, and every access to partials and counters is one of these.
template <int D>
__device__ __forceinline__ void split_merge(float (&qt)[kMaxGroup][D], float (&sm)[64][kMaxGroup],
                                            float (&sl)[64][kMaxGroup], int& last, const float* __restrict__ pbase,
                                            uint32_t* __restrict__ counter, int nsplit, int G, float* __restrict__ out_b) {
  constexpr int PS = D + 2;
  const int tid = threadIdx.x;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last = prev == static_cast<uint32_t>(nsplit - 1);
  }
  __syncthreads();
  if (!last) return;
  if (tid == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (int e = tid; e < nsplit * kMaxGroup; e += kDecThreads) {
    const int sp = e / kMaxGroup, h = e - sp * kMaxGroup;
    const float* pp = pbase + (static_cast<size_t>(sp) * kMaxGroup + h) * PS;
    sm[sp][h] = h < G ? load_coherent(pp + D) : -INFINITY;
    sl[sp][h] = h < G ? load_coherent(pp + D + 1) : 0.f;
  }
  __syncthreads();
  for (int e = tid; e < kMaxGroup * D; e += kDecThreads) {
    const int h = e / D, j = e - h * D;
    float val = 0.f;
    if (h < G) {
      float mx = -INFINITY;
      for (int sp = 0; sp < nsplit; ++sp) mx = fmaxf(mx, sm[sp][h]);
      float num = 0.f, den = 0.f;
      for (int sp = 0; sp < nsplit; ++sp) {
        const float ms = sm[sp][h];
        const float wgt = ms == -INFINITY ? 0.f : ex2(ms - mx);
        den = fmaf(wgt, sl[sp][h], den);
        num = fmaf(wgt, load_coherent(pbase + (static_cast<size_t>(sp) * kMaxGroup + h) * PS + j), num);
      }
      val = den > 0.f ? num / den : 0.f;
    }
    qt[h][j] = val;
  }
  __syncthreads();
  lds_fwht_rows<D>(qt, kMaxGroup);
  for (int e = tid; e < G * D; e += kDecThreads) out_b[e] = qt[e / D][e % D] * HdGeom<D>::kInvSqrtD;
}

template <int D, int KB, int VB, int GS>
struct DhdLds {
  using PK = HdPage<D, false, KB, GS>;
  using PV = HdPage<D, true, VB, GS>;
  static constexpr int KH = kBlockTokens / GS;       // key groups per channel (token halves)
  static constexpr int NVG = D / PV::kVGroup;        // value groups per token (channel groups)
  static constexpr int kKStride = D + 8;             // fp16 per key coefficient column (padded)
  static constexpr int kVStride = kBlockTokens + 8;  // fp16 per value weight column (padded)
  float qt[kMaxGroup][D];                            // q~ per head; the split's o~, then the output
  _Float16 kcoef[KH][16][kKStride];                  // key B operand: hi (columns 0-7), lo (8-15) of a_j sa
  _Float16 vcoef[NVG][16][kVStride];                 // value B operand: hi, lo of w_t sw
  float score[kMaxGroup][kBlockTokens];              // scores (log2 units)
  float krho[kBlockTokens];                          // 2^rho_t / sa * scale (keys)
  float vsr[NVG][kBlockTokens], vzr[NVG][kBlockTokens];  // 2^rho_t s sw, 2^rho_t z sw (values)
  float gsv[D];                                      // 2^gamma_j / sw (values)
  float bpart[kDecWaves][KH][kMaxGroup];             // per-wave sums of b sa, offsets removed
  float upart[kDecWaves][NVG][kMaxGroup];            // per-wave sums of u sw, offsets removed
  float red[kDecWaves][2];                           // per-wave maxima of the key and value scale factors
  float qred[kDecWaves];                             // per-wave maxima of |q~|
  float alpha[kMaxGroup];                            // this page's rescale factor per head
  float mrun[kMaxGroup], lrun[kMaxGroup];            // running maximum and sum per head
  float sm[64][kMaxGroup], sl[64][kMaxGroup];        // split maxima and sums during the merge
  int last;
};

}  // namespace

// Decode over pages of D-channel heads: grid (Hkv, batch, splits), four waves per workgroup.
// Per page, with the notation of the 128-channel decode (a_j = q~_j 2^gamma_j s_j, b = sum_j q~_j
// 2^gamma_j z_j; w_t = p_t 2^rho_t s_t, u = sum_t p_t 2^rho_t z_t):
//   (1) largest key and value scale factors of the page, then fp16 hi/lo operands a_j sa and the
//       constants b, in power-of-two page scales sa and sw that keep every operand below 2^14;
//   (2) scores on the matrix cores: wave w takes tokens 32w .. 32w+31 (two 16-token tiles, D/32 chained
//       v_mfma_f32_16x16x32_f16 each), lane (n, g) loading its token's codes of channels
//       (D/4)g .. (D/4)(g+1)-1; the columns are the heads' hi and lo coefficients;
//   (3) online softmax per head (wave w: heads w and w + 4), writing the value operands w_t sw;
//   (4) values on the matrix cores: wave w takes channels (D/4)w .. (D/4)(w+1)-1, 16 per tile, lane
//       (n, g) loading its channel's codes of tokens 32g .. 32g+31; o~_j <- alpha o~_j + 2^gamma_j (...).
// Codes enter as fp16 off + c (kvarn_codes.h); the offsets leave with sums of the fp16 operands used.
// Each part of a page is loaded into registers right after its last use on the previous page.
template <int D, int KB, int VB, int GS>
__global__ __launch_bounds__(kDecThreads) void decode_hd_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ k_pool, const uint8_t* __restrict__ v_pool,
    int num_pages, const int32_t* __restrict__ block_table, int max_blocks, const int32_t* __restrict__ seq_lens,
    int hq, int hkv, int blocks_per_split, int max_splits, float scale_log2, float* __restrict__ out,
    float* __restrict__ part, uint32_t* __restrict__ counters, uint32_t* __restrict__ flags) {
  using L = DhdLds<D, KB, VB, GS>;
  using PK = typename L::PK;
  using PV = typename L::PV;
  constexpr int KH = L::KH, NVG = L::NVG, VGC = PV::kVGroup;
  constexpr int PS = D + 2;              // partial stride: o~[D], m, l
  constexpr int KC = D / 32;             // 32-channel steps of a key tile
  constexpr int KWT = D * KB / 128;      // key code dwords of a lane per token tile
  constexpr int VMT = D / 64;            // 16-channel value tiles per wave
  constexpr int VWT = VB;                // value code dwords of a lane per value tile (32 tokens)
  static_assert(KWT == 2 || KWT % 4 == 0, "key code loads");
  __shared__ __align__(16) L s;

  const int kvh = blockIdx.x, b = blockIdx.y, split = blockIdx.z;
  const int G = hq / hkv;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, n = lane & 15, g = lane >> 4;
  const int sl_b = seq_lens[b];
  float* out_b = out + (static_cast<size_t>(b) * hq + static_cast<size_t>(kvh) * G) * D;
  const bool bad = sl_b < 0 || sl_b > max_blocks * kBlockTokens || (sl_b & (kBlockTokens - 1)) != 0;
  const int nblk = bad ? 0 : sl_b / kBlockTokens;
  if (nblk == 0) {
    if (split == 0) {
      if (bad && tid == 0 && flags) atomicOr(flags, kFlagBadSeqLen);
      for (int e = tid; e < G * D; e += kDecThreads) out_b[e] = 0.f;
    }
    return;
  }
  const int nsplit = (nblk + blocks_per_split - 1) / blocks_per_split;
  if (split >= nsplit) return;
  const size_t pair = static_cast<size_t>(b) * hkv + kvh;
  float* pbase = part + pair * max_splits * kMaxGroup * PS;

  // ---- q~ = H q / sqrt(D) for the G heads (rows past G are zero), and max |q~| -------------------
  const uint16_t* qb = q + (static_cast<size_t>(b) * hq + static_cast<size_t>(kvh) * G) * D;
  for (int e = tid; e < kMaxGroup * D; e += kDecThreads) {
    const int h = e / D, j = e - h * D;
    s.qt[h][j] = h < G ? half_bits_to_float(qb[h * D + j]) : 0.f;
  }
  __syncthreads();
  lds_fwht_rows<D>(s.qt, kMaxGroup);
  {
    float qm = 0.f;
    for (int e = tid; e < kMaxGroup * D; e += kDecThreads) {
      const float v = s.qt[e / D][e % D] * HdGeom<D>::kInvSqrtD;
      s.qt[e / D][e % D] = v;
      qm = fmaxf(qm, fabsf(v));
    }
    qm = wave_maxp(qm);
    if (lane == 0) s.qred[w] = qm;
  }
  if (tid < kMaxGroup) {
    s.mrun[tid] = -INFINITY;
    s.lrun[tid] = 0.f;
  }
  __syncthreads();
  const float qmax = fmaxf(fmaxf(s.qred[0], s.qred[1]), fmaxf(s.qred[2], s.qred[3]));

  // exponent patterns of the code conversions, kept in vector registers
  uint32_t mag4 = 0x44004400u, mag16 = 0x4C004C00u, mag64 = 0x54005400u, mag1024 = 0x64006400u;
  asm volatile("" : "+v"(mag4), "+v"(mag16), "+v"(mag64), "+v"(mag1024));

  const int p0 = split * blocks_per_split;
  const int p1 = min(nblk, p0 + blocks_per_split);
  const int32_t* bt_b = block_table + static_cast<size_t>(b) * max_blocks;
  bool bad_page = false;
  // next valid page at or after position pi (page ids outside [0, num_pages) are skipped)
  auto next_valid = [&](int pi) {
    for (; pi < p1; ++pi) {
      const int pg = bt_b[pi];
      if (pg >= 0 && pg < num_pages) return pi;
      bad_page = true;
    }
    return p1;
  };
  const int kh_w = (32 * w) / GS;  // key group (token half) of this wave's tokens
  // One page's data in registers.
  uint32_t kw[2][KWT];   // key codes: token tile mt, token 32w + 16mt + n, channel quarter g
  uint32_t vw[VMT][VWT];  // value codes: channel (D/4)w + 16mt + n, tokens 32g .. 32g+31
  float m_kg = 0.f, m_ks[KH], m_kz[KH], m_vg = 0.f;  // channel tid: key gamma, scale, zero; value gamma
  float m_kr = 0.f, m_vr = 0.f, m_vs[NVG], m_vz[NVG];  // token tid: key rho; value rho, scale, zero
#pragma unroll
  for (int kh = 0; kh < KH; ++kh) m_ks[kh] = m_kz[kh] = 0.f;
#pragma unroll
  for (int vg = 0; vg < NVG; ++vg) m_vs[vg] = m_vz[vg] = 0.f;
  auto page_k = [&](int pi) { return k_pool + (static_cast<size_t>(bt_b[pi]) * hkv + kvh) * PK::kBytes; };
  auto page_v = [&](int pi) { return v_pool + (static_cast<size_t>(bt_b[pi]) * hkv + kvh) * PV::kBytes; };
  auto load_meta = [&](int pi) {
    const uint8_t* kp = page_k(pi);
    const uint8_t* vp = page_v(pi);
    if (tid < D) {
      m_kg = reinterpret_cast<const float*>(kp + PK::kGamma)[tid];
      m_vg = reinterpret_cast<const float*>(vp + PV::kGamma)[tid];
#pragma unroll
      for (int kh = 0; kh < KH; ++kh) {
        m_ks[kh] = half_bits_to_float(reinterpret_cast<const uint16_t*>(kp + PK::kScale)[D * kh + tid]);
        m_kz[kh] = half_bits_to_float(reinterpret_cast<const uint16_t*>(kp + PK::kZero)[D * kh + tid]);
      }
    }
    if (tid < kBlockTokens) {
      m_kr = reinterpret_cast<const float*>(kp + PK::kRho)[tid];
      m_vr = reinterpret_cast<const float*>(vp + PV::kRho)[tid];
#pragma unroll
      for (int vg = 0; vg < NVG; ++vg) {
        m_vs[vg] = half_bits_to_float(reinterpret_cast<const uint16_t*>(vp + PV::kScale)[kBlockTokens * vg + tid]);
        m_vz[vg] = half_bits_to_float(reinterpret_cast<const uint16_t*>(vp + PV::kZero)[kBlockTokens * vg + tid]);
      }
    }
  };
  auto load_k = [&](int pi) {
    const uint8_t* kp = page_k(pi);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const uint8_t* src = kp + (32 * w + 16 * mt + n) * (D * KB / 8) + g * (D * KB / 32);
      if constexpr (KWT == 2) {
        const u32x2 x = *reinterpret_cast<const u32x2*>(src);
        kw[mt][0] = x[0];
        kw[mt][1] = x[1];
      } else {
#pragma unroll
        for (int k4 = 0; k4 < KWT / 4; ++k4) {
          const u32x4 x = *reinterpret_cast<const u32x4*>(src + 16 * k4);
#pragma unroll
          for (int e = 0; e < 4; ++e) kw[mt][4 * k4 + e] = x[e];
        }
      }
    }
  };
  auto load_v = [&](int pi) {
    const uint8_t* vp = page_v(pi);
#pragma unroll
    for (int mt = 0; mt < VMT; ++mt) {
      const uint8_t* src = vp + ((D / 4) * w + 16 * mt + n) * (kBlockTokens * VB / 8) + g * (32 * VB / 8);
      if constexpr (VB == 2) {
        const u32x2 x = *reinterpret_cast<const u32x2*>(src);
        vw[mt][0] = x[0];
        vw[mt][1] = x[1];
      } else {
        const u32x4 x = *reinterpret_cast<const u32x4*>(src);
#pragma unroll
        for (int e = 0; e < 4; ++e) vw[mt][e] = x[e];
      }
    }
  };
  f32x4 oacc[VMT];  // o~ (rotated basis) of channels (D/4)w + 16mt + 4g + r, head n & 7
#pragma unroll
  for (int mt = 0; mt < VMT; ++mt) oacc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Columns of heads >= G are zero for the whole loop and the pages fill only those of heads < G;
  // every u slot starts at zero and a page writes only the slots of the heads its wave handles.
  // (The first page's barriers order these stores before any read.)
  for (int e = tid; e < KH * 16 * L::kKStride; e += kDecThreads)
    if (((e / L::kKStride) & 7) >= G) (&s.kcoef[0][0][0])[e] = static_cast<_Float16>(0.f);
  for (int e = tid; e < NVG * 16 * L::kVStride; e += kDecThreads)
    if (((e / L::kVStride) & 7) >= G) (&s.vcoef[0][0][0])[e] = static_cast<_Float16>(0.f);
  for (int e = tid; e < kDecWaves * NVG * kMaxGroup; e += kDecThreads) (&s.upart[0][0][0])[e] = 0.f;
  if (tid < kMaxGroup) s.alpha[tid] = 1.f;

  int cur = next_valid(p0);
  if (cur < p1) {
    load_meta(cur);
    load_k(cur);
    load_v(cur);
  }
  while (cur < p1) {
    const int nxt = next_valid(cur + 1);
    const int pf = nxt < p1 ? nxt : cur;  // page whose data is fetched during this one
    // (1) largest scale factors, then the operands and constants of the page
    {
      float ek = 0.f, ev = 0.f;
      if (tid < D) {
        float mx = 0.f;
#pragma unroll
        for (int kh = 0; kh < KH; ++kh) mx = fmaxf(mx, m_ks[kh]);
        ek = ex2(m_kg) * mx;
      }
      if (tid < kBlockTokens) {
        float mx = 0.f;
#pragma unroll
        for (int vg = 0; vg < NVG; ++vg) mx = fmaxf(mx, m_vs[vg]);
        ev = ex2(m_vr) * mx;
      }
      ek = wave_maxp(ek);
      ev = wave_maxp(ev);
      if (lane == 0) {
        s.red[w][0] = ek;
        s.red[w][1] = ev;
      }
    }
    // every wave is past the previous page's value step (which reads gsv, vcoef, upart, alpha)
    __syncthreads();
    {
      const float ek = fmaxf(fmaxf(s.red[0][0], s.red[1][0]), fmaxf(s.red[2][0], s.red[3][0]));
      const float ev = fmaxf(fmaxf(s.red[0][1], s.red[1][1]), fmaxf(s.red[2][1], s.red[3][1]));
      // |a_j sa| < 2^14 and, as p <= 1, |w_t sw| < 2^14; with no positive factor the page keeps unit scale
      const float kprod = qmax * ek;
      int ex = 0, exv = 0;
      frexpf(kprod, &ex);
      frexpf(ev, &exv);
      ex = min(max(ex, -100), 100);
      exv = min(max(exv, -100), 100);
      const float sa = kprod > 0.f ? pow2i(14 - ex) : 1.f, inv_sa = kprod > 0.f ? pow2i(ex - 14) : 1.f;
      const float sw = ev > 0.f ? pow2i(14 - exv) : 1.f, inv_sw = ev > 0.f ? pow2i(exv - 14) : 1.f;
      float bp[KH][kMaxGroup];
#pragma unroll
      for (int kh = 0; kh < KH; ++kh)
#pragma unroll
        for (int h = 0; h < kMaxGroup; ++h) bp[kh][h] = 0.f;
      if (tid < D) {
        const int j = tid, slot = key_slot<KB>(j);
        const float gk = ex2(m_kg) * sa, off = key_offset<KB>(j);
#pragma unroll
        for (int kh = 0; kh < KH; ++kh)
#pragma unroll
          for (int h = 0; h < kMaxGroup; ++h) {
            if (h < G) {
              const float qg = s.qt[h][j] * gk;
              _Float16 hi, lo;
              split_hl(qg * m_ks[kh], hi, lo);
              s.kcoef[kh][h][slot] = hi;
              s.kcoef[kh][8 + h][slot] = lo;
              bp[kh][h] = fmaf(qg, m_kz[kh], -off * (static_cast<float>(hi) + static_cast<float>(lo)));
            }
          }
        s.gsv[j] = ex2(m_vg) * inv_sw;
      }
#pragma unroll
      for (int kh = 0; kh < KH; ++kh)
#pragma unroll
        for (int h = 0; h < kMaxGroup; ++h) {
          if (h < G) {
            const float t = wave_sump(bp[kh][h]);
            if (lane == 0) s.bpart[w][kh][h] = t;
          }
        }
      if (tid < kBlockTokens) {
        s.krho[tid] = ex2(m_kr) * inv_sa * scale_log2;
        const float vr = ex2(m_vr) * sw;
#pragma unroll
        for (int vg = 0; vg < NVG; ++vg) {
          s.vsr[vg][tid] = vr * m_vs[vg];
          s.vzr[vg][tid] = vr * m_vz[vg];
        }
      }
      load_meta(pf);
    }
    __syncthreads();
    // (2) scores of tokens 32w + 16mt + 4g + r for the head of column n (hi and lo columns summed)
    {
      f32x4 d[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
      const _Float16* cb = &s.kcoef[kh_w][n][(D / 4) * g];
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const f16x8 bop = *reinterpret_cast<const f16x8*>(cb + 8 * kc);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          f16x8 aop;
          if constexpr (KB == 4) {
            aop = key_codes(kw[mt][kc], mag16, mag64);
          } else {
            aop = key_codes8(kw[mt][2 * kc], kw[mt][2 * kc + 1], mag1024);
          }
          d[mt] = mfma16x16x32(aop, bop, d[mt]);
        }
      }
      load_k(pf);
      const int h = n & 7;
      const float bsum = s.bpart[0][kh_w][h] + s.bpart[1][kh_w][h] + s.bpart[2][kh_w][h] + s.bpart[3][kh_w][h];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float x = d[mt][r] + dpp<kDppXor8>(d[mt][r]);
          const int t = 32 * w + 16 * mt + 4 * g + r;
          if (n < 8) s.score[h][t] = (x + bsum) * s.krho[t];
        }
    }
    __syncthreads();
    // (3) online softmax per head: wave w takes heads w and w + 4; lane l tokens 2l, 2l + 1
    {
      const int t0 = 2 * lane, t1 = 2 * lane + 1;
      const int v0 = value_slot(t0), v1 = value_slot(t1);
      for (int h = w; h < G; h += kDecWaves) {
        const float s0 = s.score[h][t0], s1 = s.score[h][t1];
        const float pm = wave_maxp(fmaxf(s0, s1));
        const float mold = s.mrun[h];
        const float mnew = fmaxf(mold, pm);
        const float e0 = ex2(s0 - mnew), e1 = ex2(s1 - mnew);
        const float lp = wave_sump(e0 + e1);
#pragma unroll
        for (int vg = 0; vg < NVG; ++vg) {
          _Float16 h0, l0, h1, l1;
          split_hl(e0 * s.vsr[vg][t0], h0, l0);
          split_hl(e1 * s.vsr[vg][t1], h1, l1);
          s.vcoef[vg][h][v0] = h0;
          s.vcoef[vg][8 + h][v0] = l0;
          s.vcoef[vg][h][v1] = h1;
          s.vcoef[vg][8 + h][v1] = l1;
          const float off = value_offset<VB>(t0) * (static_cast<float>(h0) + static_cast<float>(l0)) +
                            value_offset<VB>(t1) * (static_cast<float>(h1) + static_cast<float>(l1));
          const float u = wave_sump(fmaf(e0, s.vzr[vg][t0], e1 * s.vzr[vg][t1]) - off);
          if (lane == 0) s.upart[w][vg][h] = u;
        }
        if (lane == 0) {
          const float al = mold == -INFINITY ? 0.f : ex2(mold - mnew);
          s.alpha[h] = al;
          s.lrun[h] = fmaf(al, s.lrun[h], lp);
          s.mrun[h] = mnew;
        }
      }
    }
    __syncthreads();
    // (4) values: channels (D/4)w + 16mt + 4g + r for the head of column n (hi and lo columns summed)
    {
      const int h = n & 7;
      const float al = s.alpha[h];
#pragma unroll
      for (int mt = 0; mt < VMT; ++mt) {
        const int jb = (D / 4) * w + 16 * mt;
        const int vg = jb / VGC;
        const _Float16* wb = &s.vcoef[vg][n][32 * g];
        f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          f16x8 c0, c1;
          if constexpr (VB == 2) {
            value_codes(vw[mt][u], mag4, mag16, c0, c1);
          } else {
            value_codes4(vw[mt][2 * u], vw[mt][2 * u + 1], mag64, c0, c1);
          }
          d = mfma16x16x32(c0, *reinterpret_cast<const f16x8*>(wb + 16 * u), d);
          d = mfma16x16x32(c1, *reinterpret_cast<const f16x8*>(wb + 16 * u + 8), d);
        }
        const float uh = s.upart[0][vg][h] + s.upart[1][vg][h] + s.upart[2][vg][h] + s.upart[3][vg][h];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float x = d[r] + dpp<kDppXor8>(d[r]);
          oacc[mt][r] = fmaf(al, oacc[mt][r], s.gsv[jb + 4 * g + r] * (x + uh));
        }
      }
      load_v(pf);
    }
    // no barrier here: the next page's step (1) writes only s.red before its barrier
    cur = nxt;
  }
  if (bad_page && tid == 0 && flags) atomicOr(flags, kFlagBadPage);

  // ---- this split's partial: o~ (rotated basis), m, l per head ----------------------------------
  __syncthreads();  // every wave is out of the page loop (q~ is no longer read)
  if (n < 8) {
#pragma unroll
    for (int mt = 0; mt < VMT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) s.qt[n][(D / 4) * w + 16 * mt + 4 * g + r] = oacc[mt][r];
  }
  __syncthreads();
  for (int e = tid; e < G * D; e += kDecThreads) {
    const int h = e / D, j = e - h * D;
    store_coherent(pbase + (static_cast<size_t>(split) * kMaxGroup + h) * PS + j, s.qt[h][j]);
  }
  if (tid < G) {
    float* pp = pbase + (static_cast<size_t>(split) * kMaxGroup + tid) * PS;
    store_coherent(pp + D, s.mrun[tid]);
    store_coherent(pp + D + 1, s.lrun[tid]);
  }
  split_merge<D>(s.qt, s.sm, s.sl, s.last, pbase, counters + pair, nsplit, G, out_b);
}

namespace {

// Sums over the 64 lanes of v[lane & 7]: every lane gets the total of head lane & 7 (three pairwise
// stages halve the values per lane, lanes l^1, l^2 and (l + 4) mod 16, then lanes l^8, l^16, l^32).
__device__ __forceinline__ float head_sums8(const float (&v)[kMaxGroup], int lane) {
  const bool b0 = lane & 1, b1 = lane & 2, b2 = lane & 4;
  float s4[4], s2[2];
#pragma unroll
  for (int k = 0; k < 4; ++k) s4[k] = (b0 ? v[2 * k + 1] : v[2 * k]) + dpp<kDppXor1>(b0 ? v[2 * k] : v[2 * k + 1]);
#pragma unroll
  for (int m = 0; m < 2; ++m)
    s2[m] = (b1 ? s4[2 * m + 1] : s4[2 * m]) + dpp<kDppXor2>(b1 ? s4[2 * m] : s4[2 * m + 1]);
  // (lane + 4) mod 16 always has the other value of bit 2
  float t = (b2 ? s2[1] : s2[0]) + dpp<kDppRor4>(b2 ? s2[0] : s2[1]);
  t += dpp<kDppXor8>(t);
  return rows_sum(t);
}

template <int KB, int VB, int GS>
struct D64Lds {
  static constexpr int KH = kBlockTokens / GS;  // key groups per channel (token halves)
  struct Wave {
    _Float16 kcoef[KH][16][64 + 8];             // key B operand: hi (columns 0-7), lo (8-15) of a_j sa
    _Float16 vcoef[16][kBlockTokens + 8];       // value B operand: hi, lo of w_t sw
    float krho[kBlockTokens];                   // 2^rho_t / sa * scale (keys)
    float vsr[kBlockTokens], vzr[kBlockTokens];  // 2^rho_t s sw, 2^rho_t z sw (values)
    float gsv[64];                              // 2^gamma_j / sw (values)
  };
  float qt[kMaxGroup][64];                      // q~ per head; the merged output at the end
  union {
    Wave wv[kDecWaves];                         // each wave's page, during the page loop
    float wo[kDecWaves][kMaxGroup][64];         // each wave's o~ for the merge of the waves
  } u;
  float wm[kDecWaves][kMaxGroup], wl[kDecWaves][kMaxGroup];
  float qred[kDecWaves];
  float sm[64][kMaxGroup], sl[64][kMaxGroup];
  int last;
};

}  // namespace

// Decode over pages of 64-channel heads, one page per wave: grid (Hkv, batch, splits), four waves per
// workgroup, wave w taking every fourth page of the split.  A 64-channel page is small enough for one
// wave, so no page needs a workgroup barrier: per page the wave builds its fp16 hi/lo coefficient
// operands in its own LDS (lane j: channel j), scores 128 tokens on the matrix cores (eight 16-token
// tiles, two chained products each), runs the online softmax in registers (lane (n, g) holds the 32
// scores of head n & 7 for tokens 16mt + 4g + r; the four 16-lane rows finish the max and sum), writes
// its weight column of the value operand and accumulates o~ of all 64 channels (four 16-channel tiles,
// four products each).  The four waves merge through LDS at the end; the split partial, hand-off and
// last-workgroup merge are those of the head-size decode.  Each part of the next page is loaded right
// after its last use on the current one.
template <int KB, int VB, int GS>
__global__ __launch_bounds__(kDecThreads) void decode_hd64_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ k_pool, const uint8_t* __restrict__ v_pool,
    int num_pages, const int32_t* __restrict__ block_table, int max_blocks, const int32_t* __restrict__ seq_lens,
    int hq, int hkv, int blocks_per_split, int max_splits, float scale_log2, float* __restrict__ out,
    float* __restrict__ part, uint32_t* __restrict__ counters, uint32_t* __restrict__ flags) {
  constexpr int D = 64;
  using L = D64Lds<KB, VB, GS>;
  using PK = HdPage<D, false, KB, GS>;
  using PV = HdPage<D, true, VB, GS>;
  constexpr int KH = L::KH;
  constexpr int PS = D + 2;
  constexpr int KWT = KB / 2;  // key code dwords of a lane per token tile (16 channels)
  constexpr int KROW = D * KB / 8, VROW = kBlockTokens * VB / 8;
  static_assert(PV::kVGroup == D, "one value group per token at 64 channels");
  __shared__ __align__(16) L s;

  const int kvh = blockIdx.x, b = blockIdx.y, split = blockIdx.z;
  const int G = hq / hkv;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, n = lane & 15, g = lane >> 4;
  const int sl_b = seq_lens[b];
  float* out_b = out + (static_cast<size_t>(b) * hq + static_cast<size_t>(kvh) * G) * D;
  const bool bad = sl_b < 0 || sl_b > max_blocks * kBlockTokens || (sl_b & (kBlockTokens - 1)) != 0;
  const int nblk = bad ? 0 : sl_b / kBlockTokens;
  if (nblk == 0) {
    if (split == 0) {
      if (bad && tid == 0 && flags) atomicOr(flags, kFlagBadSeqLen);
      for (int e = tid; e < G * D; e += kDecThreads) out_b[e] = 0.f;
    }
    return;
  }
  const int nsplit = (nblk + blocks_per_split - 1) / blocks_per_split;
  if (split >= nsplit) return;
  const size_t pair = static_cast<size_t>(b) * hkv + kvh;
  float* pbase = part + pair * max_splits * kMaxGroup * PS;

  // ---- q~ = H q / sqrt(D) for the G heads (rows past G are zero), and max |q~| -------------------
  const uint16_t* qb = q + (static_cast<size_t>(b) * hq + static_cast<size_t>(kvh) * G) * D;
  for (int e = tid; e < kMaxGroup * D; e += kDecThreads) {
    const int hh = e / D, j = e - hh * D;
    s.qt[hh][j] = hh < G ? half_bits_to_float(qb[hh * D + j]) : 0.f;
  }
  __syncthreads();
  lds_fwht_rows<D>(s.qt, kMaxGroup);
  {
    float qm = 0.f;
    for (int e = tid; e < kMaxGroup * D; e += kDecThreads) {
      const float v = s.qt[e / D][e % D] * HdGeom<D>::kInvSqrtD;
      s.qt[e / D][e % D] = v;
      qm = fmaxf(qm, fabsf(v));
    }
    qm = wave_maxp(qm);
    if (lane == 0) s.qred[w] = qm;
  }
  __syncthreads();
  const float qmax = fmaxf(fmaxf(s.qred[0], s.qred[1]), fmaxf(s.qred[2], s.qred[3]));
  float qj[kMaxGroup];  // q~ of channel `lane`, every head
#pragma unroll
  for (int hh = 0; hh < kMaxGroup; ++hh) qj[hh] = s.qt[hh][lane];

  uint32_t mag4 = 0x44004400u, mag16 = 0x4C004C00u, mag64 = 0x54005400u, mag1024 = 0x64006400u;
  asm volatile("" : "+v"(mag4), "+v"(mag16), "+v"(mag64), "+v"(mag1024));

  const int p0 = split * blocks_per_split;
  const int cnt = min(nblk, p0 + blocks_per_split) - p0;
  const int32_t* bt = block_table + static_cast<size_t>(b) * max_blocks + p0;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  auto& W = s.u.wv[w];

  // one page's data in registers
  uint32_t kw[8][KWT];  // key codes: token 16mt + n, channels 16g .. 16g+15
  uint32_t vw[4][VB];   // value codes: channel 16mt + n, tokens 32g .. 32g+31
  float m_kg = 0.f, m_ks[KH], m_kz[KH], m_vg = 0.f;  // channel `lane`
  float2 m_kr, m_vr;                                 // tokens 2 lane, 2 lane + 1
  uint32_t m_vs = 0u, m_vz = 0u;                     // value scale / zero (fp16 pair) of those tokens
  // The wave visits only its valid pages: a scalar search over the page ids passes over invalid ones
  // and flags them, so the page loop has no per-page branch and the next page's loads land in the
  // very registers of the current one.  Loads take the wave-uniform page base from scalar registers
  // and an unsigned lane offset.
  bool bad_page = false;
  auto next_valid = [&](int i) {  // first index >= i in steps of kDecWaves with a valid page id, or >= cnt
    for (; i < cnt; i += kDecWaves) {
      const int pg = bt[i];
      if (pg >= 0 && pg < num_pages) break;
      bad_page = true;
    }
    return i;
  };
  auto base_k = [&](int i) { return k_pool + (static_cast<size_t>(bt[i]) * hkv + kvh) * PK::kBytes; };
  auto base_v = [&](int i) { return v_pool + (static_cast<size_t>(bt[i]) * hkv + kvh) * PV::kBytes; };
  auto load_meta = [&](int i) {
    const uint8_t* kp = base_k(i);
    const uint8_t* vp = base_v(i);
    const uint32_t l2 = 2u * static_cast<uint32_t>(lane), l4 = 4u * static_cast<uint32_t>(lane);
    const uint32_t l8 = 8u * static_cast<uint32_t>(lane);
    m_kg = *reinterpret_cast<const float*>(kp + l4 + PK::kGamma);
    m_vg = *reinterpret_cast<const float*>(vp + l4 + PV::kGamma);
#pragma unroll
    for (int kh = 0; kh < KH; ++kh) {
      m_ks[kh] = half_bits_to_float(*reinterpret_cast<const uint16_t*>(kp + l2 + (PK::kScale + 2 * D * kh)));
      m_kz[kh] = half_bits_to_float(*reinterpret_cast<const uint16_t*>(kp + l2 + (PK::kZero + 2 * D * kh)));
    }
    m_kr = *reinterpret_cast<const float2*>(kp + l8 + PK::kRho);
    m_vr = *reinterpret_cast<const float2*>(vp + l8 + PV::kRho);
    m_vs = *reinterpret_cast<const uint32_t*>(vp + l4 + PV::kScale);
    m_vz = *reinterpret_cast<const uint32_t*>(vp + l4 + PV::kZero);
  };
  auto load_k = [&](int i) {
    const uint8_t* kp = base_k(i);
    const uint32_t off = static_cast<uint32_t>(n * KROW + g * (KROW / 4));
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      const uint8_t* src = kp + off + 16 * mt * KROW;
      if constexpr (KWT == 2) {
        const u32x2 x = *reinterpret_cast<const u32x2*>(src);
        kw[mt][0] = x[0];
        kw[mt][1] = x[1];
      } else {
        const u32x4 x = *reinterpret_cast<const u32x4*>(src);
#pragma unroll
        for (int e = 0; e < 4; ++e) kw[mt][e] = x[e];
      }
    }
  };
  auto load_v = [&](int i) {
    const uint8_t* vp = base_v(i);
    const uint32_t off = static_cast<uint32_t>(n * VROW + g * (VROW / 4));
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const uint8_t* src = vp + off + 16 * mt * VROW;
      if constexpr (VB == 2) {
        const u32x2 x = *reinterpret_cast<const u32x2*>(src);
        vw[mt][0] = x[0];
        vw[mt][1] = x[1];
      } else {
        const u32x4 x = *reinterpret_cast<const u32x4*>(src);
#pragma unroll
        for (int e = 0; e < 4; ++e) vw[mt][e] = x[e];
      }
    }
  };

  float m_run = -INFINITY, l_run = 0.f;  // online softmax of head h (lane's column)
  f32x4 oacc[4];                        // o~ of channels 16mt + 4g + r, head h
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) oacc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int i0 = next_valid(wu);
  if (i0 < cnt) {
    load_meta(i0);
    load_k(i0);
    load_v(i0);
  }
  // key operand columns of heads >= G stay zero for the whole loop; the pages fill the others
  for (int e = lane; e < KH * 16 * (64 + 8); e += 64)
    if (((e / (64 + 8)) & 7) >= G) (&W.kcoef[0][0][0])[e] = static_cast<_Float16>(0.f);
  for (int i = i0; i < cnt;) {
    const int nx = next_valid(i + kDecWaves);  // the wave's next valid page
    const bool more = nx < cnt;                // wave-uniform, like everything decided per page
    // (1) page scales, coefficient operands, per-token and per-channel factors
    float b_h[KH];  // b sa (offsets removed) of head h, per token half
    {
      float kmx = 0.f;
#pragma unroll
      for (int kh = 0; kh < KH; ++kh) kmx = fmaxf(kmx, m_ks[kh]);
      const float ek = wave_maxp(ex2(m_kg) * kmx);
      const float vr0 = ex2(m_vr.x), vr1 = ex2(m_vr.y);
      const float vs0 = half_bits_to_float(m_vs & 0xFFFFu), vs1 = half_bits_to_float(m_vs >> 16);
      const float ev = wave_maxp(fmaxf(vr0 * vs0, vr1 * vs1));
      const float kprod = qmax * ek;
      int ex = 0, exv = 0;
      frexpf(kprod, &ex);
      frexpf(ev, &exv);
      ex = min(max(ex, -100), 100);
      exv = min(max(exv, -100), 100);
      const float sa = kprod > 0.f ? pow2i(14 - ex) : 1.f, inv_sa = kprod > 0.f ? pow2i(ex - 14) : 1.f;
      const float sw = ev > 0.f ? pow2i(14 - exv) : 1.f, inv_sw = ev > 0.f ? pow2i(exv - 14) : 1.f;
      const int slot = key_slot<KB>(lane);
      const float gk = ex2(m_kg) * sa, off = key_offset<KB>(lane);
#pragma unroll
      for (int kh = 0; kh < KH; ++kh) {
        float bp[kMaxGroup];
#pragma unroll
        for (int hh = 0; hh < kMaxGroup; ++hh) {
          bp[hh] = 0.f;
          if (hh < G) {
            const float qg = qj[hh] * gk;
            _Float16 hi, lo;
            split_hl(qg * m_ks[kh], hi, lo);
            W.kcoef[kh][hh][slot] = hi;
            W.kcoef[kh][8 + hh][slot] = lo;
            bp[hh] = fmaf(qg, m_kz[kh], -off * (static_cast<float>(hi) + static_cast<float>(lo)));
          }
        }
        b_h[kh] = head_sums8(bp, lane);
      }
      const int t0 = 2 * lane;
      W.krho[t0] = ex2(m_kr.x) * inv_sa * scale_log2;
      W.krho[t0 + 1] = ex2(m_kr.y) * inv_sa * scale_log2;
      W.vsr[t0] = vr0 * sw * vs0;
      W.vsr[t0 + 1] = vr1 * sw * vs1;
      W.vzr[t0] = vr0 * sw * half_bits_to_float(m_vz & 0xFFFFu);
      W.vzr[t0 + 1] = vr1 * sw * half_bits_to_float(m_vz >> 16);
      W.gsv[lane] = ex2(m_vg) * inv_sw;
      if (more) load_meta(nx);
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    // (2) scores of tokens 16mt + 4g + r for head h (hi and lo columns summed; b enters the hi
    // column's accumulator)
    float sc[8][4];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      const int kh = (16 * mt) / GS;
      const _Float16* cb = &W.kcoef[kh][n][16 * g];
      const float bi = n < 8 ? b_h[kh] : 0.f;
      f32x4 d = {bi, bi, bi, bi};
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        f16x8 aop;
        if constexpr (KB == 4) {
          aop = key_codes(kw[mt][kc], mag16, mag64);
        } else {
          aop = key_codes8(kw[mt][2 * kc], kw[mt][2 * kc + 1], mag1024);
        }
        d = mfma16x16x32(aop, *reinterpret_cast<const f16x8*>(cb + 8 * kc), d);
      }
      const float4 kr = *reinterpret_cast<const float4*>(&W.krho[16 * mt + 4 * g]);
      const float krv[4] = {kr.x, kr.y, kr.z, kr.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) sc[mt][r] = (d[r] + dpp<kDppXor8>(d[r])) * krv[r];
    }
    if (more) load_k(nx);
    // (3) online softmax of head h over the page's 128 tokens, and the value operands
    float u_h;
    {
      float pm = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) pm = fmaxf(pm, sc[mt][r]);
      pm = rows_max(pm);
      const float mnew = fmaxf(m_run, pm);
      const float al = m_run == -INFINITY ? 0.f : ex2(m_run - mnew);
      // the value offsets of exactly the fp16 weights used: sum over tokens of off_t (hi + lo), one
      // v_dot2 of the packed pair per token (t has the parity of r)
      typedef _Float16 h2 __attribute__((ext_vector_type(2)));
      const h2 off_even = {static_cast<_Float16>(value_offset<VB>(0)), static_cast<_Float16>(value_offset<VB>(0))};
      const h2 off_odd = {static_cast<_Float16>(value_offset<VB>(1)), static_cast<_Float16>(value_offset<VB>(1))};
      float lp = 0.f, up = 0.f, uo = 0.f;
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        const float4 vs4 = *reinterpret_cast<const float4*>(&W.vsr[16 * mt + 4 * g]);
        const float4 vz4 = *reinterpret_cast<const float4*>(&W.vzr[16 * mt + 4 * g]);
        const float vsv[4] = {vs4.x, vs4.y, vs4.z, vs4.w}, vzv[4] = {vz4.x, vz4.y, vz4.z, vz4.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 16 * mt + 4 * g + r;
          const float e = ex2(sc[mt][r] - mnew);
          lp += e;
          _Float16 hi, lo;
          split_hl(e * vsv[r], hi, lo);
          W.vcoef[n][value_slot(t)] = n < 8 ? hi : lo;  // this lane's column: hi for n < 8, lo for n >= 8
          up = fmaf(e, vzv[r], up);
          const h2 hl = {hi, lo};
          uo = __builtin_amdgcn_fdot2(hl, (r & 1) ? off_odd : off_even, uo, false);
        }
      }
      lp = rows_sum(lp);
      u_h = rows_sum(up - uo);
      l_run = fmaf(al, l_run, lp);
      m_run = mnew;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) oacc[mt][r] *= al;
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    // (4) values: o~_j += 2^gamma_j (sum_t w_t c_tj + u), channels 16mt + 4g + r (u enters the hi
    // column's accumulator)
    {
      const float ui = n < 8 ? u_h : 0.f;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const _Float16* wb = &W.vcoef[n][32 * g];
        f32x4 d = {ui, ui, ui, ui};
#pragma unroll
        for (int uu = 0; uu < 2; ++uu) {
          f16x8 c0, c1;
          if constexpr (VB == 2) {
            value_codes(vw[mt][uu], mag4, mag16, c0, c1);
          } else {
            value_codes4(vw[mt][2 * uu], vw[mt][2 * uu + 1], mag64, c0, c1);
          }
          d = mfma16x16x32(c0, *reinterpret_cast<const f16x8*>(wb + 16 * uu), d);
          d = mfma16x16x32(c1, *reinterpret_cast<const f16x8*>(wb + 16 * uu + 8), d);
        }
        const float4 gs4 = *reinterpret_cast<const float4*>(&W.gsv[16 * mt + 4 * g]);
        const float gsv[4] = {gs4.x, gs4.y, gs4.z, gs4.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) oacc[mt][r] = fmaf(gsv[r], d[r] + dpp<kDppXor8>(d[r]), oacc[mt][r]);
      }
    }
    if (more) load_v(nx);
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    i = nx;
  }
  if (bad_page && lane == 0 && flags) atomicOr(flags, kFlagBadPage);

  // ---- merge the four waves, then this split's partial: o~ (rotated basis), m, l per head ----------
  __syncthreads();  // every wave is out of the page loop: its page buffers may be reused
  if (n < 8) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) s.u.wo[w][n][16 * mt + 4 * g + r] = oacc[mt][r];
    if (g == 0) {
      s.wm[w][n] = m_run;
      s.wl[w][n] = l_run;
    }
  }
  __syncthreads();
  for (int e = tid; e < G * D; e += kDecThreads) {
    const int hh = e / D, j = e - hh * D;
    float mx = -INFINITY;
#pragma unroll
    for (int x = 0; x < kDecWaves; ++x) mx = fmaxf(mx, s.wm[x][hh]);
    float o = 0.f, lsum = 0.f;
#pragma unroll
    for (int x = 0; x < kDecWaves; ++x) {
      const float wgt = s.wm[x][hh] == -INFINITY ? 0.f : ex2(s.wm[x][hh] - mx);
      o = fmaf(wgt, s.u.wo[x][hh][j], o);
      lsum = fmaf(wgt, s.wl[x][hh], lsum);
    }
    float* pp = pbase + (static_cast<size_t>(split) * kMaxGroup + hh) * PS;
    store_coherent(pp + j, o);
    if (j == 0) {
      store_coherent(pp + D, mx);
      store_coherent(pp + D + 1, lsum);
    }
  }
  split_merge<D>(s.qt, s.sm, s.sl, s.last, pbase, counters + pair, nsplit, G, out_b);
}

hipError_t launch_quantize_hd(const void* k, const void* v, int n_blocks, int hkv, int head_dim,
                              const int32_t* dst_pages, void* k_pool, void* v_pool, int num_pages, int kbits,
                              int vbits, int group, uint32_t* flags, hipStream_t stream) {
  const unsigned tiles = 2u * static_cast<unsigned>(n_blocks) * static_cast<unsigned>(hkv);
  if (tiles == 0) return hipSuccess;
#define KVARN_QHD(D, KB, VB, GS)                                                                                 \
  if (head_dim == D && kbits == KB && vbits == VB && group == GS) {                                                \
    hipLaunchKernelGGL((quantize_hd_kernel<D, KB, VB, GS>), dim3(tiles), dim3(HdGeom<D>::kThreads), 0, stream,      \
                       static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), hkv, dst_pages,           \
                       static_cast<uint8_t*>(k_pool), static_cast<uint8_t*>(v_pool), num_pages, flags);            \
    return hipGetLastError();                                                                                      \
  }
#define KVARN_QHD_D(D)                                                                                             \
  KVARN_QHD(D, 4, 2, 128) KVARN_QHD(D, 4, 4, 128) KVARN_QHD(D, 8, 2, 128) KVARN_QHD(D, 8, 4, 128)                 \
  KVARN_QHD(D, 4, 2, 64) KVARN_QHD(D, 4, 4, 64) KVARN_QHD(D, 8, 2, 64) KVARN_QHD(D, 8, 4, 64)
  KVARN_QHD_D(64)
  KVARN_QHD_D(256)
#undef KVARN_QHD_D
#undef KVARN_QHD
  return hipErrorInvalidValue;
}

hipError_t launch_dequantize_hd(const void* k_pool, const void* v_pool, int num_pages, const int32_t* pages,
                                int n_blocks, int hkv, int head_dim, int kbits, int vbits, int group, float* k_out,
                                float* v_out, uint32_t* flags, hipStream_t stream) {
  const unsigned tiles = 2u * static_cast<unsigned>(n_blocks) * static_cast<unsigned>(hkv);
  if (head_dim == 64)
    hipLaunchKernelGGL(dequantize_hd_kernel<64>, dim3(tiles), dim3(256), 0, stream,
                       static_cast<const uint8_t*>(k_pool), static_cast<const uint8_t*>(v_pool), num_pages, pages,
                       hkv, kbits, vbits, group, k_out, v_out, flags);
  else if (head_dim == 256)
    hipLaunchKernelGGL(dequantize_hd_kernel<256>, dim3(2 * tiles), dim3(256), 0, stream,
                       static_cast<const uint8_t*>(k_pool), static_cast<const uint8_t*>(v_pool), num_pages, pages,
                       hkv, kbits, vbits, group, k_out, v_out, flags);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_decode_hd(const void* q, const void* k_pool, const void* v_pool, int num_pages,
                            const int32_t* block_table, int max_blocks, const int32_t* seq_lens, int batch, int hq,
                            int hkv, int head_dim, int kbits, int vbits, int group, int blocks_per_split,
                            int max_splits, float scale_log2, float* out, float* part, uint32_t* counters,
                            uint32_t* flags, hipStream_t stream) {
#define KVARN_DHD(D, KB, VB, GS)                                                                                   \
  if (head_dim == D && kbits == KB && vbits == VB && group == GS) {                                                \
    auto kern = D == 64 ? decode_hd64_kernel<KB, VB, GS> : decode_hd_kernel<D, KB, VB, GS>;                         \
    hipLaunchKernelGGL(kern, dim3(hkv, batch, max_splits), dim3(kDecThreads), 0,                                     \
                       stream, static_cast<const uint16_t*>(q), static_cast<const uint8_t*>(k_pool),              \
                       static_cast<const uint8_t*>(v_pool), num_pages, block_table, max_blocks, seq_lens, hq, hkv,  \
                       blocks_per_split, max_splits, scale_log2, out, part, counters, flags);                      \
    return hipGetLastError();                                                                                      \
  }
#define KVARN_DHD_D(D)                                                                                             \
  KVARN_DHD(D, 4, 2, 128) KVARN_DHD(D, 4, 4, 128) KVARN_DHD(D, 8, 2, 128) KVARN_DHD(D, 8, 4, 128)                 \
  KVARN_DHD(D, 4, 2, 64) KVARN_DHD(D, 4, 4, 64) KVARN_DHD(D, 8, 2, 64) KVARN_DHD(D, 8, 4, 64)
  KVARN_DHD_D(64)
  KVARN_DHD_D(256)
#undef KVARN_DHD_D
#undef KVARN_DHD
  return hipErrorInvalidValue;
}

}  // namespace kvarn
