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
// fp32 cancellation can lose digits.  The page is assembled in LDS (codes, scale/zero, rho, gamma)
// and written with 16-byte stores.
//
// Decode.  One workgroup of four waves per (sequence, KV head, split), the same split plan, partial
// layout and fence-free hand-off as the 128-channel decode.  With q~ = H q (orthonormal H) the page
// contractions run in the rotated basis on the vector ALU:
//     score_t = 2^rho_t * sum_j q~_j 2^gamma_j (s c_tj + z)       (key group of channel j, half of t)
//     o~_j   += 2^gamma_j * sum_t p_t 2^rho_t (s c_tj + z)        (value group of token t, group of j)
// with online softmax; the last workgroup of a (sequence, KV head) merges the splits and applies H.
#include "kvarn_common.h"

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
__device__ __forceinline__ float lg2(float x) { return __builtin_amdgcn_logf(x); }

// Rounded product the compiler may not fuse into a later add (a constant group must get range 0).
__device__ __forceinline__ float mul_rn(float a, float b) {
  float p = a * b;
  asm("" : "+v"(p));
  return p;
}

// Sum / min / max over lanes l, l^16, l^32, l^48 (permlane swaps return the pair in lane order, so
// every lane combines the same values in the same order and gets identical bits).
__device__ __forceinline__ float rows_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float rows_min(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fminf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fminf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float rows_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float wave_sump(float x) { return rows_sum(row16_sum(x)); }
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
  f16x8 hb[2], hbn[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bool neg = __popc((8 * g + i) & (2 * n + hh)) & 1;
      hb[hh][i] = neg ? static_cast<_Float16>(-1.0f) : static_cast<_Float16>(1.0f);
      hbn[hh][i] = neg ? static_cast<_Float16>(1.0f) : static_cast<_Float16>(-1.0f);
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

  // ---- normalisation: rf = 2^-rho / sqrt(D) per token, cf = 2^-gamma per channel -------------
  float rho[NT], rf[NT], cf[NC];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    rho[i] = 0.f;
    rf[i] = Gm::kInvSqrtD;
  }
#pragma unroll
  for (int c = 0; c < NC; ++c) cf[c] = 1.f;
  float gam_red = 0.f, cf_red = 1.f;  // gamma of channel tid, kept by reducer thread tid < D
  for (int it = 0; it < kNormIters; ++it) {
    // row pass: per token, over its D channels (16 lanes of a DPP row)
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
    // column pass: per channel, over the 128 tokens (four rows of the wave, then the waves)
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      float s1 = 0.f;
#pragma unroll
      for (int i = 0; i < NT; ++i) s1 = fmaf(R[i][c], rf[i], s1);
      s1 = rows_sum(s1);
      if (g == 0) s.part_a[w][chan(c)] = s1;
    }
    __syncthreads();
    if (tid < D) {
      float t = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) t += s.part_a[ww][tid];
      s.col[tid] = t * kInvBlock;
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const float m = s.col[chan(c)];
      float s2 = 0.f;
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        const float d = fmaf(R[i][c], rf[i], -m);
        s2 = fmaf(d, d, s2);
      }
      s2 = rows_sum(s2);
      if (g == 0) s.part_a[w][chan(c)] = s2;
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
  if (n == 0) {
#pragma unroll
    for (int i = 0; i < NT; ++i) *reinterpret_cast<float*>(&s.page[Pg::kRho + 4 * tok(i)]) = rho[i];
  }
  if (tid < D) *reinterpret_cast<float*>(&s.page[Pg::kGamma + 4 * tid]) = gam_red;

  // ---- groups: min/max, fp16 scale and zero, rounding factors, codes --------------------------
  uint32_t code[NT][NC];
  if constexpr (!kIsV) {
    // key groups: channel j over the GS tokens of half h (a lane's tokens lie in one half)
    constexpr int KH = kBlockTokens / GS;
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
      for (int c = 0; c < NC; ++c) R[i][c] *= rf[i];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      float a = R[0][c], b = R[0][c];
#pragma unroll
      for (int i = 1; i < NT; ++i) {
        a = fminf(a, R[i][c]);
        b = fmaxf(b, R[i][c]);
      }
      a = rows_min(a);
      b = rows_max(b);
      if (g == 0) {
        s.part_a[w][chan(c)] = a;
        s.part_b[w][chan(c)] = b;
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
    for (int c = 0; c < NC; ++c) {
      const float qa = s.qa[kh][chan(c)], qb = s.qb[kh][chan(c)];
#pragma unroll
      for (int i = 0; i < NT; ++i) code[i][c] = rne_code<L>(fmaf(R[i][c], qa, qb));
    }
  } else {
    // value groups: token t over the channels of group vg (a chunk pair's worth or more)
    constexpr int VGC = Pg::kVGroup, NVG = D / VGC, CPG = NC / NVG;  // lane channels per group
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
      for (int c = 0; c < NC; ++c) R[i][c] *= cf[c];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
#pragma unroll
      for (int vg = 0; vg < NVG; ++vg) {
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
        const float qa = rf[i] * inv, qb = -zf * inv;
#pragma unroll
        for (int c = CPG * vg; c < CPG * (vg + 1); ++c) code[i][c] = rne_code<L>(fmaf(R[i][c], qa, qb));
      }
    }
  }

  // ---- pack into the page image ----------------------------------------------------------------
  if constexpr (!kIsV) {
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
      for (int ho = 0; ho < CH; ++ho) {
        if constexpr (BITS == 4)
          s.page[(D / 2) * tok(i) + 16 * ho + n] = static_cast<uint8_t>(code[i][2 * ho] | (code[i][2 * ho + 1] << 4));
        else
          *reinterpret_cast<uint16_t*>(&s.page[D * tok(i) + 32 * ho + 2 * n]) =
              static_cast<uint16_t>(code[i][2 * ho] | (code[i][2 * ho + 1] << 8));
      }
  } else {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int t0 = w * TW + 16 * mt + 4 * g;  // four consecutive tokens of this lane
        if constexpr (BITS == 2)
          s.page[32 * chan(c) + t0 / 4] = static_cast<uint8_t>(code[4 * mt][c] | (code[4 * mt + 1][c] << 2) |
                                                               (code[4 * mt + 2][c] << 4) | (code[4 * mt + 3][c] << 6));
        else
          *reinterpret_cast<uint16_t*>(&s.page[64 * chan(c) + t0 / 2]) = static_cast<uint16_t>(
              code[4 * mt][c] | (code[4 * mt + 1][c] << 4) | (code[4 * mt + 2][c] << 8) | (code[4 * mt + 3][c] << 12));
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
__global__ __launch_bounds__(HdGeom<D>::kThreads) void quantize_hd_kernel(
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

template <int D, int KB, int VB, int GS>
struct DhdLds {
  using PK = HdPage<D, false, KB, GS>;
  using PV = HdPage<D, true, VB, GS>;
  static constexpr int KH = kBlockTokens / GS;     // key token halves
  static constexpr int NVG = D / PV::kVGroup;      // value channel groups
  float qt[kMaxGroup][D];                          // q~ per head (and the merged output at the end)
  float acoef[KH][D][kMaxGroup];                   // q~_j 2^gamma_j s, per key half, channel, head
  float bpart[kDecWaves][KH][kMaxGroup];           // per-wave sums of q~_j 2^gamma_j z
  float score[kMaxGroup][kBlockTokens];            // scores (log2 units), then p
  float wcoef[NVG][kBlockTokens][kMaxGroup];       // p_t 2^rho_t s, per value group, token, head
  float upart[kDecWaves][NVG][kMaxGroup];          // per-wave sums of p_t 2^rho_t z
  float vs[NVG][kBlockTokens], vz[NVG][kBlockTokens];  // 2^rho_t s and 2^rho_t z of the value page
  float krho[kBlockTokens];                        // 2^rho_t of the key page
  float mstat[kMaxGroup], alpha[kMaxGroup], lpage[kMaxGroup];
  float opart[kDecThreads / D > 1 ? kDecThreads / D : 1][kMaxGroup][D];  // value-side token parts
  float sm[64][kMaxGroup], sl[64][kMaxGroup];      // split maxima and sums during the merge
  int last;
};

}  // namespace

// Decode over pages of D-channel heads: grid (Hkv, batch, splits), four waves per workgroup.
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
  constexpr int PS = D + 2;                           // partial stride: o~[D], m, l
  constexpr int VPARTS = kDecThreads / D > 1 ? kDecThreads / D : 1;  // threads per value channel
  constexpr int VTOK = kBlockTokens / VPARTS;         // tokens per value thread
  constexpr int CPT = D / 2;                          // key channels per score thread
  __shared__ __align__(16) L s;

  const int kvh = blockIdx.x, b = blockIdx.y, split = blockIdx.z;
  const int G = hq / hkv;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
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

  // ---- q~ = H q / sqrt(D) for the G heads (rows past G are zero) --------------------------------
  const uint16_t* qb = q + (static_cast<size_t>(b) * hq + static_cast<size_t>(kvh) * G) * D;
  for (int e = tid; e < kMaxGroup * D; e += kDecThreads) {
    const int h = e / D, j = e - h * D;
    s.qt[h][j] = h < G ? half_bits_to_float(qb[h * D + j]) : 0.f;
  }
  __syncthreads();
  lds_fwht_rows<D>(s.qt, kMaxGroup);
  for (int e = tid; e < kMaxGroup * D; e += kDecThreads) s.qt[e / D][e % D] *= HdGeom<D>::kInvSqrtD;
  __syncthreads();

  // value side: thread owns channel vj, tokens [vpart * VTOK, + VTOK)
  const int vj = tid % D, vpart = tid / D;
  const bool vthread = vpart < VPARTS;
  const int vgrp = vj / VGC;
  float o[kMaxGroup];
  float m_run[kMaxGroup], l_run[kMaxGroup];
#pragma unroll
  for (int h = 0; h < kMaxGroup; ++h) {
    o[h] = 0.f;
    m_run[h] = -INFINITY;
    l_run[h] = 0.f;
  }
  // score side: thread owns token st, channel half sh
  const int st = tid >> 1, sh = tid & 1;

  const int p0 = split * blocks_per_split;
  const int p1 = min(nblk, p0 + blocks_per_split);
  bool bad_page = false;
  for (int pi = p0; pi < p1; ++pi) {
    const int page = block_table[static_cast<size_t>(b) * max_blocks + pi];
    if (page < 0 || page >= num_pages) {
      bad_page = true;
      continue;
    }
    const uint8_t* kp = k_pool + (static_cast<size_t>(page) * hkv + kvh) * PK::kBytes;
    const uint8_t* vp = v_pool + (static_cast<size_t>(page) * hkv + kvh) * PV::kBytes;
    // (1) page coefficients
    {
      float bp[KH][kMaxGroup];
#pragma unroll
      for (int kh = 0; kh < KH; ++kh)
#pragma unroll
        for (int h = 0; h < kMaxGroup; ++h) bp[kh][h] = 0.f;
      for (int j = tid; j < D; j += kDecThreads) {
        const float gj = ex2(reinterpret_cast<const float*>(kp + PK::kGamma)[j]);
#pragma unroll
        for (int kh = 0; kh < KH; ++kh) {
          const float sj = half_bits_to_float(reinterpret_cast<const uint16_t*>(kp + PK::kScale)[D * kh + j]);
          const float zj = half_bits_to_float(reinterpret_cast<const uint16_t*>(kp + PK::kZero)[D * kh + j]);
#pragma unroll
          for (int h = 0; h < kMaxGroup; ++h) {
            const float qg = s.qt[h][j] * gj;
            s.acoef[kh][j][h] = qg * sj;
            bp[kh][h] = fmaf(qg, zj, bp[kh][h]);
          }
        }
      }
#pragma unroll
      for (int kh = 0; kh < KH; ++kh)
#pragma unroll
        for (int h = 0; h < kMaxGroup; ++h) {
          const float t = wave_sump(bp[kh][h]);
          if (lane == 0) s.bpart[w][kh][h] = t;
        }
      if (tid < kBlockTokens) {
        const int t = tid;
        s.krho[t] = ex2(reinterpret_cast<const float*>(kp + PK::kRho)[t]);
        const float vr = ex2(reinterpret_cast<const float*>(vp + PV::kRho)[t]);
#pragma unroll
        for (int vg = 0; vg < NVG; ++vg) {
          s.vs[vg][t] = vr * half_bits_to_float(reinterpret_cast<const uint16_t*>(vp + PV::kScale)[kBlockTokens * vg + t]);
          s.vz[vg][t] = vr * half_bits_to_float(reinterpret_cast<const uint16_t*>(vp + PV::kZero)[kBlockTokens * vg + t]);
        }
      }
    }
    __syncthreads();
    // (2) scores: thread (token st, channel half sh)
    {
      const int kh = st / GS;
      float acc[kMaxGroup];
#pragma unroll
      for (int h = 0; h < kMaxGroup; ++h) acc[h] = 0.f;
      if constexpr (KB == 4) {
        const uint32_t* row = reinterpret_cast<const uint32_t*>(kp + (D / 2) * st + (D / 4) * sh);
#pragma unroll 2
        for (int k = 0; k < CPT / 8; ++k) {
          const uint32_t x = row[k];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float c = static_cast<float>((x >> (4 * e)) & 15u);
            const int j = CPT * sh + 8 * k + e;
            const float4 a0 = *reinterpret_cast<const float4*>(&s.acoef[kh][j][0]);
            const float4 a1 = *reinterpret_cast<const float4*>(&s.acoef[kh][j][4]);
            acc[0] = fmaf(a0.x, c, acc[0]);
            acc[1] = fmaf(a0.y, c, acc[1]);
            acc[2] = fmaf(a0.z, c, acc[2]);
            acc[3] = fmaf(a0.w, c, acc[3]);
            acc[4] = fmaf(a1.x, c, acc[4]);
            acc[5] = fmaf(a1.y, c, acc[5]);
            acc[6] = fmaf(a1.z, c, acc[6]);
            acc[7] = fmaf(a1.w, c, acc[7]);
          }
        }
      } else {
        const uint32_t* row = reinterpret_cast<const uint32_t*>(kp + D * st + (D / 2) * sh);
#pragma unroll 2
        for (int k = 0; k < CPT / 4; ++k) {
          const uint32_t x = row[k];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float c = static_cast<float>((x >> (8 * e)) & 255u);
            const int j = CPT * sh + 4 * k + e;
            const float4 a0 = *reinterpret_cast<const float4*>(&s.acoef[kh][j][0]);
            const float4 a1 = *reinterpret_cast<const float4*>(&s.acoef[kh][j][4]);
            acc[0] = fmaf(a0.x, c, acc[0]);
            acc[1] = fmaf(a0.y, c, acc[1]);
            acc[2] = fmaf(a0.z, c, acc[2]);
            acc[3] = fmaf(a0.w, c, acc[3]);
            acc[4] = fmaf(a1.x, c, acc[4]);
            acc[5] = fmaf(a1.y, c, acc[5]);
            acc[6] = fmaf(a1.z, c, acc[6]);
            acc[7] = fmaf(a1.w, c, acc[7]);
          }
        }
      }
      // the two halves of the token (lanes 2k, 2k+1) add in the same order
#pragma unroll
      for (int h = 0; h < kMaxGroup; ++h) {
        const float other = dpp<kDppXor1>(acc[h]);
        acc[h] = sh ? other + acc[h] : acc[h] + other;
      }
      if (sh == 0) {
        const float rt = s.krho[st] * scale_log2;
#pragma unroll
        for (int h = 0; h < kMaxGroup; ++h) {
          const float bsum = s.bpart[0][kh][h] + s.bpart[1][kh][h] + s.bpart[2][kh][h] + s.bpart[3][kh][h];
          s.score[h][st] = (acc[h] + bsum) * rt;
        }
      }
    }
    __syncthreads();
    // (3) online softmax per head: wave w takes heads w and w + 4; lane l tokens 2l, 2l + 1
    for (int h = w; h < kMaxGroup; h += kDecWaves) {
      if (h >= G) {
        if (lane == 0) {
          s.alpha[h] = 1.f;
          s.lpage[h] = 0.f;
          s.mstat[h] = 0.f;
        }
#pragma unroll
        for (int vg = 0; vg < NVG; ++vg) {
          s.wcoef[vg][2 * lane][h] = 0.f;
          s.wcoef[vg][2 * lane + 1][h] = 0.f;
          if (lane == 0) s.upart[w][vg][h] = 0.f;
        }
        continue;
      }
      const float s0 = s.score[h][2 * lane], s1 = s.score[h][2 * lane + 1];
      const float pm = wave_maxp(fmaxf(s0, s1));
      const float mnew = fmaxf(m_run[h], pm);
      const float e0 = ex2(s0 - mnew), e1 = ex2(s1 - mnew);
      const float lp = wave_sump(e0 + e1);
#pragma unroll
      for (int vg = 0; vg < NVG; ++vg) {
        s.wcoef[vg][2 * lane][h] = e0 * s.vs[vg][2 * lane];
        s.wcoef[vg][2 * lane + 1][h] = e1 * s.vs[vg][2 * lane + 1];
        const float u = wave_sump(fmaf(e0, s.vz[vg][2 * lane], e1 * s.vz[vg][2 * lane + 1]));
        if (lane == 0) s.upart[w][vg][h] = u;
      }
      if (lane == 0) {
        s.alpha[h] = m_run[h] == -INFINITY ? 0.f : ex2(m_run[h] - mnew);
        s.lpage[h] = lp;
        s.mstat[h] = mnew;
      }
    }
    // heads h >= G and waves without heads leave upart of their (w, h) unwritten above only when
    // h >= G is handled by another wave: clear this wave's other slots
    for (int h = 0; h < kMaxGroup; ++h)
      if ((h % kDecWaves) != w && lane == 0) {
#pragma unroll
        for (int vg = 0; vg < NVG; ++vg) s.upart[w][vg][h] = 0.f;
      }
    __syncthreads();
    // every thread keeps the running statistics of every head
#pragma unroll
    for (int h = 0; h < kMaxGroup; ++h) {
      if (h < G) {
        l_run[h] = fmaf(s.alpha[h], l_run[h], s.lpage[h]);
        m_run[h] = s.mstat[h];
      }
    }
    // (4) values: o~_j <- alpha o~_j + 2^gamma_j (sum_t w_t c_tj + u); the u term from part 0 only
    if (vthread) {
      float acc[kMaxGroup];
#pragma unroll
      for (int h = 0; h < kMaxGroup; ++h) acc[h] = 0.f;
      const int t0 = vpart * VTOK;
      if constexpr (VB == 2) {
        const uint32_t* col = reinterpret_cast<const uint32_t*>(vp + 32 * vj + t0 / 4);
#pragma unroll 2
        for (int k = 0; k < VTOK / 16; ++k) {
          const uint32_t x = col[k];
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const float c = static_cast<float>((x >> (2 * e)) & 3u);
            const int t = t0 + 16 * k + e;
            const float4 a0 = *reinterpret_cast<const float4*>(&s.wcoef[vgrp][t][0]);
            const float4 a1 = *reinterpret_cast<const float4*>(&s.wcoef[vgrp][t][4]);
            acc[0] = fmaf(a0.x, c, acc[0]);
            acc[1] = fmaf(a0.y, c, acc[1]);
            acc[2] = fmaf(a0.z, c, acc[2]);
            acc[3] = fmaf(a0.w, c, acc[3]);
            acc[4] = fmaf(a1.x, c, acc[4]);
            acc[5] = fmaf(a1.y, c, acc[5]);
            acc[6] = fmaf(a1.z, c, acc[6]);
            acc[7] = fmaf(a1.w, c, acc[7]);
          }
        }
      } else {
        const uint32_t* col = reinterpret_cast<const uint32_t*>(vp + 64 * vj + t0 / 2);
#pragma unroll 2
        for (int k = 0; k < VTOK / 8; ++k) {
          const uint32_t x = col[k];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float c = static_cast<float>((x >> (4 * e)) & 15u);
            const int t = t0 + 8 * k + e;
            const float4 a0 = *reinterpret_cast<const float4*>(&s.wcoef[vgrp][t][0]);
            const float4 a1 = *reinterpret_cast<const float4*>(&s.wcoef[vgrp][t][4]);
            acc[0] = fmaf(a0.x, c, acc[0]);
            acc[1] = fmaf(a0.y, c, acc[1]);
            acc[2] = fmaf(a0.z, c, acc[2]);
            acc[3] = fmaf(a0.w, c, acc[3]);
            acc[4] = fmaf(a1.x, c, acc[4]);
            acc[5] = fmaf(a1.y, c, acc[5]);
            acc[6] = fmaf(a1.z, c, acc[6]);
            acc[7] = fmaf(a1.w, c, acc[7]);
          }
        }
      }
      const float gj = ex2(reinterpret_cast<const float*>(vp + PV::kGamma)[vj]);
#pragma unroll
      for (int h = 0; h < kMaxGroup; ++h) {
        float u = 0.f;
        if (vpart == 0) u = s.upart[0][vgrp][h] + s.upart[1][vgrp][h] + s.upart[2][vgrp][h] + s.upart[3][vgrp][h];
        o[h] = fmaf(s.alpha[h], o[h], gj * (acc[h] + u));
      }
    }
    __syncthreads();  // the next page rewrites the coefficient arrays
  }
  if (bad_page && tid == 0 && flags) atomicOr(flags, kFlagBadPage);

  // ---- this split's partial: o~ (rotated basis), m, l per head ----------------------------------
  if (vthread) {
#pragma unroll
    for (int h = 0; h < kMaxGroup; ++h) s.opart[vpart][h][vj] = o[h];
  }
  __syncthreads();
  for (int e = tid; e < G * D; e += kDecThreads) {
    const int h = e / D, j = e - h * D;
    float t = 0.f;
#pragma unroll
    for (int pp = 0; pp < VPARTS; ++pp) t += s.opart[pp][h][j];
    store_coherent(pbase + (static_cast<size_t>(split) * kMaxGroup + h) * PS + j, t);
  }
  if (tid < G) {
    float* pp = pbase + (static_cast<size_t>(split) * kMaxGroup + tid) * PS;
    float mr = 0.f, lr = 0.f;
#pragma unroll
    for (int h = 0; h < kMaxGroup; ++h)
      if (h == tid) {
        mr = m_run[h];
        lr = l_run[h];
      }
    store_coherent(pp + D, mr);
    store_coherent(pp + D + 1, lr);
  }
  // Hand-off without fences, as in the 128-channel decode: partials go through agent-scope (sc1)
  // atomic accesses, vmcnt(0) covers the stores before the workgroup counts in with an agent-scope
  // add, and every access to partials and counters is one of these.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(counters + pair, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s.last = prev == static_cast<uint32_t>(nsplit - 1);
  }
  __syncthreads();
  if (!s.last) return;
  if (tid == 0) __hip_atomic_store(counters + pair, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // ---- merge the splits (log-sum-exp), then o = H o~ / sqrt(D) ----------------------------------
  for (int e = tid; e < nsplit * kMaxGroup; e += kDecThreads) {
    const int sp = e / kMaxGroup, h = e - sp * kMaxGroup;
    const float* pp = pbase + (static_cast<size_t>(sp) * kMaxGroup + h) * PS;
    s.sm[sp][h] = h < G ? load_coherent(pp + D) : -INFINITY;
    s.sl[sp][h] = h < G ? load_coherent(pp + D + 1) : 0.f;
  }
  __syncthreads();
  for (int e = tid; e < kMaxGroup * D; e += kDecThreads) {
    const int h = e / D, j = e - h * D;
    float val = 0.f;
    if (h < G) {
      float mx = -INFINITY;
      for (int sp = 0; sp < nsplit; ++sp) mx = fmaxf(mx, s.sm[sp][h]);
      float num = 0.f, den = 0.f;
      for (int sp = 0; sp < nsplit; ++sp) {
        const float ms = s.sm[sp][h];
        const float wgt = ms == -INFINITY ? 0.f : ex2(ms - mx);
        den = fmaf(wgt, s.sl[sp][h], den);
        num = fmaf(wgt, load_coherent(pbase + (static_cast<size_t>(sp) * kMaxGroup + h) * PS + j), num);
      }
      val = den > 0.f ? num / den : 0.f;
    }
    s.qt[h][j] = val;
  }
  __syncthreads();
  lds_fwht_rows<D>(s.qt, kMaxGroup);
  for (int e = tid; e < G * D; e += kDecThreads) out_b[e] = s.qt[e / D][e % D] * HdGeom<D>::kInvSqrtD;
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
    hipLaunchKernelGGL((decode_hd_kernel<D, KB, VB, GS>), dim3(hkv, batch, max_splits), dim3(kDecThreads), 0,       \
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
