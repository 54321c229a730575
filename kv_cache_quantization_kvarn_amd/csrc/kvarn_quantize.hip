// KVarN block quantisation kernel for gfx950.
//
// One workgroup (4 waves) quantises one tile: a 128-token x 128-channel fp16
// block of one KV head of K or V (KVarN blog post, section "KVarN Nasıl
// Çalışır?"): Hadamard rotation along channels, four row/column passes of
// log2-variance normalisation, per-group min/max, round to nearest, packing.
//
// Data distribution.  Wave w owns tokens [32w, 32w+32).  The rotation runs on
// the matrix cores: the 128-point Hadamard factors as H4 (x) H32 (channel bits
// 5-6 and 0-4), so each wave multiplies its fp16 tokens by the exact +-1 H32
// block (v_mfma_f32_16x16x32_f16, fp32 accumulation; the products are exact)
// and finishes H4 with two in-register butterfly stages.  The MFMA result
// layout then fixes what each lane holds: lane (n = lane%16, g = lane/16) keeps
// 8 tokens x 8 channels,
//     token   T(i) = 32w + 16*(i/4) + 4g + i%4          i = 0..7
//     channel C(c) = 32*(c/2) + 16*(c%2) + n            c = 0..7
//
// Normalisation.  A pass needs, per row (or column), the mean and the mean
// square of Y = R 2^-rho 2^-gamma.  Each lane forms partial sums over its 8
// channels (or tokens) with one FMA per element for each moment (R and R^2
// are kept in registers), writes them to LDS, and a pair of threads per row
// (column) adds the 16 partials, takes the variance, and updates that row's
// (column's) normaliser, which it keeps in a register across iterations.
// Where the variance is small against the mean square (mean^2 > var, so the
// one-sweep formula could lose digits) the pass is redone with centred sums.
// Every sum has a fixed order, so all threads see identical values.
#include "kvarn_common.h"

namespace kvarn {

namespace {

__device__ __forceinline__ int tok_of(int w, int g, int i) { return 32 * w + 16 * (i >> 2) + 4 * g + (i & 3); }
__device__ __forceinline__ int chan_of(int n, int c) { return 32 * (c >> 1) + 16 * (c & 1) + n; }
// position of channel ch in the per-lane-contiguous order used for per-channel LDS arrays
__device__ __forceinline__ int chan_slot(int ch) { return 8 * (ch & 15) + 2 * (ch >> 5) + ((ch >> 4) & 1); }

constexpr int kPartStride = 36;  // floats per row of the partial-sum array (16 slots x 2 + pad)

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float lg2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ float dpp_xor1(float x) { return dpp<kDppXor1>(x); }

// Sum of the 8 (s1, s2) slot pairs of one row half, then with the partner thread (lane ^ 1).
__device__ __forceinline__ float2 reduce_pairs(const float* row, int hf) {
  const float4* p = reinterpret_cast<const float4*>(row + 16 * hf);
  float a = 0.f, b = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float4 v = p[k];
    a += v.x;
    b += v.y;
    a += v.z;
    b += v.w;
  }
  // both threads of the pair add (first half + second half) in the same order
  const float a2 = dpp_xor1(a), b2 = dpp_xor1(b);
  return hf ? make_float2(a2 + a, b2 + b) : make_float2(a + a2, b + b2);
}

}  // namespace

__global__ __launch_bounds__(256, 2) void quantize_kernel(const uint16_t* __restrict__ kin,
                                                         const uint16_t* __restrict__ vin, int hkv,
                                                         const int32_t* __restrict__ dst_pages,
                                                         uint8_t* __restrict__ k_pool, uint8_t* __restrict__ v_pool,
                                                         int num_pages, uint32_t* __restrict__ flags) {
  __shared__ __align__(16) float part[kBlockTokens][kPartStride];  // per row / column: 16 partial pairs
  __shared__ __align__(16) float rfl[kBlockTokens];                // 2^-rho, token order
  __shared__ __align__(16) float cfl[kHeadDim];                    // 2^-gamma, chan_slot order
  __shared__ __align__(16) float mul_a[kHeadDim], mul_b[kHeadDim]; // 1/s and -z/s of each group
  __shared__ __align__(16) float mul_c[kHeadDim];                  // means for centred fallback
  __shared__ __align__(16) uint8_t codes[kBlockTokens * kHeadDim]; // staged codes, one byte each

  const int tile = blockIdx.x;
  const bool is_v = tile & 1;
  const int bh = tile >> 1;
  const int blk = bh / hkv;
  const int head = bh - blk * hkv;
  const int page = dst_pages[blk];
  if (page < 0 || page >= num_pages) {
    if (threadIdx.x == 0 && flags) atomicOr(flags, kFlagBadPage);
    return;
  }
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, n = lane & 15, g = lane >> 4;
  const size_t tstride = static_cast<size_t>(hkv) * kHeadDim;
  const uint16_t* src = (is_v ? vin : kin) + (static_cast<size_t>(blk) * kBlockTokens * hkv + head) * kHeadDim;

  // ---- 1. rotation: R = X H / sqrt(128) --------------------------------------
  float R[8][8];
  {
    f16x8 xa[2][4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int gi = 0; gi < 4; ++gi)
        xa[mt][gi] = *reinterpret_cast<const f16x8*>(src + static_cast<size_t>(32 * w + 16 * mt + n) * tstride +
                                                      32 * gi + 8 * g);
    f16x8 hb[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int i = 0; i < 8; ++i)
        hb[hh][i] = (__popc((8 * g + i) & (16 * hh + n)) & 1) ? static_cast<_Float16>(-1.0f)
                                                              : static_cast<_Float16>(1.0f);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        f32x4 d0 = mfma16x16x32(xa[mt][0], hb[hh], z);
        f32x4 d1 = mfma16x16x32(xa[mt][1], hb[hh], z);
        f32x4 d2 = mfma16x16x32(xa[mt][2], hb[hh], z);
        f32x4 d3 = mfma16x16x32(xa[mt][3], hb[hh], z);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float a = d0[r] + d1[r], b = d0[r] - d1[r], c = d2[r] + d3[r], e = d2[r] - d3[r];
          R[4 * mt + r][0 + hh] = (a + c) * kInvSqrt128;
          R[4 * mt + r][2 + hh] = (b + e) * kInvSqrt128;
          R[4 * mt + r][4 + hh] = (a - c) * kInvSqrt128;
          R[4 * mt + r][6 + hh] = (b - e) * kInvSqrt128;
        }
      }
    }
  }
  float P[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int c = 0; c < 8; ++c) P[i][c] = R[i][c] * R[i][c];

  // ---- 2. log2-variance normalisation, rows then columns, kNormIters times --
  // Reducer role of this thread: row t_red (row passes) / channel c_red (column passes).
  const int t_red = tid >> 1, hf = tid & 1;
  float rho_t = 0.f, rf_t = 1.f;   // normaliser of row t_red
  float gam_c = 0.f, cf_c = 1.f;   // normaliser of column c_red (= t_red)
  float rf[8], cf[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    rf[k] = 1.f;
    cf[k] = 1.f;
  }
  constexpr float inv128 = 1.0f / 128.0f;

  for (int it = 0; it < kNormIters; ++it) {
    // ---------------- row pass: moments over channels of R * cf -------------
    {
      float c2[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) c2[c] = cf[c] * cf[c];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float s1 = 0.f, s2 = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          s1 = fmaf(R[i][c], cf[c], s1);
          s2 = fmaf(P[i][c], c2[c], s2);
        }
        *reinterpret_cast<float2*>(&part[tok_of(w, g, i)][2 * n]) = make_float2(s1, s2);
      }
    }
    __syncthreads();
    float2 m = reduce_pairs(part[t_red], hf);
    float mu = m.x * inv128, ey2 = m.y * inv128;
    float var = fmaf(-mu, mu, ey2);
    if (__syncthreads_or(!(var >= 0.5f * ey2))) {
      // centred second moment for the whole pass
      if (hf == 0) mul_c[t_red] = mu;
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float mi = mul_c[tok_of(w, g, i)];
        float q = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const float d = fmaf(R[i][c], cf[c], -mi);
          q = fmaf(d, d, q);
        }
        *reinterpret_cast<float2*>(&part[tok_of(w, g, i)][2 * n]) = make_float2(q, 0.f);
      }
      __syncthreads();
      var = reduce_pairs(part[t_red], hf).x * inv128;
    }
    rho_t += 0.5f * lg2(fmaf(var, rf_t * rf_t, kNormEps));
    rf_t = ex2(-rho_t);
    if (hf == 0) rfl[t_red] = rf_t;
    __syncthreads();
    {
      const float4 a = *reinterpret_cast<const float4*>(&rfl[32 * w + 4 * g]);
      const float4 b = *reinterpret_cast<const float4*>(&rfl[32 * w + 16 + 4 * g]);
      rf[0] = a.x; rf[1] = a.y; rf[2] = a.z; rf[3] = a.w;
      rf[4] = b.x; rf[5] = b.y; rf[6] = b.z; rf[7] = b.w;
    }
    // ---------------- column pass: moments over tokens of R * rf ------------
    {
      float r2[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) r2[i] = rf[i] * rf[i];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        float s1 = 0.f, s2 = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          s1 = fmaf(R[i][c], rf[i], s1);
          s2 = fmaf(P[i][c], r2[i], s2);
        }
        *reinterpret_cast<float2*>(&part[chan_of(n, c)][2 * (4 * w + g)]) = make_float2(s1, s2);
      }
    }
    __syncthreads();
    m = reduce_pairs(part[t_red], hf);
    mu = m.x * inv128;
    ey2 = m.y * inv128;
    var = fmaf(-mu, mu, ey2);
    if (__syncthreads_or(!(var >= 0.5f * ey2))) {
      if (hf == 0) mul_c[chan_slot(t_red)] = mu;
      __syncthreads();
      const float4 ma = *reinterpret_cast<const float4*>(&mul_c[8 * n]);
      const float4 mb = *reinterpret_cast<const float4*>(&mul_c[8 * n + 4]);
      const float mc[8] = {ma.x, ma.y, ma.z, ma.w, mb.x, mb.y, mb.z, mb.w};
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        float q = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float d = fmaf(R[i][c], rf[i], -mc[c]);
          q = fmaf(d, d, q);
        }
        *reinterpret_cast<float2*>(&part[chan_of(n, c)][2 * (4 * w + g)]) = make_float2(q, 0.f);
      }
      __syncthreads();
      var = reduce_pairs(part[t_red], hf).x * inv128;
    }
    gam_c += 0.5f * lg2(fmaf(var, cf_c * cf_c, kNormEps));
    cf_c = ex2(-gam_c);
    if (hf == 0) cfl[chan_slot(t_red)] = cf_c;
    __syncthreads();
    {
      const float4 a = *reinterpret_cast<const float4*>(&cfl[8 * n]);
      const float4 b = *reinterpret_cast<const float4*>(&cfl[8 * n + 4]);
      cf[0] = a.x; cf[1] = a.y; cf[2] = a.z; cf[3] = a.w;
      cf[4] = b.x; cf[5] = b.y; cf[6] = b.z; cf[7] = b.w;
    }
  }

  // Normalised values N = R * 2^-rho * 2^-gamma (in place).
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int c = 0; c < 8; ++c) R[i][c] = R[i][c] * rf[i] * cf[c];

  uint8_t* page_base = is_v ? v_pool + (static_cast<size_t>(page) * hkv + head) * kVPageBytes
                            : k_pool + (static_cast<size_t>(page) * hkv + head) * kKPageBytes;
  uint8_t* meta = page_base + (is_v ? kVCodeBytes : kKCodeBytes);
  if (hf == 0) {
    reinterpret_cast<float*>(meta + kMetaRho)[t_red] = rho_t;
    reinterpret_cast<float*>(meta + kMetaGamma)[t_red] = gam_c;
  }

  // ---- 3. per-group min/max, fp16 scale and zero, round to nearest ----------
  // Codes come out of u + 1.5*2^23, whose low mantissa bits hold round-half-even(u).
  constexpr float kRoundMagic = 12582912.0f;
  constexpr uint32_t kMagicBits = 0x4B400000u;
  if (!is_v) {
    // key groups: one channel over the 128 tokens, 16 levels
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float a = R[0][c], b = R[0][c];
#pragma unroll
      for (int i = 1; i < 8; ++i) {
        a = fminf(a, R[i][c]);
        b = fmaxf(b, R[i][c]);
      }
      *reinterpret_cast<float2*>(&part[chan_of(n, c)][2 * (4 * w + g)]) = make_float2(a, b);
    }
    __syncthreads();
    {
      const float4* p = reinterpret_cast<const float4*>(part[t_red] + 16 * hf);
      float mn = INFINITY, mx = -INFINITY;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float4 v = p[k];
        mn = fminf(mn, fminf(v.x, v.z));
        mx = fmaxf(mx, fmaxf(v.y, v.w));
      }
      mn = fminf(mn, dpp_xor1(mn));
      mx = fmaxf(mx, dpp_xor1(mx));
      const uint32_t sb = float_to_half_bits((mx - mn) / 15.0f);
      const uint32_t zb = float_to_half_bits(mn);
      const float sf = half_bits_to_float(sb), zf = half_bits_to_float(zb);
      const float inv = sf > 0.f ? 1.0f / sf : 0.f;
      if (hf == 0) {
        reinterpret_cast<uint16_t*>(meta + kMetaScale)[t_red] = static_cast<uint16_t>(sb);
        reinterpret_cast<uint16_t*>(meta + kMetaZero)[t_red] = static_cast<uint16_t>(zb);
        mul_a[chan_slot(t_red)] = inv;
        mul_b[chan_slot(t_red)] = -zf * inv;
      }
    }
    __syncthreads();
    const float4 a0 = *reinterpret_cast<const float4*>(&mul_a[8 * n]);
    const float4 a1 = *reinterpret_cast<const float4*>(&mul_a[8 * n + 4]);
    const float4 b0 = *reinterpret_cast<const float4*>(&mul_b[8 * n]);
    const float4 b1 = *reinterpret_cast<const float4*>(&mul_b[8 * n + 4]);
    const float qa[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
    const float qb[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int ch = chan_of(n, c);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float u = fmaf(R[i][c], qa[c], qb[c]) + kRoundMagic;
        const uint32_t bits = min(max(__float_as_uint(u), kMagicBits), kMagicBits + 15u);
        codes[tok_of(w, g, i) * kHeadDim + ch] = static_cast<uint8_t>(bits);
      }
    }
  } else {
    // value groups: one token over the 128 channels, 4 levels
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float a = R[i][0], b = R[i][0];
#pragma unroll
      for (int c = 1; c < 8; ++c) {
        a = fminf(a, R[i][c]);
        b = fmaxf(b, R[i][c]);
      }
      *reinterpret_cast<float2*>(&part[tok_of(w, g, i)][2 * n]) = make_float2(a, b);
    }
    __syncthreads();
    {
      const float4* p = reinterpret_cast<const float4*>(part[t_red] + 16 * hf);
      float mn = INFINITY, mx = -INFINITY;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float4 v = p[k];
        mn = fminf(mn, fminf(v.x, v.z));
        mx = fmaxf(mx, fmaxf(v.y, v.w));
      }
      mn = fminf(mn, dpp_xor1(mn));
      mx = fmaxf(mx, dpp_xor1(mx));
      const uint32_t sb = float_to_half_bits((mx - mn) / 3.0f);
      const uint32_t zb = float_to_half_bits(mn);
      const float sf = half_bits_to_float(sb), zf = half_bits_to_float(zb);
      const float inv = sf > 0.f ? 1.0f / sf : 0.f;
      if (hf == 0) {
        reinterpret_cast<uint16_t*>(meta + kMetaScale)[t_red] = static_cast<uint16_t>(sb);
        reinterpret_cast<uint16_t*>(meta + kMetaZero)[t_red] = static_cast<uint16_t>(zb);
        mul_a[t_red] = inv;
        mul_b[t_red] = -zf * inv;
      }
    }
    __syncthreads();
    float qa[8], qb[8];
    {
      const float4 a0 = *reinterpret_cast<const float4*>(&mul_a[32 * w + 4 * g]);
      const float4 a1 = *reinterpret_cast<const float4*>(&mul_a[32 * w + 16 + 4 * g]);
      const float4 b0 = *reinterpret_cast<const float4*>(&mul_b[32 * w + 4 * g]);
      const float4 b1 = *reinterpret_cast<const float4*>(&mul_b[32 * w + 16 + 4 * g]);
      qa[0] = a0.x; qa[1] = a0.y; qa[2] = a0.z; qa[3] = a0.w; qa[4] = a1.x; qa[5] = a1.y; qa[6] = a1.z; qa[7] = a1.w;
      qb[0] = b0.x; qb[1] = b0.y; qb[2] = b0.z; qb[3] = b0.w; qb[4] = b1.x; qb[5] = b1.y; qb[6] = b1.z; qb[7] = b1.w;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int t = tok_of(w, g, i);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float u = fmaf(R[i][c], qa[i], qb[i]) + kRoundMagic;
        const uint32_t bits = min(max(__float_as_uint(u), kMagicBits), kMagicBits + 3u);
        codes[chan_of(n, c) * kBlockTokens + t] = static_cast<uint8_t>(bits);
      }
    }
  }
  __syncthreads();

  // ---- 4. pack codes and store ---------------------------------------------
  if (!is_v) {
    // K: token t = tid/2, channels 64*(tid%2) .. +63 -> 32 bytes, two nibbles per byte
    const int t = tid >> 1;
    const u32x4* srcv = reinterpret_cast<const u32x4*>(codes + t * kHeadDim + 64 * hf);
    u32x4 o[2];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const u32x4 x = srcv[q4];
      uint32_t pk[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t v = x[e];  // four codes, one per byte
        pk[e] = (v & 0xFu) | ((v >> 4) & 0xF0u) | (((v >> 16) & 0xFu) << 8) | (((v >> 20) & 0xF0u) << 8);
      }
      o[q4 >> 1][(q4 & 1) * 2 + 0] = pk[0] | (pk[1] << 16);
      o[q4 >> 1][(q4 & 1) * 2 + 1] = pk[2] | (pk[3] << 16);
    }
    u32x4* dst = reinterpret_cast<u32x4*>(page_base + t * 64 + 32 * hf);
    dst[0] = o[0];
    dst[1] = o[1];
  } else {
    // V: channel c = tid/2, tokens 64*(tid%2) .. +63 -> 16 bytes, four codes per byte
    const int c = tid >> 1;
    const u32x4* srcv = reinterpret_cast<const u32x4*>(codes + c * kBlockTokens + 64 * hf);
    u32x4 o;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const u32x4 x = srcv[q4];
      uint32_t word = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t v = x[e];
        const uint32_t byte = (v & 3u) | ((v >> 6) & 0xCu) | ((v >> 12) & 0x30u) | ((v >> 18) & 0xC0u);
        word |= byte << (8 * e);
      }
      o[q4] = word;
    }
    *reinterpret_cast<u32x4*>(page_base + c * 32 + 16 * hf) = o;
  }
}

// Test / inspection export: rebuild fp32 K^ or V^ of one tile in the original basis.
__global__ __launch_bounds__(256) void dequantize_kernel(const uint8_t* __restrict__ k_pool,
                                                         const uint8_t* __restrict__ v_pool, int num_pages,
                                                         const int32_t* __restrict__ pages, int hkv,
                                                         float* __restrict__ k_out, float* __restrict__ v_out,
                                                         uint32_t* __restrict__ flags) {
  __shared__ float buf[kBlockTokens][kHeadDim + 1];
  const int tile = blockIdx.x;
  const bool is_v = tile & 1;
  const int bh = tile >> 1;
  const int blk = bh / hkv;
  const int head = bh - blk * hkv;
  float* out = is_v ? v_out : k_out;
  if (out == nullptr) return;
  const int page = pages[blk];
  if (page < 0 || page >= num_pages) {
    if (threadIdx.x == 0 && flags) atomicOr(flags, kFlagBadPage);
    return;
  }
  const uint8_t* pb = is_v ? v_pool + (static_cast<size_t>(page) * hkv + head) * kVPageBytes
                           : k_pool + (static_cast<size_t>(page) * hkv + head) * kKPageBytes;
  const uint8_t* meta = pb + (is_v ? kVCodeBytes : kKCodeBytes);
  const uint16_t* sc = reinterpret_cast<const uint16_t*>(meta + kMetaScale);
  const uint16_t* zr = reinterpret_cast<const uint16_t*>(meta + kMetaZero);
  const float* rho = reinterpret_cast<const float*>(meta + kMetaRho);
  const float* gam = reinterpret_cast<const float*>(meta + kMetaGamma);
  for (int e = threadIdx.x; e < kBlockTokens * kHeadDim; e += blockDim.x) {
    const int t = e >> 7, j = e & 127;
    uint32_t code;
    float s, z;
    if (is_v) {
      code = (pb[32 * j + (t >> 2)] >> (2 * (t & 3))) & 3u;
      s = half_bits_to_float(sc[t]);
      z = half_bits_to_float(zr[t]);
    } else {
      code = (pb[64 * t + (j >> 1)] >> (4 * (j & 1))) & 15u;
      s = half_bits_to_float(sc[j]);
      z = half_bits_to_float(zr[j]);
    }
    buf[t][j] = fmaf(s, static_cast<float>(code), z) * exp2f(rho[t] + gam[j]);
  }
  __syncthreads();
  // in-LDS fast Walsh-Hadamard transform along channels of every token
  for (int half = 1; half < kHeadDim; half <<= 1) {
    for (int u = threadIdx.x; u < kBlockTokens * kHeadDim / 2; u += blockDim.x) {
      const int t = u >> 6, p = u & 63;
      const int i = (p / half) * 2 * half + (p % half);
      const float a = buf[t][i], b = buf[t][i + half];
      buf[t][i] = a + b;
      buf[t][i + half] = a - b;
    }
    __syncthreads();
  }
  for (int e = threadIdx.x; e < kBlockTokens * kHeadDim; e += blockDim.x) {
    const int t = e >> 7, j = e & 127;
    out[(static_cast<size_t>(blk) * kBlockTokens + t) * hkv * kHeadDim + static_cast<size_t>(head) * kHeadDim + j] =
        buf[t][j] * kInvSqrt128;
  }
}

}  // namespace kvarn

namespace kvarn {

hipError_t launch_quantize(const void* k, const void* v, int n_blocks, int hkv, const int32_t* dst_pages,
                           void* k_pool, void* v_pool, int num_pages, uint32_t* flags, hipStream_t stream) {
  const unsigned tiles = 2u * static_cast<unsigned>(n_blocks) * static_cast<unsigned>(hkv);
  hipLaunchKernelGGL(quantize_kernel, dim3(tiles), dim3(256), 0, stream, static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), hkv, dst_pages, static_cast<uint8_t*>(k_pool),
                     static_cast<uint8_t*>(v_pool), num_pages, flags);
  return hipGetLastError();
}

hipError_t launch_dequantize(const void* k_pool, const void* v_pool, int num_pages, const int32_t* pages,
                             int n_blocks, int hkv, float* k_out, float* v_out, uint32_t* flags, hipStream_t stream) {
  const unsigned tiles = 2u * static_cast<unsigned>(n_blocks) * static_cast<unsigned>(hkv);
  hipLaunchKernelGGL(dequantize_kernel, dim3(tiles), dim3(256), 0, stream, static_cast<const uint8_t*>(k_pool),
                     static_cast<const uint8_t*>(v_pool), num_pages, pages, hkv, k_out, v_out, flags);
  return hipGetLastError();
}

}  // namespace kvarn
