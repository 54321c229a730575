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
// Row statistics (over channels) reduce over the 16 lanes of a DPP row;
// column statistics (over tokens) reduce over the four rows of the wave and
// then over the four waves through LDS.  Every reduction uses a fixed
// pairing so all lanes that share a row or column see identical bits.
#include "kvarn_common.h"

namespace kvarn {

namespace {

__device__ __forceinline__ int tok_of(int w, int g, int i) { return 32 * w + 16 * (i >> 2) + 4 * g + (i & 3); }
__device__ __forceinline__ int chan_of(int n, int c) { return 32 * (c >> 1) + 16 * (c & 1) + n; }

}  // namespace

__global__ __launch_bounds__(256, 2) void quantize_kernel(const uint16_t* __restrict__ kin,
                                                         const uint16_t* __restrict__ vin, int hkv,
                                                         const int32_t* __restrict__ dst_pages,
                                                         uint8_t* __restrict__ k_pool, uint8_t* __restrict__ v_pool,
                                                         int num_pages, uint32_t* __restrict__ flags) {
  __shared__ float red[2][4][kHeadDim];                // cross-wave column partials (double buffered)
  __shared__ __align__(16) uint8_t codes[kBlockTokens * kHeadDim];  // staged codes, one byte each

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

  // ---- 2. log2-variance normalisation, rows then columns, kNormIters times --
  float rho[8], gam[8], rf[8], cf[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    rho[k] = 0.f;
    gam[k] = 0.f;
    rf[k] = 1.f;
    cf[k] = 1.f;
  }
  int buf = 0;
  // Column reduction of v[c] over all 128 tokens (rows of the wave, then waves).
  auto col_sum = [&](float (&v)[8]) {
#pragma unroll
    for (int c = 0; c < 8; ++c) v[c] = rows4_sum(v[c]);
    if (g == 0) {
#pragma unroll
      for (int c = 0; c < 8; ++c) red[buf][w][chan_of(n, c)] = v[c];
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int ch = chan_of(n, c);
      v[c] = ((red[buf][0][ch] + red[buf][1][ch]) + red[buf][2][ch]) + red[buf][3][ch];
    }
    buf ^= 1;
  };

  constexpr float inv128 = 1.0f / 128.0f;
  for (int it = 0; it < kNormIters; ++it) {
    // row pass: variance over channels of Y = R * rf[i] * cf[c]
    float mu[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float s = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) s = fmaf(R[i][c], cf[c], s);
      mu[i] = row16_sum(s) * inv128;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float q = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float d = fmaf(R[i][c], cf[c], -mu[i]);
        q = fmaf(d, d, q);
      }
      const float var = row16_sum(q) * inv128 * (rf[i] * rf[i]);
      rho[i] += 0.5f * log2f(var + kNormEps);
      rf[i] = exp2f(-rho[i]);
    }
    // column pass: variance over tokens of Y = R * rf[i] * cf[c]
    float cm[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) s = fmaf(R[i][c], rf[i], s);
      cm[c] = s;
    }
    col_sum(cm);
#pragma unroll
    for (int c = 0; c < 8; ++c) cm[c] *= inv128;
    float cq[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float q = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float d = fmaf(R[i][c], rf[i], -cm[c]);
        q = fmaf(d, d, q);
      }
      cq[c] = q;
    }
    col_sum(cq);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float var = cq[c] * inv128 * (cf[c] * cf[c]);
      gam[c] += 0.5f * log2f(var + kNormEps);
      cf[c] = exp2f(-gam[c]);
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

  // ---- 3. per-group min/max, fp16 scale and zero, round to nearest ----------
  if (!is_v) {
    // key groups: one channel over the 128 tokens, 16 levels
    float mn[8], mx[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float a = R[0][c], b = R[0][c];
#pragma unroll
      for (int i = 1; i < 8; ++i) {
        a = fminf(a, R[i][c]);
        b = fmaxf(b, R[i][c]);
      }
      mn[c] = rows4_min(a);
      mx[c] = rows4_max(b);
    }
    __syncthreads();  // the last column reduction may still be reading red
    if (g == 0) {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        red[0][w][chan_of(n, c)] = mn[c];
        red[1][w][chan_of(n, c)] = mx[c];
      }
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int ch = chan_of(n, c);
      mn[c] = fminf(fminf(red[0][0][ch], red[0][1][ch]), fminf(red[0][2][ch], red[0][3][ch]));
      mx[c] = fmaxf(fmaxf(red[1][0][ch], red[1][1][ch]), fmaxf(red[1][2][ch], red[1][3][ch]));
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint32_t sb = float_to_half_bits((mx[c] - mn[c]) / 15.0f);
      const uint32_t zb = float_to_half_bits(mn[c]);
      const float s = half_bits_to_float(sb), z = half_bits_to_float(zb);
      const float inv = s > 0.f ? 1.0f / s : 0.f;
      const int ch = chan_of(n, c);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float u = rintf((R[i][c] - z) * inv);
        const float qc = fminf(fmaxf(u, 0.f), 15.f);
        codes[tok_of(w, g, i) * kHeadDim + ch] = static_cast<uint8_t>(qc);
      }
      if (w == 0 && g == 0) {
        reinterpret_cast<uint16_t*>(meta + kMetaScale)[ch] = static_cast<uint16_t>(sb);
        reinterpret_cast<uint16_t*>(meta + kMetaZero)[ch] = static_cast<uint16_t>(zb);
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
      const float mn = row16_min(a), mx = row16_max(b);
      const uint32_t sb = float_to_half_bits((mx - mn) / 3.0f);
      const uint32_t zb = float_to_half_bits(mn);
      const float s = half_bits_to_float(sb), z = half_bits_to_float(zb);
      const float inv = s > 0.f ? 1.0f / s : 0.f;
      const int t = tok_of(w, g, i);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float u = rintf((R[i][c] - z) * inv);
        const float qc = fminf(fmaxf(u, 0.f), 3.f);
        codes[chan_of(n, c) * kBlockTokens + t] = static_cast<uint8_t>(qc);
      }
      if (n == 0) {
        reinterpret_cast<uint16_t*>(meta + kMetaScale)[t] = static_cast<uint16_t>(sb);
        reinterpret_cast<uint16_t*>(meta + kMetaZero)[t] = static_cast<uint16_t>(zb);
      }
    }
  }

  // normalisers: rho per token (lanes n == 0), gamma per channel (wave 0, row 0)
  if (n == 0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) reinterpret_cast<float*>(meta + kMetaRho)[tok_of(w, g, i)] = rho[i];
  }
  if (w == 0 && g == 0) {
#pragma unroll
    for (int c = 0; c < 8; ++c) reinterpret_cast<float*>(meta + kMetaGamma)[chan_of(n, c)] = gam[c];
  }
  __syncthreads();

  // ---- 4. pack codes and store ---------------------------------------------
  if (!is_v) {
    // K: token t = tid/2, channels 64*(tid%2) .. +63 -> 32 bytes, two nibbles per byte
    const int t = tid >> 1, hf = tid & 1;
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
      // 8 input dwords (32 codes) -> 4 output dwords: out dword = pk[2e] | pk[2e+1] << 16
      o[q4 >> 1][(q4 & 1) * 2 + 0] = pk[0] | (pk[1] << 16);
      o[q4 >> 1][(q4 & 1) * 2 + 1] = pk[2] | (pk[3] << 16);
    }
    u32x4* dst = reinterpret_cast<u32x4*>(page_base + t * 64 + 32 * hf);
    dst[0] = o[0];
    dst[1] = o[1];
  } else {
    // V: channel c = tid/2, tokens 64*(tid%2) .. +63 -> 16 bytes, four codes per byte
    const int c = tid >> 1, hf = tid & 1;
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
