// Decode attention over the packed KVarN cache for gfx950.
//
// One wave handles one (sequence, KV head, split): the G <= 8 query heads that
// share the KV head attend to a contiguous run of 128-token pages.  Nothing is
// dequantised to memory.  Because the rotation is orthonormal (KVarN blog post,
// section "KVarN Nasıl Çalışır?": it keeps attention scores), the query is
// rotated once, q~ = H q, and both contractions run in the rotated basis:
//
//   key page:   score_t = 2^rho_t * ( sum_j a_j c_tj + b ),
//               a_j = q~_j 2^gamma_j s_j,   b = sum_j q~_j 2^gamma_j z_j
//   value page: o_j += 2^gamma_j * ( sum_t w_t c_tj + u ),
//               w_t = p_t 2^rho_t s_t,      u = sum_t p_t 2^rho_t z_t
//
// with online softmax over the pages of the split (scores kept in log2 units).
// Both sums over codes are dense (G x 128) x (128 x 128) products per page,
// run on v_mfma_f32_16x16x32_f16: codes enter as exact small integers (16 + c
// for 4-bit, 4 + c for 2-bit codes built with one mask-and-or per pair), the
// fp32 coefficients a_j and w_t as an fp16 hi + lo pair (22 significant bits)
// in the matrix's N columns 0-7 (hi) and 8-15 (lo), after scaling each page's
// coefficients by a power of two so the pair stays in fp16 range.  Lane n and
// lane n^8 of a DPP row then hold the two halves of the same head and add them.
//
// The splits of one (sequence, KV head) write (m, l, o[128]) partials; the last
// wave to arrive (per-pair counter in the workspace) merges them with
// log-sum-exp weights, applies the inverse rotation H and writes fp32 output.
#include "kvarn_common.h"

namespace kvarn {

namespace {

constexpr int kPartStride = kHeadDim + 2;  // o[128], m, l per (split, query head)

// Four fp16 pairs (16 + c) from one dword of 8 key nibbles; element order c0,c4,c1,c5,c2,c6,c3,c7.
__device__ __forceinline__ f16x8 key_codes_to_f16(u32x4 x4, int ks) {
  const uint32_t x = x4[ks];
  u32x4 p;
  p[0] = ((x << 6) & 0x03C003C0u) | 0x4C004C00u;
  p[1] = ((x << 2) & 0x03C003C0u) | 0x4C004C00u;
  p[2] = ((x >> 2) & 0x03C003C0u) | 0x4C004C00u;
  p[3] = ((x >> 6) & 0x03C003C0u) | 0x4C004C00u;
  return __builtin_bit_cast(f16x8, p);
}

// Channel (within the lane's 8-channel K-step chunk) of element i of key_codes_to_f16.
__device__ __forceinline__ constexpr int key_elem_channel(int i) { return (i >> 1) + 4 * (i & 1); }

// Four fp16 pairs (4 + c) from a word of 16 value codes (tokens 16u .. 16u+15 of the lane's 32):
// K-step half hf, pair j holds tokens 4hf + j and 4hf + j + 8.
__device__ __forceinline__ f16x8 value_codes_to_f16(uint32_t wd, int hf) {
  u32x4 p;
  if (hf == 0) {
    p[0] = ((wd << 8) & 0x03000300u) | 0x44004400u;
    p[1] = ((wd << 6) & 0x03000300u) | 0x44004400u;
    p[2] = ((wd << 4) & 0x03000300u) | 0x44004400u;
    p[3] = ((wd << 2) & 0x03000300u) | 0x44004400u;
  } else {
    p[0] = (wd & 0x03000300u) | 0x44004400u;
    p[1] = ((wd >> 2) & 0x03000300u) | 0x44004400u;
    p[2] = ((wd >> 4) & 0x03000300u) | 0x44004400u;
    p[3] = ((wd >> 6) & 0x03000300u) | 0x44004400u;
  }
  return __builtin_bit_cast(f16x8, p);
}

__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  return float_to_half_bits(lo) | (float_to_half_bits(hi) << 16);
}

// In-LDS 128-point Walsh-Hadamard transform of `rows` vectors of 128 floats (one wave).
__device__ void lds_fwht(float (*v)[kHeadDim], int rows) {
  for (int half = 1; half < kHeadDim; half <<= 1) {
    for (int u = threadIdx.x; u < rows * 64; u += 64) {
      const int r = u >> 6, p = u & 63;
      const int i = (p / half) * 2 * half + (p % half);
      const float a = v[r][i], b = v[r][i + half];
      v[r][i] = a + b;
      v[r][i + half] = a - b;
    }
    __syncthreads();
  }
}

}  // namespace

__global__ __launch_bounds__(64) void decode_kernel(const uint16_t* __restrict__ q, const uint8_t* __restrict__ k_pool,
                                                    const uint8_t* __restrict__ v_pool, int num_pages,
                                                    const int32_t* __restrict__ block_table, int max_blocks,
                                                    const int32_t* __restrict__ seq_lens, int hq, int hkv,
                                                    int blocks_per_split, int max_splits, float scale_log2,
                                                    float* __restrict__ out, float* __restrict__ part,
                                                    uint32_t* __restrict__ counters, uint32_t* __restrict__ flags) {
  __shared__ float qs[kMaxGroup][kHeadDim];
  __shared__ float e_k[kHeadDim], f_k[kHeadDim], p_k[kHeadDim];      // per page: 2^g s, 2^g z (K), 2^rho (K)
  __shared__ float f_v[kHeadDim], z_v[kHeadDim], g_v[kHeadDim];      // per page: 2^rho s, 2^rho z (V), 2^g (V)
  __shared__ int last_flag;

  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int G = hq / hkv;
  const int lane = threadIdx.x, n = lane & 15, g = lane >> 4;
  const int hd = n & 7;        // query head (within the group) of this lane's MFMA column
  const bool lo_col = n >= 8;  // column holds the lo fp16 part
  const int sl = seq_lens[b];
  float* out_b = out + (static_cast<size_t>(b) * hq + static_cast<size_t>(kvh) * G) * kHeadDim;

  const bool bad = sl < 0 || (sl & (kBlockTokens - 1)) != 0 || sl > max_blocks * kBlockTokens;
  const int nblk = bad ? 0 : sl / kBlockTokens;
  if (nblk == 0) {
    if (split == 0) {
      if (bad && lane == 0 && flags) atomicOr(flags, kFlagBadSeqLen);
      for (int e = lane; e < G * kHeadDim; e += 64) out_b[e] = 0.f;
    }
    return;
  }
  const int nsplit = (nblk + blocks_per_split - 1) / blocks_per_split;
  if (split >= nsplit) return;
  const int blk0 = split * blocks_per_split;
  const int blk1 = min(nblk, blk0 + blocks_per_split);

  // ---- rotated, scaled query: qs[h][j] = scale*log2(e) * (H q_h)_j ----------
  const uint16_t* qb = q + (static_cast<size_t>(b) * hq + static_cast<size_t>(kvh) * G) * kHeadDim;
  for (int e = lane; e < kMaxGroup * kHeadDim; e += 64) {
    const int h = e >> 7, j = e & 127;
    qs[h][j] = h < G ? half_bits_to_float(qb[h * kHeadDim + j]) : 0.f;
  }
  __syncthreads();
  lds_fwht(qs, kMaxGroup);
  float qv[32];  // q~[hd][32g + k] for this lane's head and channel quarter
  float qmax = 0.f;
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    qv[k] = qs[hd][32 * g + k] * (kInvSqrt128 * scale_log2);
    qmax = fmaxf(qmax, fabsf(qv[k]));
  }
  qmax = rows4_max(qmax);  // max |q~| of head hd (same on lanes n and n^8)

  float m_run = -INFINITY, l_run = 0.f;
  float acc[8][4];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[mt][r] = 0.f;

  const int32_t* bt = block_table + static_cast<size_t>(b) * max_blocks;
  for (int blk = blk0; blk < blk1; ++blk) {
    const int page = bt[blk];
    if (page < 0 || page >= num_pages) {
      if (lane == 0 && flags) atomicOr(flags, kFlagBadPage);
      continue;
    }
    const uint8_t* kp = k_pool + (static_cast<size_t>(page) * hkv + kvh) * kKPageBytes;
    const uint8_t* vp = v_pool + (static_cast<size_t>(page) * hkv + kvh) * kVPageBytes;

    // key codes: M-tile mt, row n -> token 32*(n/4) + 4*mt + n%4, channels 32g .. 32g+31
    u32x4 kc[8];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      const int tok = 32 * (n >> 2) + 4 * mt + (n & 3);
      kc[mt] = *reinterpret_cast<const u32x4*>(kp + tok * 64 + 16 * g);
    }
    // value codes: M-tile mt, row n -> channel 16mt + n, tokens 32g .. 32g+31
    u32x2 vc[8];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) vc[mt] = *reinterpret_cast<const u32x2*>(vp + (16 * mt + n) * 32 + 8 * g);

    // per-page factors, two entries per lane
    {
      const uint8_t* km = kp + kKCodeBytes;
      const uint8_t* vm = vp + kVCodeBytes;
      const uint32_t ks2 = reinterpret_cast<const uint32_t*>(km + kMetaScale)[lane];
      const uint32_t kz2 = reinterpret_cast<const uint32_t*>(km + kMetaZero)[lane];
      const float2 kr2 = reinterpret_cast<const float2*>(km + kMetaRho)[lane];
      const float2 kg2 = reinterpret_cast<const float2*>(km + kMetaGamma)[lane];
      const uint32_t vs2 = reinterpret_cast<const uint32_t*>(vm + kMetaScale)[lane];
      const uint32_t vz2 = reinterpret_cast<const uint32_t*>(vm + kMetaZero)[lane];
      const float2 vr2 = reinterpret_cast<const float2*>(vm + kMetaRho)[lane];
      const float2 vg2 = reinterpret_cast<const float2*>(vm + kMetaGamma)[lane];
      const float kgx = exp2f(kg2.x), kgy = exp2f(kg2.y);
      const float vrx = exp2f(vr2.x), vry = exp2f(vr2.y);
      e_k[2 * lane] = kgx * half_bits_to_float(ks2 & 0xFFFFu);
      e_k[2 * lane + 1] = kgy * half_bits_to_float(ks2 >> 16);
      f_k[2 * lane] = kgx * half_bits_to_float(kz2 & 0xFFFFu);
      f_k[2 * lane + 1] = kgy * half_bits_to_float(kz2 >> 16);
      p_k[2 * lane] = exp2f(kr2.x);
      p_k[2 * lane + 1] = exp2f(kr2.y);
      f_v[2 * lane] = vrx * half_bits_to_float(vs2 & 0xFFFFu);
      f_v[2 * lane + 1] = vry * half_bits_to_float(vs2 >> 16);
      z_v[2 * lane] = vrx * half_bits_to_float(vz2 & 0xFFFFu);
      z_v[2 * lane + 1] = vry * half_bits_to_float(vz2 >> 16);
      g_v[2 * lane] = exp2f(vg2.x);
      g_v[2 * lane + 1] = exp2f(vg2.y);
    }
    __syncthreads();

    // ---- key side: coefficients (B operand) -------------------------------
    float emax = 0.f;
#pragma unroll
    for (int k = 0; k < 2; ++k) emax = fmaxf(emax, e_k[2 * lane + k]);
    emax = wave_max(emax);
    int ex;
    frexpf(qmax * emax, &ex);
    ex = min(max(ex, -100), 100);
    const float sa = (qmax * emax > 0.f) ? pow2i(14 - ex) : 1.f;  // keeps |a| <= 2^14
    const float inv_sa = (qmax * emax > 0.f) ? pow2i(ex - 14) : 1.f;
    f16x8 coef[4];
    float asum = 0.f, bsum = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4 pk;
#pragma unroll
      for (int pr = 0; pr < 4; ++pr) {
        float part2[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const int kk = 8 * ks + key_elem_channel(2 * pr + s);  // channel offset within the lane's 32
          const float a = qv[kk] * e_k[32 * g + kk] * sa;
          const float hi = half_bits_to_float(float_to_half_bits(a));
          const float lo = half_bits_to_float(float_to_half_bits(a - hi));
          asum += hi + lo;
          bsum = fmaf(qv[kk], f_k[32 * g + kk], bsum);
          part2[s] = lo_col ? lo : hi;
        }
        pk[pr] = pack_f16x2(part2[0], part2[1]);
      }
      coef[ks] = __builtin_bit_cast(f16x8, pk);
    }
    asum = rows4_sum(asum);
    bsum = rows4_sum(bsum);
    const float off = bsum - 16.f * asum * inv_sa;

    // ---- key side: scores -------------------------------------------------
    float s[8][4];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) d = mfma16x16x32(key_codes_to_f16(kc[mt], ks), coef[ks], d);
#pragma unroll
      for (int r = 0; r < 4; ++r) s[mt][r] = d[r] + dpp<kDppXor8>(d[r]);
    }
    // s[mt][r] belongs to token 32g + 4mt + r
    float mloc = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        s[mt][r] = p_k[32 * g + 4 * mt + r] * fmaf(s[mt][r], inv_sa, off);
        mloc = fmaxf(mloc, s[mt][r]);
      }
    mloc = rows4_max(mloc);
    const float m_new = fmaxf(m_run, mloc);
    const float alpha = exp2f(m_run - m_new);
    m_run = m_new;

    // ---- softmax weights and value-side coefficients ----------------------
    float fmax_ = 0.f;
#pragma unroll
    for (int k = 0; k < 2; ++k) fmax_ = fmaxf(fmax_, f_v[2 * lane + k]);
    fmax_ = wave_max(fmax_);
    frexpf(fmax_, &ex);
    ex = min(max(ex, -100), 100);
    const float sw = fmax_ > 0.f ? pow2i(14 - ex) : 1.f;  // p <= 1, so |w| <= 2^14
    const float inv_sw = fmax_ > 0.f ? pow2i(ex - 14) : 1.f;
    float lsum = 0.f, usum = 0.f, wsum = 0.f;
    float wv[8][4];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 32 * g + 4 * mt + r;
        const float p = exp2f(s[mt][r] - m_new);
        lsum += p;
        usum = fmaf(p, z_v[t], usum);
        const float wt = p * f_v[t] * sw;
        const float hi = half_bits_to_float(float_to_half_bits(wt));
        const float lo = half_bits_to_float(float_to_half_bits(wt - hi));
        wsum += hi + lo;
        wv[mt][r] = lo_col ? lo : hi;
      }
    lsum = rows4_sum(lsum);
    usum = rows4_sum(usum);
    wsum = rows4_sum(wsum);
    l_run = l_run * alpha + lsum;
    // B operand per K-step ks = 2u + hf: pair j = (token 16u + 4hf + j, +8) of the lane's 32
    f16x8 wb[4];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        u32x4 pk;
#pragma unroll
        for (int j = 0; j < 4; ++j) pk[j] = pack_f16x2(wv[4 * u + hf][j], wv[4 * u + hf + 2][j]);
        wb[2 * u + hf] = __builtin_bit_cast(f16x8, pk);
      }
    const float voff = usum - 4.f * wsum * inv_sw;

    // ---- value side: o (rotated basis) ------------------------------------
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) d = mfma16x16x32(value_codes_to_f16(vc[mt][u], hf), wb[2 * u + hf], d);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float tot = d[r] + dpp<kDppXor8>(d[r]);
        const int ch = 16 * mt + 4 * g + r;
        acc[mt][r] = fmaf(acc[mt][r], alpha, g_v[ch] * fmaf(tot, inv_sw, voff));
      }
    }
    __syncthreads();  // the per-page factor arrays are rewritten by the next page
  }

  // ---- write this split's partial ------------------------------------------
  const size_t pair = static_cast<size_t>(b) * hkv + kvh;
  float* pbase = part + pair * max_splits * kMaxGroup * kPartStride;
  if (!lo_col && hd < G) {
    float* pp = pbase + (static_cast<size_t>(split) * kMaxGroup + hd) * kPartStride;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) pp[16 * mt + 4 * g + r] = acc[mt][r];
    if (g == 0) {
      pp[kHeadDim] = m_run;
      pp[kHeadDim + 1] = l_run;
    }
  }
  __threadfence();
  __syncthreads();
  if (lane == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(counters + pair, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    last_flag = (prev == static_cast<uint32_t>(nsplit - 1));
  }
  __syncthreads();
  if (!last_flag) return;
  __threadfence();
  if (lane == 0) counters[pair] = 0u;  // leave the counter ready for the next call

  // ---- merge the splits (log-sum-exp) and undo the rotation ---------------
  for (int e = lane; e < G * kHeadDim; e += 64) {
    const int h = e >> 7, j = e & 127;
    float mx = -INFINITY;
    for (int sp = 0; sp < nsplit; ++sp)
      mx = fmaxf(mx, pbase[(static_cast<size_t>(sp) * kMaxGroup + h) * kPartStride + kHeadDim]);
    float num = 0.f, den = 0.f;
    for (int sp = 0; sp < nsplit; ++sp) {
      const float* pp = pbase + (static_cast<size_t>(sp) * kMaxGroup + h) * kPartStride;
      const float ms = pp[kHeadDim];
      if (ms == -INFINITY) continue;  // a split whose pages were all rejected
      const float wgt = exp2f(ms - mx);
      num = fmaf(wgt, pp[j], num);
      den = fmaf(wgt, pp[kHeadDim + 1], den);
    }
    qs[h][j] = den > 0.f ? num / den : 0.f;
  }
  __syncthreads();
  lds_fwht(qs, G);
  for (int e = lane; e < G * kHeadDim; e += 64) out_b[e] = qs[e >> 7][e & 127] * kInvSqrt128;
}

}  // namespace kvarn

namespace kvarn {

hipError_t launch_decode(const void* q, const void* k_pool, const void* v_pool, int num_pages,
                         const int32_t* block_table, int max_blocks, const int32_t* seq_lens, int batch, int hq,
                         int hkv, int blocks_per_split, int max_splits, float scale_log2, float* out, float* part,
                         uint32_t* counters, uint32_t* flags, hipStream_t stream) {
  hipLaunchKernelGGL(decode_kernel, dim3(max_splits, hkv, batch), dim3(64), 0, stream, static_cast<const uint16_t*>(q),
                     static_cast<const uint8_t*>(k_pool), static_cast<const uint8_t*>(v_pool), num_pages, block_table,
                     max_blocks, seq_lens, hq, hkv, blocks_per_split, max_splits, scale_log2, out, part, counters,
                     flags);
  return hipGetLastError();
}

}  // namespace kvarn
