// Decode attention over the packed KVarN cache for gfx950.
//
// A workgroup of four waves handles one (sequence, KV head, split): the G <= 8
// query heads that share the KV head attend to a run of 128-token pages, wave
// w taking every fourth page.  Nothing is dequantised to memory.  Because the
// rotation is orthonormal (KVarN blog post, section "KVarN Nasıl Çalışır?": it
// keeps attention scores), the query is rotated once, q~ = H q, and both
// contractions run in the rotated basis:
//
//   key page:   score_t = 2^rho_t * ( sum_j a_j c_tj + b ),
//               a_j = q~_j 2^gamma_j s_j,   b = sum_j q~_j 2^gamma_j z_j
//   value page: o_j += 2^gamma_j * ( sum_t w_t c_tj + u ),
//               w_t = p_t 2^rho_t s_t,      u = sum_t p_t 2^rho_t z_t
//
// with online softmax over the pages (scores in log2 units).  Both sums over
// codes are dense (G x 128) x (128 x 128) products per page and run on
// v_mfma_f32_16x16x32_f16.  Codes enter as exact fp16 integers 16 + c (4-bit
// keys) or 4 + c (2-bit values): one shift and one mask-and-or per pair of codes
// places c in the top mantissa bits under a fixed exponent.  The offset is
// removed afterwards with the page's sum of coefficients (16 sum a, 4 sum w).
// (fp16 subnormal operands would avoid the offset, but the matrix cores lose
// precision on them, biased toward zero.)  The fp32 coefficients a_j and w_t
// enter as an fp16 hi + lo pair (hi in matrix columns 0-7, lo in columns 8-15,
// after a power-of-two page scale keeps them in fp16 range); lane n and lane
// n^8 of a DPP row then hold the two halves of the same query head.
//
// Each wave keeps (m, l, o[128]) per head; the four waves merge through LDS,
// the workgroup writes one partial per split, and the last workgroup of a
// (sequence, KV head) to arrive merges the splits with log-sum-exp weights,
// applies the inverse rotation H and writes fp32 output.
#include "kvarn_common.h"

namespace kvarn {

namespace {

constexpr int kWaves = 4;
constexpr int kPartStride = kHeadDim + 2;  // o[128], m, l per (split, query head)
constexpr int kCoefStride = 68;            // dwords per coefficient column (64 slots + pad)
constexpr int kMaxSplits = 64;             // the host plan never exceeds this many splits per (sequence, KV head)

// Mask-and-or with the mask in a scalar register and the fp16 exponent pattern in a
// vector register (one v_and_or_b32; the two literal constants would not fit one VOP3).
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t mask, uint32_t bits) {
  return (x & mask) | bits;
}

// Four fp16 pairs (16 + c) from one dword of 8 key nibbles (channel c at bits 4c):
// elements (0..7) = channels 0,4,1,5,2,6,3,7.  `mag` holds 0x4C004C00 (fp16 16.0 twice).
__device__ __forceinline__ f16x8 key_codes(uint32_t x, uint32_t mag) {
  u32x4 p;
  p[0] = and_or(x << 6, 0x03C003C0u, mag);
  p[1] = and_or(x << 2, 0x03C003C0u, mag);
  p[2] = and_or(x >> 2, 0x03C003C0u, mag);
  p[3] = and_or(x >> 6, 0x03C003C0u, mag);
  return __builtin_bit_cast(f16x8, p);
}

// Four fp16 pairs (4 + c) from a word of 16 value codes (code k at bits 2k), K-step half hf:
// pair j holds codes k = 4hf + j and k + 8, moved to mantissa bits 8-9 of each half.
// `mag` holds 0x44004400 (fp16 4.0 twice).
__device__ __forceinline__ f16x8 value_codes(uint32_t w, int hf, uint32_t mag) {
  u32x4 p;
  if (hf == 0) {
    p[0] = and_or(w << 8, 0x03000300u, mag);
    p[1] = and_or(w << 6, 0x03000300u, mag);
    p[2] = and_or(w << 4, 0x03000300u, mag);
    p[3] = and_or(w << 2, 0x03000300u, mag);
  } else {
    p[0] = and_or(w, 0x03000300u, mag);
    p[1] = and_or(w >> 2, 0x03000300u, mag);
    p[2] = and_or(w >> 4, 0x03000300u, mag);
    p[3] = and_or(w >> 6, 0x03000300u, mag);
  }
  return __builtin_bit_cast(f16x8, p);
}

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Split two fp32 values into packed fp16 hi and lo parts, both rounded to nearest even
// (v_cvt_pk_f16_f32, which keeps fp16 subnormals; the round-toward-zero packing
// instruction flushes them, and a flushed lo part biases every sum it enters).  The
// residual x - hi is exact in fp32, so hi + lo carries about 22 significant bits.
// The empty asm pins a and b as rounded fp32 values: otherwise the compiler may fuse the
// caller's product into a mixed-precision FMA for one of the two uses of hi (rounding the
// exact product to fp16 once) and not for the other, and at an fp32 rounding tie the two
// hi values differ by one fp16 ulp, which hi + lo then carries as an error.
__device__ __forceinline__ void split_pair(float a, float b, uint32_t& hi, uint32_t& lo) {
  asm("" : "+v"(a), "+v"(b));
  const f16x2 h = {static_cast<_Float16>(a), static_cast<_Float16>(b)};
  const f16x2 l = {static_cast<_Float16>(a - static_cast<float>(h[0])),
                   static_cast<_Float16>(b - static_cast<float>(h[1]))};
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

// Max / sum over the 8 lanes that hold one query head (lanes n, n^8 in each of the 4 rows).
__device__ __forceinline__ float head_max(float x) {
  x = fmaxf(x, dpp<kDppXor8>(x));
  return rows4_max(x);
}
__device__ __forceinline__ float head_sum(float x) {
  x += dpp<kDppXor8>(x);
  return rows4_sum(x);
}

__device__ __forceinline__ float wave_sum(float x) { return rows4_sum(row16_sum(x)); }

// In-LDS 128-point Walsh-Hadamard transform of `rows` vectors (whole workgroup).
__device__ void lds_fwht(float (*v)[kHeadDim], int rows) {
  for (int half = 1; half < kHeadDim; half <<= 1) {
    for (int u = threadIdx.x; u < rows * 64; u += blockDim.x) {
      const int r = u >> 6, p = u & 63;
      const int i = (p / half) * 2 * half + (p % half);
      const float a = v[r][i], b = v[r][i + half];
      v[r][i] = a + b;
      v[r][i + half] = a - b;
    }
    __syncthreads();
  }
}

struct WaveLds {
  uint32_t coef[16][kCoefStride];  // key-side B operand: [column][slot] packed fp16 pairs
  float pk[kHeadDim];              // 2^rho (K) per token
  float fv[kHeadDim];              // 2^rho s (V) * value scale, per token
  float zv[kHeadDim];              // 2^rho z (V) per token
  float gv[kHeadDim];              // 2^gamma (V) per channel
  float gs[kHeadDim];              // 2^gamma (V) / value scale, per channel
  float bq[kMaxGroup];             // b = sum_j q~_j 2^gamma_j z_j per query head
};

}  // namespace

__global__ __launch_bounds__(256, 2) void decode_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ k_pool, const uint8_t* __restrict__ v_pool,
    int num_pages, const int32_t* __restrict__ block_table, int max_blocks, const int32_t* __restrict__ seq_lens,
    int hq, int hkv, int blocks_per_split, int max_splits, float scale_log2, float* __restrict__ out,
    float* __restrict__ part, uint32_t* __restrict__ counters, uint32_t* __restrict__ flags) {
  __shared__ float qs[kMaxGroup][kHeadDim];
  __shared__ WaveLds wl[kWaves];
  __shared__ float wm[kWaves][kMaxGroup], wls[kWaves][kMaxGroup];
  __shared__ float wacc[kWaves][kMaxGroup][kHeadDim];
  __shared__ float mw[kMaxGroup][kMaxSplits];
  __shared__ int last_flag;

  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int G = hq / hkv;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, n = lane & 15, g = lane >> 4;
  const int hd = n & 7;
  const int lo_col = n >> 3;  // this lane's MFMA column carries the lo fp16 part
  const int sl = seq_lens[b];
  float* out_b = out + (static_cast<size_t>(b) * hq + static_cast<size_t>(kvh) * G) * kHeadDim;

  const bool bad = sl < 0 || (sl & (kBlockTokens - 1)) != 0 || sl > max_blocks * kBlockTokens;
  const int nblk = bad ? 0 : sl / kBlockTokens;
  if (nblk == 0) {
    if (split == 0) {
      if (bad && tid == 0 && flags) atomicOr(flags, kFlagBadSeqLen);
      for (int e = tid; e < G * kHeadDim; e += blockDim.x) out_b[e] = 0.f;
    }
    return;
  }
  const int nsplit = (nblk + blocks_per_split - 1) / blocks_per_split;
  if (split >= nsplit) return;
  const int blk0 = split * blocks_per_split;
  const int blk1 = min(nblk, blk0 + blocks_per_split);

  // ---- rotated, scaled query ------------------------------------------------
  const uint16_t* qb = q + (static_cast<size_t>(b) * hq + static_cast<size_t>(kvh) * G) * kHeadDim;
  for (int e = tid; e < kMaxGroup * kHeadDim; e += blockDim.x) {
    const int h = e >> 7, j = e & 127;
    qs[h][j] = h < G ? half_bits_to_float(qb[h * kHeadDim + j]) : 0.f;
  }
  __syncthreads();
  lds_fwht(qs, kMaxGroup);
  WaveLds& L = wl[w];
  // coefficient slot of this lane: channels ch0 = 32*(lane/16) + 8*((lane/4)%4) + lane%4 and ch0 + 4
  const int ch0 = 32 * (lane >> 4) + 8 * ((lane >> 2) & 3) + (lane & 3);
  const int ch1 = ch0 + 4;
  uint32_t kmag = 0x4C004C00u, vmag = 0x44004400u;  // fp16 16.0 / 4.0 pairs, kept in vector registers
  asm volatile("" : "+v"(kmag), "+v"(vmag));
  float q0[kMaxGroup], q1[kMaxGroup];
  float qmax = 0.f;
#pragma unroll
  for (int h = 0; h < kMaxGroup; ++h) {
    q0[h] = qs[h][ch0] * (kInvSqrt128 * scale_log2);
    q1[h] = qs[h][ch1] * (kInvSqrt128 * scale_log2);
    qmax = fmaxf(qmax, fmaxf(fabsf(q0[h]), fabsf(q1[h])));
  }
  qmax = wave_max(qmax);
  // unused coefficient columns stay zero
  for (int e = lane; e < 16 * kCoefStride; e += 64) (&L.coef[0][0])[e] = 0u;

  float m_run = -INFINITY, l_run = 0.f;
  float acc[8][4];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[mt][r] = 0.f;

  const int32_t* bt = block_table + static_cast<size_t>(b) * max_blocks;
  for (int blk = blk0 + w; blk < blk1; blk += kWaves) {
    const int page = bt[blk];
    if (page < 0 || page >= num_pages) {
      if (lane == 0 && flags) atomicOr(flags, kFlagBadPage);
      continue;
    }
    const uint8_t* kp = k_pool + (static_cast<size_t>(page) * hkv + kvh) * kKPageBytes;
    const uint8_t* vp = v_pool + (static_cast<size_t>(page) * hkv + kvh) * kVPageBytes;
    const uint8_t* km = kp + kKCodeBytes;
    const uint8_t* vm = vp + kVCodeBytes;

    // key codes: M-tile mt, row n -> token 32*(n/4) + 4*mt + n%4, channels 32g .. 32g+31
    u32x4 kc[8];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
      kc[mt] = *reinterpret_cast<const u32x4*>(kp + (32 * (n >> 2) + 4 * mt + (n & 3)) * 64 + 16 * g);
    // value codes: M-tile mt, row n -> channel 16mt + n, tokens 32g .. 32g+31
    u32x2 vc[8];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) vc[mt] = *reinterpret_cast<const u32x2*>(vp + (16 * mt + n) * 32 + 8 * g);
    // metadata
    const uint16_t* ksc = reinterpret_cast<const uint16_t*>(km + kMetaScale);
    const uint16_t* kzr = reinterpret_cast<const uint16_t*>(km + kMetaZero);
    const float* kgm = reinterpret_cast<const float*>(km + kMetaGamma);
    const float s0 = half_bits_to_float(ksc[ch0]), s1 = half_bits_to_float(ksc[ch1]);
    const float z0 = half_bits_to_float(kzr[ch0]), z1 = half_bits_to_float(kzr[ch1]);
    const float eg0 = ex2(kgm[ch0]), eg1 = ex2(kgm[ch1]);
    const float2 kr2 = reinterpret_cast<const float2*>(km + kMetaRho)[lane];
    const uint32_t vs2 = reinterpret_cast<const uint32_t*>(vm + kMetaScale)[lane];
    const uint32_t vz2 = reinterpret_cast<const uint32_t*>(vm + kMetaZero)[lane];
    const float2 vr2 = reinterpret_cast<const float2*>(vm + kMetaRho)[lane];
    const float2 vg2 = reinterpret_cast<const float2*>(vm + kMetaGamma)[lane];

    // ---- key-side coefficients (this lane: one slot, all heads) -------------
    const float e0 = eg0 * s0, e1 = eg1 * s1;
    const float emax = wave_max(fmaxf(e0, e1));
    int ex;
    frexpf(qmax * emax, &ex);
    ex = min(max(ex, -100), 100);
    const bool live = qmax * emax > 0.f;
    const float sa = live ? pow2i(14 - ex) : 1.f;        // |a * sa| < 2^14
    const float inv_sa = live ? pow2i(ex - 14) : 0.f;
    const float f0 = eg0 * z0, f1 = eg1 * z1;
    const float e0s = e0 * sa, e1s = e1 * sa;
    float bh[kMaxGroup];
#pragma unroll
    for (int h = 0; h < kMaxGroup; ++h) {
      if (h < G) {
        uint32_t hi, lo;
        split_pair(q0[h] * e0s, q1[h] * e1s, hi, lo);
        L.coef[h][lane] = hi;
        L.coef[8 + h][lane] = lo;
        const f16x2 hv = __builtin_bit_cast(f16x2, hi), lv = __builtin_bit_cast(f16x2, lo);
        const float asum = (static_cast<float>(hv[0]) + static_cast<float>(lv[0])) +
                           (static_cast<float>(hv[1]) + static_cast<float>(lv[1]));
        // b minus the 16-offset of the key codes, both per query head
        bh[h] = fmaf(-16.f * inv_sa, asum, fmaf(q0[h], f0, q1[h] * f1));
      } else {
        bh[h] = 0.f;
      }
    }
#pragma unroll
    for (int h = 0; h < kMaxGroup; ++h) {
      if (h < G) bh[h] = wave_sum(bh[h]);
      if (lane == h) L.bq[h] = bh[h];
    }

    // ---- per-token / per-channel factors (this lane: entries 2*lane, 2*lane+1)
    const float pr0 = ex2(kr2.x), pr1 = ex2(kr2.y);
    const float vr0 = ex2(vr2.x), vr1 = ex2(vr2.y);
    const float F0 = vr0 * half_bits_to_float(vs2 & 0xFFFFu), F1 = vr1 * half_bits_to_float(vs2 >> 16);
    const float fmaxv = wave_max(fmaxf(F0, F1));
    int exf;
    frexpf(fmaxv, &exf);
    exf = min(max(exf, -100), 100);
    const bool livef = fmaxv > 0.f;
    const float sw = livef ? pow2i(14 - exf) : 1.f;       // p <= 1, so |w * sw| < 2^14
    const float inv_sw = livef ? pow2i(exf - 14) : 0.f;
    const int t0 = 2 * lane;
    L.pk[t0] = pr0;
    L.pk[t0 + 1] = pr1;
    L.fv[t0] = F0 * sw;
    L.fv[t0 + 1] = F1 * sw;
    L.zv[t0] = vr0 * half_bits_to_float(vz2 & 0xFFFFu);
    L.zv[t0 + 1] = vr1 * half_bits_to_float(vz2 >> 16);
    const float gv0 = ex2(vg2.x), gv1 = ex2(vg2.y);
    L.gv[t0] = gv0;
    L.gv[t0 + 1] = gv1;
    L.gs[t0] = gv0 * inv_sw;
    L.gs[t0 + 1] = gv1 * inv_sw;
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    const float bmine = L.bq[hd];

    // ---- key side: scores ---------------------------------------------------
    f16x8 cb[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      cb[ks] = __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4*>(&L.coef[n][16 * g + 4 * ks]));
    float s[8][4];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) d = mfma16x16x32(key_codes(kc[mt][ks], kmag), cb[ks], d);
#pragma unroll
      for (int r = 0; r < 4; ++r) s[mt][r] = d[r] + dpp<kDppXor8>(d[r]);
    }
    // this lane keeps tokens 32g + 16*lo_col + 4mt' + r (mt' = 0..3)
    float sm[4][4];
    float mloc = -INFINITY;
    const float* pkp = &L.pk[32 * g + 16 * lo_col];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const float4 pk4 = *reinterpret_cast<const float4*>(pkp + 4 * mt);
      const float pkv[4] = {pk4.x, pk4.y, pk4.z, pk4.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float sv = sel_lo(s[mt][r], s[mt + 4][r]);
        sm[mt][r] = pkv[r] * fmaf(sv, inv_sa, bmine);
        mloc = fmaxf(mloc, sm[mt][r]);
      }
    }
    mloc = head_max(mloc);
    const float m_new = fmaxf(m_run, mloc);
    const float alpha = ex2(m_run - m_new);
    m_run = m_new;

    // ---- softmax weights, value-side B operand -------------------------------
    const float* fvp = &L.fv[32 * g + 16 * lo_col];
    const float* zvp = &L.zv[32 * g + 16 * lo_col];
    float lsum = 0.f, usum = 0.f, wsum = 0.f;
    float wv[4][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const float4 f4 = *reinterpret_cast<const float4*>(fvp + 4 * mt);
      const float4 z4 = *reinterpret_cast<const float4*>(zvp + 4 * mt);
      const float fvv[4] = {f4.x, f4.y, f4.z, f4.w};
      const float zvv[4] = {z4.x, z4.y, z4.z, z4.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = ex2(sm[mt][r] - m_new);
        lsum += p;
        usum = fmaf(p, zvv[r], usum);
        wv[mt][r] = p * fvv[r];
        wsum += wv[mt][r];
      }
    }
    lsum = head_sum(lsum);
    // u minus the 4-offset of the value codes (w is carried with the page scale sw)
    usum = fmaf(-4.f * inv_sw, head_sum(wsum), head_sum(usum));
    l_run = fmaf(l_run, alpha, lsum);
    // pair (hf, j) = tokens 4hf + j and 4hf + j + 8 of this lane's 16
    uint32_t own_hi[2][4], own_lo[2][4];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int j = 0; j < 4; ++j) split_pair(wv[hf][j], wv[hf + 2][j], own_hi[hf][j], own_lo[hf][j]);
    f16x8 wb[2][2];  // [u][hf]
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      u32x4 mine, other;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        mine[j] = sel_lo_u32(own_hi[hf][j], own_lo[hf][j]);
        other[j] = dpp_u32_xor8(sel_lo_u32(own_lo[hf][j], own_hi[hf][j]));
      }
      u32x4 u0, u1;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u0[j] = sel_lo_u32(mine[j], other[j]);
        u1[j] = sel_lo_u32(other[j], mine[j]);
      }
      wb[0][hf] = __builtin_bit_cast(f16x8, u0);
      wb[1][hf] = __builtin_bit_cast(f16x8, u1);
    }
    const float ulane = sel_lo(usum, 0.f);

    // ---- value side: o (rotated basis), hi and lo columns kept apart ----------
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) d = mfma16x16x32(value_codes(vc[mt][u], hf, vmag), wb[u][hf], d);
      const float4 gs4 = *reinterpret_cast<const float4*>(&L.gs[16 * mt + 4 * g]);
      const float4 gv4 = *reinterpret_cast<const float4*>(&L.gv[16 * mt + 4 * g]);
      const float gsv[4] = {gs4.x, gs4.y, gs4.z, gs4.w};
      const float gvv[4] = {gv4.x, gv4.y, gv4.z, gv4.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[mt][r] = fmaf(acc[mt][r], alpha, fmaf(d[r], gsv[r], ulane * gvv[r]));
    }
  }

  // ---- merge the four waves through LDS --------------------------------------
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[mt][r] += dpp<kDppXor8>(acc[mt][r]);
  if (!lo_col && hd < G) {
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) wacc[w][hd][16 * mt + 4 * g + r] = acc[mt][r];
    if (g == 0) {
      wm[w][hd] = m_run;
      wls[w][hd] = l_run;
    }
  }
  __syncthreads();
  const size_t pair = static_cast<size_t>(b) * hkv + kvh;
  float* pbase = part + pair * max_splits * kMaxGroup * kPartStride;
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
    pp[j] = o;
    if (j == 0) {
      pp[kHeadDim] = mx;
      pp[kHeadDim + 1] = lsum;
    }
  }
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(counters + pair, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    last_flag = (prev == static_cast<uint32_t>(nsplit - 1));
  }
  __syncthreads();
  if (!last_flag) return;
  __threadfence();
  if (tid == 0) counters[pair] = 0u;  // leave the counter ready for the next call

  // ---- merge the splits (log-sum-exp) and undo the rotation ---------------
  for (int e = tid; e < G * kMaxSplits; e += blockDim.x) {
    const int h = e / kMaxSplits, sp = e % kMaxSplits;
    mw[h][sp] = sp < nsplit ? pbase[(static_cast<size_t>(sp) * kMaxGroup + h) * kPartStride + kHeadDim] : -INFINITY;
  }
  __syncthreads();
  for (int e = tid; e < G * kHeadDim; e += blockDim.x) {
    const int h = e >> 7, j = e & 127;
    float mx = -INFINITY;
    for (int sp = 0; sp < nsplit; ++sp) mx = fmaxf(mx, mw[h][sp]);
    float num = 0.f, den = 0.f;
    for (int sp = 0; sp < nsplit; ++sp) {
      const float ms = mw[h][sp];
      const float wgt = ms == -INFINITY ? 0.f : ex2(ms - mx);
      const float* pp = pbase + (static_cast<size_t>(sp) * kMaxGroup + h) * kPartStride;
      num = fmaf(wgt, pp[j], num);
      den = fmaf(wgt, pp[kHeadDim + 1], den);
    }
    qs[h][j] = den > 0.f ? num / den : 0.f;
  }
  __syncthreads();
  lds_fwht(qs, G);
  for (int e = tid; e < G * kHeadDim; e += blockDim.x) out_b[e] = qs[e >> 7][e & 127] * kInvSqrt128;
}

hipError_t launch_decode(const void* q, const void* k_pool, const void* v_pool, int num_pages,
                         const int32_t* block_table, int max_blocks, const int32_t* seq_lens, int batch, int hq,
                         int hkv, int blocks_per_split, int max_splits, float scale_log2, float* out, float* part,
                         uint32_t* counters, uint32_t* flags, hipStream_t stream) {
  hipLaunchKernelGGL(decode_kernel, dim3(max_splits, hkv, batch), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint8_t*>(k_pool),
                     static_cast<const uint8_t*>(v_pool), num_pages, block_table, max_blocks, seq_lens, hq, hkv,
                     blocks_per_split, max_splits, scale_log2, out, part, counters, flags);
  return hipGetLastError();
}

}  // namespace kvarn
