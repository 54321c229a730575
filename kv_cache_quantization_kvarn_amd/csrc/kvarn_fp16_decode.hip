// FP16 paged decode attention for gfx950: the uncompressed baseline that the packed KVarN cache is
// measured against (KVarN blog post, section "KVarN (Varyans Normalize Edilmiş KV-Cache) Nedir?":
// the packed cache is compared with FP16 serving).  Same harness as the packed decode: the same
// split plan, workspace, partials and merge, and the same paged addressing (KV Cache glossary page,
// section "KV Cache'in Çalışma Mekanizması ve Türleri": block table, grouped query heads).
//
// Page layout: fp16 K and V pools [num_pages][Hkv][128 tokens][128 channels], 32 KiB per (page,
// KV head) each -- 65,536 B per block per KV head against 15,360 B packed.
//
// A workgroup of four waves handles the G <= 8 query heads of one KV head over a run of pages,
// wave w taking every fourth page.  Both contractions of a page run on v_mfma_f32_16x16x32_f16:
//
//   scores  D[token][head]  = K rows (A operand, straight 16 B loads) x q (B operand, exact fp16)
//   output  D[head][channel] = p (A operand) x V (B operand)
//
// The B operand of the second product needs eight tokens of one channel per lane, while a page
// row holds the channels of one token.  The transpose is a product with a 0/1 selection matrix:
// V rows times the columns of the identity that pick 16 of a row's 32 channels give, in the
// MFMA output layout, exactly the eight token slots at which the score layout already holds the
// softmax weights p.  The weights enter as fp16 hi (rows 0-7) plus lo (rows 8-15) so that their
// fp32 accuracy survives; the two row halves are added at the end.
#include "kvarn_common.h"

namespace kvarn {

namespace {

constexpr int kWavesF16 = 4;
constexpr int kPartStrideF16 = kHeadDim + 2;  // o[128], m, l per (split, query head)
constexpr int kHalfsPerPage = kBlockTokens * kHeadDim;

// Max / sum over the four 16-lane rows (lanes l, l^16, l^32, l^48); identical bits in every lane.
__device__ __forceinline__ float rows_max4(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows_sum4(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ float wave_max64(float x) { return rows_max4(row16_max(x)); }
__device__ __forceinline__ float wave_sum64(float x) { return rows_sum4(row16_sum(x)); }

// Split partials cross XCDs: agent-scope relaxed accesses go through to the device-coherent level.
__device__ __forceinline__ void store_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_agent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float ex2f(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ f16x8 load16(const uint16_t* p) { return *reinterpret_cast<const f16x8*>(p); }

// fp32 -> fp16 pairs (round to nearest even), packed for an MFMA operand.
__device__ __forceinline__ f16x8 pack8(const float (&v)[8]) {
  f16x8 r;
#pragma unroll
  for (int s = 0; s < 8; ++s) r[s] = static_cast<_Float16>(v[s]);
  return r;
}

}  // namespace

__global__ __launch_bounds__(256, 3) void fp16_decode_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache, const uint16_t* __restrict__ v_cache,
    int num_pages, const int32_t* __restrict__ block_table, int max_blocks, const int32_t* __restrict__ seq_lens,
    int hq, int hkv, int blocks_per_split, int max_splits, float scale_log2, float* __restrict__ out,
    float* __restrict__ part, uint32_t* __restrict__ counters, uint32_t* __restrict__ flags) {
  __shared__ __align__(16) float wacc[kWavesF16][kMaxGroup][kHeadDim];  // per-wave o
  __shared__ __align__(16) float alpha_l[kWavesF16][kMaxGroup];          // per-wave rescale of each head
  __shared__ float wm[kWavesF16][kMaxGroup], wls[kWavesF16][kMaxGroup];
  __shared__ int last_flag;

  // KV head fastest in dispatch order (workgroups go to the XCDs round-robin): every XCD gets an
  // equal share of each sequence; split positions vary slowest, so empty splits come last.
  const int kvh = blockIdx.x, b = blockIdx.y, split = blockIdx.z;
  const int G = hq / hkv;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, n = lane & 15, g = lane >> 4;
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
  const int cnt = min(nblk, blk0 + blocks_per_split) - blk0;
  const int32_t* bt = block_table + static_cast<size_t>(b) * max_blocks + blk0;
  const int wu = __builtin_amdgcn_readfirstlane(w);

  // ---- operands that stay: q (B operand of the scores) and the selection matrices ----
  // qb[cg]: lane (head n, g) holds q[n][32cg + 8g .. +7] (zero for heads past G)
  const uint16_t* qrow = q + (static_cast<size_t>(b) * hq + static_cast<size_t>(kvh) * G + (n < G ? n : 0)) * kHeadDim;
  f16x8 qb[4];
#pragma unroll
  for (int cg = 0; cg < 4; ++cg) {
    const f16x8 v = load16(qrow + 32 * cg + 8 * g);
    const f16x8 zero = {};
    qb[cg] = n < G ? v : zero;
  }
  // sel[h2]: B[k][col] = 1 where k = 16*h2 + col, so that (V rows) x sel[h2] picks channels
  // 16*h2 .. 16*h2 + 15 of a 32-channel group
  f16x8 sel[2];
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
    for (int s = 0; s < 8; ++s)
      sel[h2][s] = (8 * g + s == 16 * h2 + n) ? static_cast<_Float16>(1.0f) : static_cast<_Float16>(0.0f);

  // ---- per-wave online softmax state -----------------------------------------
  // m_run, l_run: head n (lanes n < 8; the same in the four lanes of one n);
  // acc[ct]: output channel tile ct (16 channels), lane (channel j, g) rows 4g .. 4g+3 of
  //          [hi heads 0-7 | lo heads 0-7]
  float m_run = -INFINITY, l_run = 0.f;
  f32x4 acc[8];
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};

  bool bad_page = false;
  for (int i = wu; i < cnt; i += kWavesF16) {
    const int page = bt[i];
    if (page < 0 || page >= num_pages) {
      bad_page = true;
      continue;
    }
    const size_t base = (static_cast<size_t>(page) * hkv + kvh) * kHalfsPerPage;
    const uint16_t* kp = k_cache + base;
    const uint16_t* vp = v_cache + base;

    // ---- scores: s[mt][r] = score of token 16mt + 4g + r for head n (log2 units) ----
    f32x4 s[8];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int cg = 0; cg < 4; ++cg) d = mfma16x16x32(load16(kp + (16 * mt + n) * kHeadDim + 32 * cg + 8 * g), qb[cg], d);
#pragma unroll
      for (int r = 0; r < 4; ++r) s[mt][r] = d[r] * scale_log2;
    }
    float mloc = s[0][0];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) mloc = fmaxf(mloc, s[mt][r]);
    mloc = rows_max4(mloc);
    const float m_new = fmaxf(m_run, mloc);
    const float alpha = ex2f(m_run - m_new);  // 0 on the first page
    float lsum = 0.f;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        s[mt][r] = ex2f(s[mt][r] - m_new);
        lsum += s[mt][r];
      }
    l_run = fmaf(alpha, l_run, rows_sum4(lsum));
    m_run = m_new;
    // rescale o: row 4g + r of a lane holds head (4g + r) & 7, whose factor lives in lane n = head
    if (g == 0 && n < kMaxGroup) alpha_l[w][n] = alpha;
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    {
      const float4 a = *reinterpret_cast<const float4*>(&alpha_l[w][4 * (g & 1)]);
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) {
        acc[ct][0] *= a.x;
        acc[ct][1] *= a.y;
        acc[ct][2] *= a.z;
        acc[ct][3] *= a.w;
      }
    }

    // ---- output: 32 tokens (tiles 2c, 2c+1) at a time ---------------------------
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      // A operand: slot k of lane (n, g) is token 16*(2c + k/4) + 4g + k%4; rows 0-7 take p in
      // fp16, rows 8-15 the fp16 remainder p - hi of head n - 8 (from lane n ^ 8)
      float pv[8], lov[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) pv[k] = s[2 * c + (k >> 2)][k & 3];
      const f16x8 hi = pack8(pv);
#pragma unroll
      for (int k = 0; k < 8; ++k) lov[k] = pv[k] - static_cast<float>(hi[k]);
      const f16x8 lo = pack8(lov);
      f16x8 ap;
      {
        const u32x4 lo_u = __builtin_bit_cast(u32x4, lo), hi_u = __builtin_bit_cast(u32x4, hi);
        u32x4 r;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const uint32_t from8 = static_cast<uint32_t>(
              __builtin_amdgcn_mov_dpp(static_cast<int>(lo_u[x]), kDppXor8, 0xF, 0xF, true));
          r[x] = n < 8 ? hi_u[x] : from8;
        }
        ap = __builtin_bit_cast(f16x8, r);
      }
#pragma unroll
      for (int cg = 0; cg < 4; ++cg) {
        const f16x8 v0 = load16(vp + (16 * (2 * c) + n) * kHeadDim + 32 * cg + 8 * g);
        const f16x8 v1 = load16(vp + (16 * (2 * c + 1) + n) * kHeadDim + 32 * cg + 8 * g);
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          // lane (channel j, g): t0[r] = V[32c + 4g + r][32cg + 16h2 + j], t1 the same 16 tokens on
          const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
          const f32x4 t0 = mfma16x16x32(v0, sel[h2], zero);
          const f32x4 t1 = mfma16x16x32(v1, sel[h2], zero);
          const float bv[8] = {t0[0], t0[1], t0[2], t0[3], t1[0], t1[1], t1[2], t1[3]};
          const int ct = 2 * cg + h2;
          acc[ct] = mfma16x16x32(ap, pack8(bv), acc[ct]);
        }
      }
    }
  }
  if (bad_page && lane == 0 && flags) atomicOr(flags, kFlagBadPage);

  // ---- hi + lo rows, then merge the four waves through LDS --------------------
  // after the swap, lanes g < 2 hold o of heads 4g + r (rows 0-7) for channel 16ct + n
#pragma unroll
  for (int ct = 0; ct < 8; ++ct)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[ct][r]), __float_as_uint(acc[ct][r]), false, false);
      acc[ct][r] = __uint_as_float(x[0]) + __uint_as_float(x[1]);
    }
  if (g < 2) {
#pragma unroll
    for (int ct = 0; ct < 8; ++ct)
#pragma unroll
      for (int r = 0; r < 4; ++r) wacc[w][4 * g + r][16 * ct + n] = acc[ct][r];
  }
  if (g == 0 && n < kMaxGroup) {
    wm[w][n] = m_run;
    wls[w][n] = l_run;
  }
  __syncthreads();
  const size_t pair = static_cast<size_t>(b) * hkv + kvh;
  float* pbase = part + pair * max_splits * kMaxGroup * kPartStrideF16;
  for (int e = tid; e < G * kHeadDim; e += blockDim.x) {
    const int h = e >> 7, j = e & 127;
    float mx = -INFINITY;
#pragma unroll
    for (int x = 0; x < kWavesF16; ++x) mx = fmaxf(mx, wm[x][h]);
    float o = 0.f, lsum = 0.f;
#pragma unroll
    for (int x = 0; x < kWavesF16; ++x) {
      const float wgt = wm[x][h] == -INFINITY ? 0.f : ex2f(wm[x][h] - mx);
      o = fmaf(wgt, wacc[x][h][j], o);
      lsum = fmaf(wgt, wls[x][h], lsum);
    }
    float* pp = pbase + (static_cast<size_t>(split) * kMaxGroup + h) * kPartStrideF16;
    store_agent(pp + j, o);
    if (j == 0) {
      store_agent(pp + kHeadDim, mx);
      store_agent(pp + kHeadDim + 1, lsum);
    }
  }
  // The stores are acknowledged before the workgroup counts itself in (no fence: an agent-scope
  // fence would write back or invalidate this XCD's whole L2).
  // Fence-free hand-off, as in the packed decode: agent-scope (sc1) partial stores, vmcnt(0) covering
  // them, then the agent-scope counter add; every access to partials and counters is one of these.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(counters + pair, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last_flag = (prev == static_cast<uint32_t>(nsplit - 1));
  }
  __syncthreads();
  if (!last_flag) return;
  if (tid == 0) __hip_atomic_store(counters + pair, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // ready for the next call

  // ---- merge the splits (log-sum-exp) -------------------------------------------
  // Wave w takes heads w and w + 4; lane l holds channels 2l and 2l + 1, lane s the maximum and sum
  // of split s (nsplit <= 64).
  for (int h = w; h < G; h += kWavesF16) {
    constexpr size_t kSplitStride = static_cast<size_t>(kMaxGroup) * kPartStrideF16;
    const float* ph = pbase + static_cast<size_t>(h) * kPartStrideF16;
    const int sp = lane < nsplit ? lane : 0;
    const float ms = load_agent(ph + sp * kSplitStride + kHeadDim);
    const float ls = load_agent(ph + sp * kSplitStride + kHeadDim + 1);
    const float msv = lane < nsplit ? ms : -INFINITY;
    const float mx = wave_max64(msv);
    const float wgt = msv == -INFINITY ? 0.f : ex2f(msv - mx);
    const float den = wave_sum64(wgt * (lane < nsplit ? ls : 0.f));
    float n0 = 0.f, n1 = 0.f;
    for (int s0 = 0; s0 < nsplit; s0 += 8) {
      float2 o[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float* pp = ph + (s0 + k < nsplit ? s0 + k : 0) * kSplitStride + 2 * lane;
        o[k] = make_float2(load_agent(pp), load_agent(pp + 1));
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
    reinterpret_cast<float2*>(out_b + static_cast<size_t>(h) * kHeadDim)[lane] = make_float2(n0 * inv, n1 * inv);
  }
}

hipError_t launch_fp16_decode(const void* q, const void* k_cache, const void* v_cache, int num_pages,
                              const int32_t* block_table, int max_blocks, const int32_t* seq_lens, int batch, int hq,
                              int hkv, int blocks_per_split, int max_splits, float scale_log2, float* out, float* part,
                              uint32_t* counters, uint32_t* flags, hipStream_t stream) {
  hipLaunchKernelGGL(fp16_decode_kernel, dim3(hkv, batch, max_splits), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_cache),
                     static_cast<const uint16_t*>(v_cache), num_pages, block_table, max_blocks, seq_lens, hq, hkv,
                     blocks_per_split, max_splits, scale_log2, out, part, counters, flags);
  return hipGetLastError();
}

}  // namespace kvarn
