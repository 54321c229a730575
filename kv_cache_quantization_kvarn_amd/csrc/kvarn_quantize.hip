// KVarN block quantisation kernel for gfx950.
//
// A workgroup (4 waves) quantises one tile at a time: a 128-token x 128-channel fp16
// block of one KV head of K or V (KVarN blog post, section "KVarN Nasıl
// Çalışır?"): Hadamard rotation along channels, four row/column passes of
// log2-variance normalisation, per-group min/max, round to nearest, packing.
//
// Data distribution.  Wave w owns tokens [32w, 32w+32).  The rotation runs
// entirely on the matrix cores: the 128-point Hadamard factors as H4 (x) H32
// over channel-index bits (5-6) and (0-4), so each output tile is a chain of
// four v_mfma_f32_16x16x32_f16 products of the wave's fp16 tokens with the
// exact +-1 H32 block, each input chunk entering with the sign of the H4 entry
// (fp32 accumulation; the products are exact).  The rotation is left
// unnormalised (R' = sqrt(128) R); the factor 2^-3.5 rides in the row
// normaliser 2^-rho instead, which leaves every normalised value unchanged.
// The MFMA result layout fixes what each lane holds: lane (n = lane%16,
// g = lane/16) keeps 8 tokens x 8 channels,
//     token   T(i) = 32w + 16*(i/4) + 4g + i%4          i = 0..7
//     channel C(c) = 32*(c/2) + 2n + c%2                c = 0..7
// so a lane holds channel pairs (2k, 2k+1), the two nibbles of one key byte.
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
//
// Codes.  The normaliser of the group axis is folded into the rounding FMA
// (u = M * (2^-x / s) - z / s with M the value scaled by the other normaliser),
// codes are packed in registers (two nibbles or four 2-bit codes per byte; one
// byte per 8-bit key code, two 4-bit value codes per byte in the wider
// formats), transposed across lanes into whole dwords of the page (DPP within a
// quad or a lane pair for keys, v_permlane16/32_swap across rows for values)
// and stored directly.  The code widths and the group size are template
// parameters; every other step is shared.  With group size 64 a key group is one
// channel over a token half and a value group one token over a channel half: the
// two threads of a min/max reducer pair then keep their own half (waves 0-1 vs
// 2-3 for keys; a lane's channels c = 0-3 vs 4-7 for values) instead of merging.
//
// Scheduling.  Workgroups are persistent, two per compute unit; each walks its share of the key
// tiles and then of the value tiles with a fixed stride.  The input of the next tile is fetched while the current
// one is normalised, across the switch from keys to values too; the page stores go through a buffer resource (size zero for an invalid page)
// so that every tile issues the same memory operations and the wait for the prefetched input
// never has to drain the stores.
#include "kvarn_common.h"

namespace kvarn {

namespace {

__device__ __forceinline__ int tok_of(int w, int g, int i) { return 32 * w + 16 * (i >> 2) + 4 * g + (i & 3); }
__device__ __forceinline__ int chan_of(int n, int c) { return 32 * (c >> 1) + 2 * n + (c & 1); }
// position of channel ch in the per-lane-contiguous order used for per-channel LDS arrays
// (lane n reads slots 8n .. 8n+7, slot 8n + c holding channel chan_of(n, c))
__device__ __forceinline__ int chan_slot(int ch) { return 8 * ((ch >> 1) & 15) + 2 * (ch >> 5) + (ch & 1); }

// Partial sums, 16 slots of two floats per row (token or channel), kept as two half arrays: slots
// 0-7 in half 0, 8-15 in half 1, rows kSlotStride floats apart, half 1 starting 32 floats further
// (modulo the 64 four-byte LDS banks) than a whole number of bank rows after half 0.  Both access
// patterns are then conflict-free: the reducers of 8 consecutive rows (one half each) read 16-byte
// chunks that cover all 64 banks once (row starts 20 floats apart, the halves 32 apart), and the 16
// lanes of a token-indexed write (one row, slots n) cover 32 banks, the rows 4 further the other 32.
constexpr int kSlotStride = 20;
constexpr int kHalfOffset = kBlockTokens * kSlotStride + 32;
struct PartRows {
  float f[kHalfOffset + kBlockTokens * kSlotStride];
  __device__ float* slot(int row, int sl) { return f + (sl >> 3) * kHalfOffset + row * kSlotStride + 2 * (sl & 7); }
  __device__ float* half(int row, int hf) { return f + hf * kHalfOffset + row * kSlotStride; }
};

// Slot of lane (w, g, n) in a channel's row of column partials.  The 16 lanes of a row write channels
// 2n (+ 32k) apart, i.e. rows 40 floats apart (8 banks modulo 64), which would put lanes n and n + 8
// on the same banks; the XOR with n / 4 moves them apart and keeps each slot in its half (slots 0-7:
// waves 0-1, 8-15: waves 2-3), which the group-size-64 reducers read separately.
__device__ __forceinline__ int col_slot(int w, int g, int n) { return (4 * w + g) ^ (n >> 2); }

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float lg2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ float dpp_xor1(float x) { return dpp<kDppXor1>(x); }

__device__ __forceinline__ uint32_t dpp_u32(uint32_t x, int ctrl_xor2) {
  return ctrl_xor2 ? static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(x), kDppXor2, 0xF, 0xF, true))
                   : static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(x), kDppXor1, 0xF, 0xF, true));
}

// Sum of the 8 (s1, s2) slot pairs of one row half (hf), then with the partner thread (lane ^ 1).
__device__ __forceinline__ float2 reduce_pairs(const float* half_row, int hf) {
  const float4* p = reinterpret_cast<const float4*>(half_row);
  float a = p[0].x, b = p[0].y;
  a += p[0].z;
  b += p[0].w;
#pragma unroll
  for (int k = 1; k < 4; ++k) {
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

// Minimum and maximum of partials read back from LDS (or across lanes), as the instructions
// themselves: the compiler would otherwise quiet every operand first, since it cannot tell that
// a value loaded from memory is not a signalling NaN (these are all results of arithmetic).
__device__ __forceinline__ float min3_raw(float a, float b, float c) {
  float r;
  asm("v_min3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float max3_raw(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float min_raw(float a, float b) {
  float r;
  asm("v_min_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float max_raw(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// Orders LDS accesses between lanes of one wave (LDS operations of a wave complete in order).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Rounded product that the compiler may not fuse into a later add: the group range is a
// difference of two such products, and contracting one of them into an FMA would turn an
// exactly constant group (max == min) into a range of one rounding error, of either sign.
__device__ __forceinline__ float mul_rn(float a, float b) {
  float p = a * b;
  asm("" : "+v"(p));
  return p;
}

// 4x4 byte transpose inside each quad of lanes (DPP): lane j holds bytes B[j][0..3] and
// receives B[0..3][j].
__device__ __forceinline__ uint32_t quad_transpose(uint32_t v, int j) {
  const uint32_t p = dpp_u32(v, 1);                                              // lane j ^ 2
  const uint32_t t = __builtin_amdgcn_perm(p, v, (j & 2) ? 0x03020706u : 0x05040100u);
  const uint32_t q = dpp_u32(t, 0);                                              // lane j ^ 1
  return __builtin_amdgcn_perm(q, t, (j & 1) ? 0x03070105u : 0x06020400u);
}

// The same transpose across the four 16-lane rows (row r holds B[r][0..3], receives B[0..3][r]).
// v_permlane32_swap on two copies of v returns (value of row r & 1, value of row r | 2) in that
// order; v_permlane16_swap returns (value of row r & ~1, value of row r | 1).
__device__ __forceinline__ uint32_t row_transpose(uint32_t v, int r) {
  const auto a = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  const uint32_t t = __builtin_amdgcn_perm(a[1], a[0], (r & 2) ? 0x07060302u : 0x05040100u);
  const auto b = __builtin_amdgcn_permlane16_swap(t, t, false, false);
  return __builtin_amdgcn_perm(b[1], b[0], (r & 1) ? 0x07030501u : 0x06020400u);
}


// Shared memory of one quantising workgroup.  Row partials (indexed by token) are written and
// read only by the wave that owns the token; column partials (indexed by channel) are written by
// every wave.  Separate arrays let a wave run its next row pass while others still reduce a
// column pass.
struct QuantLds {
  PartRows part_row;  // per token: 16 partial pairs
  PartRows part;      // per channel (column passes, key min/max) or per token (value min/max)
  float rfl[kBlockTokens], rfl2[kBlockTokens];  // 2^-rho / sqrt(128) and its square, token order
  float cfl[kHeadDim], cfl2[kHeadDim];          // 2^-gamma and its square, chan_slot order
  float mul_a[2][kHeadDim], mul_b[2][kHeadDim];  // rounding FMA of each group (by half for group size 64)
  float mul_c[kHeadDim];                      // column means for the centred fallback
  float mul_r[kBlockTokens];                  // row means for the centred fallback
  int recenter[2];                            // column-pass fallback flag, by parity
};

// Stores into a page go through a buffer resource.  An invalid destination page gets a resource
// of size zero, so the hardware drops its stores and every tile issues the same memory
// operations (the prefetch of the next tile then needs no conservative wait).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t page_resource(uint8_t* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, 0, bytes, 0x00020000);
}

// fp16 input of tile `tile` (block tile / hkv, head tile % hkv) in the MFMA A-operand layout:
// xa[mt][gi] = X[32w + 16mt + n][32gi + 8g .. +7].
__device__ __forceinline__ void load_tile(f16x8 (&xa)[2][4], const uint16_t* __restrict__ in, int tile, int hkv,
                                          int w, int n, int g) {
  const int blk = tile / hkv;
  const int head = tile - blk * hkv;
  const size_t tstride = static_cast<size_t>(hkv) * kHeadDim;
  const uint16_t* src = in + (static_cast<size_t>(blk) * kBlockTokens * hkv + head) * kHeadDim;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int gi = 0; gi < 4; ++gi)
      xa[mt][gi] = *reinterpret_cast<const f16x8*>(src + static_cast<size_t>(32 * w + 16 * mt + n) * tstride +
                                                    32 * gi + 8 * g);
}

// R' = X H for the wave's 32 tokens (unnormalised): output chunk h4 of each 16-token tile is the
// sum over input chunks gi of H4[gi][h4] * (X_gi H32), with H4's -1 entries taken by hbn = -hb.
// Also the first row pass's moments, straight from the fp16 input: with every column normaliser 1,
// sum_j R'_tj = 128 x_t0 (only input channel 0 meets a row of H made of ones) and sum_j R'_tj^2 =
// 128 sum_k x_tk^2 (the +-1 matrix times its transpose is 128 I).  m1[mt], m2[mt] belong to token
// 32w + 16 mt + n and are the same in the four lanes of each column n.
__device__ __forceinline__ void rotate(const f16x8 (&xa)[2][4], const f16x8 (&hb)[2], const f16x8 (&hbn)[2],
                                       float (&R)[8][8], float (&P)[8][8], float (&m1)[2], float (&m2)[2], int g) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    float q = 0.f;
#pragma unroll
    for (int gi = 0; gi < 4; ++gi)
#pragma unroll
      for (int i = 0; i < 8; i += 2) {
        const h2 x = {xa[mt][gi][i], xa[mt][gi][i + 1]};
        q = __builtin_amdgcn_fdot2(x, x, q, false);
      }
    m2[mt] = 128.f * rows4_sum(q);
    m1[mt] = 128.f * rows4_sum(g == 0 ? static_cast<float>(xa[mt][0][0]) : 0.f);
  }
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
      for (int h4 = 0; h4 < 4; ++h4) {
        f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) d = mfma16x16x32(xa[mt][gi], (__popc(gi & h4) & 1) ? hbn[hh] : hb[hh], d);
#pragma unroll
        for (int r = 0; r < 4; ++r) R[4 * mt + r][2 * h4 + hh] = d[r];
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int c = 0; c < 8; ++c) P[i][c] = R[i][c] * R[i][c];
}

// All tiles of one kind (keys or values) owned by this workgroup: tiles blockIdx.x,
// blockIdx.x + gridDim.x, ...  The next tile's input is loaded while the current one is
// normalised and packed.  One pipeline runs through both kinds: the key pass starts it, and its
// last prefetches fetch the workgroup's first value tiles (from vin), so the value pass begins with
// its first tile rotated (R, P, m1, m2) and its second in flight (xa).
template <bool kIsV, int kBits, int kGroup>
__device__ __forceinline__ void quantize_tiles(const uint16_t* __restrict__ in, const uint16_t* __restrict__ vin,
                                               int hkv, int tiles, const int32_t* __restrict__ dst_pages,
                                               uint8_t* __restrict__ pool, int num_pages,
                                               uint32_t* __restrict__ flags, QuantLds& s, f16x8 (&xa)[2][4],
                                               float (&R)[8][8], float (&P)[8][8], float (&m1)[2], float (&m2)[2]) {
  static_assert(kIsV ? (kBits == 2 || kBits == 4) : (kBits == 4 || kBits == 8), "code width");
  using Meta = MetaLayout<kGroup>;
  constexpr bool kHalf = kGroup == 64;  // two groups per channel (keys) or token (values)
  constexpr int kCodeBytes = kBlockTokens * kHeadDim * kBits / 8;
  constexpr int kPageBytes = kCodeBytes + Meta::kBytes;
  constexpr float kLevels = static_cast<float>((1 << kBits) - 1);
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, n = lane & 15, g = lane >> 4;
  // Reducer role of this thread: row t_red (row passes) / channel c_red (column passes) = t_red;
  // the two threads of a pair (hf = 0, 1) compute identical values.
  const int t_red = tid >> 1, hf = tid & 1;
  constexpr float inv128 = 1.0f / 128.0f;

  // H32 block: B[k][col] = (-1)^popcount(k & o), input index k = 8g + i, output o = 2n + hh;
  // hbn = -hb for the H4 entries that are -1
  f16x8 hb[2], hbn[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bool neg = __popc((8 * g + i) & (2 * n + hh)) & 1;
      hb[hh][i] = neg ? static_cast<_Float16>(-1.0f) : static_cast<_Float16>(1.0f);
      hbn[hh][i] = neg ? static_cast<_Float16>(1.0f) : static_cast<_Float16>(-1.0f);
    }

  if (tid == 0) {
    s.recenter[0] = 0;
    s.recenter[1] = 0;
  }
  bool bad = false;
  const int stride = static_cast<int>(gridDim.x);
  const int first = static_cast<int>(blockIdx.x);
  int tile = first;
  // software pipeline: the loop body packs tile `tile`, then rotates the next tile (whose input
  // arrived meanwhile) and fetches the one after it; the workgroup's tiles run keys first, then
  // values, and past the last value tile the last one stands in
  if constexpr (!kIsV) {
    load_tile(xa, in, tile, hkv, w, n, g);
    rotate(xa, hb, hbn, R, P, m1, m2, g);
    const bool more = tile + stride < tiles;
    load_tile(xa, more ? in : vin, more ? tile + stride : first, hkv, w, n, g);
  }
  for (; tile < tiles; tile += stride) {
    const int blk = tile / hkv;
    const int head = tile - blk * hkv;
    const int page = dst_pages[blk];
    const bool ok = page >= 0 && page < num_pages;
    bad |= !ok;
    const __amdgpu_buffer_rsrc_t dst =
        page_resource(pool + (static_cast<size_t>(ok ? page : 0) * hkv + head) * kPageBytes, ok ? kPageBytes : 0);

    // ---- 2. log2-variance normalisation, rows then columns, kNormIters times --
    // rf = 2^-rho / sqrt(128) multiplies the unnormalised R' (so R' rf = R 2^-rho).
    float rho_t = 0.f, rf_t = kInvSqrt128;  // normaliser of row t_red
    float gam_c = 0.f, cf_c = 1.f;          // normaliser of column c_red (= t_red)
    // normalisers of the lane's tokens / channels, and squares: every pass reads them from LDS
    // before use (the first row pass, from the input, needs none; its centred fallback takes the
    // column normalisers as 1)
    float rf[8], cf[8], r2[8], c2[8];
    // unrolled: the first pass's special cases resolve at compile time and the scheduler can
    // overlap each pass's tail with the next one's start (3.5% on the headline layer)
#pragma unroll
    for (int it = 0; it < kNormIters; ++it) {
      // ---------------- row pass: moments over channels of R' * cf ------------
      // Wave-local: the tokens of wave w are reduced by threads of wave w, so LDS order within
      // the wave (no workgroup barrier) is enough.  The first pass takes its moments from the
      // input (rotate), the others form 16 partial sums per token.
      if (it == 0) {
        if (g == 0) {
#pragma unroll
          for (int mt = 0; mt < 2; ++mt)
            *reinterpret_cast<float2*>(s.part_row.slot(32 * w + 16 * mt + n, 0)) = make_float2(m1[mt], m2[mt]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          float s1 = 0.f, s2 = 0.f;
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            s1 = fmaf(R[i][c], cf[c], s1);
            s2 = fmaf(P[i][c], c2[c], s2);
          }
          *reinterpret_cast<float2*>(s.part_row.slot(tok_of(w, g, i), n)) = make_float2(s1, s2);
        }
      }
      wave_lds_sync();
      {
        const float2 m = it == 0 ? *reinterpret_cast<const float2*>(s.part_row.slot(t_red, 0))
                                 : reduce_pairs(s.part_row.half(t_red, hf), hf);
        const float mu = m.x * inv128, ey2 = m.y * inv128;
        float var = fmaf(-mu, mu, ey2);
        if (__builtin_amdgcn_ballot_w64(!(var >= 0.5f * ey2)) != 0) {
          // centred second moment for every token of this wave
          if (hf == 0) s.mul_r[t_red] = mu;
          wave_lds_sync();
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float mi = s.mul_r[tok_of(w, g, i)];
            float q = 0.f;
#pragma unroll
            for (int c = 0; c < 8; ++c) {
              const float d = fmaf(R[i][c], it == 0 ? 1.f : cf[c], -mi);
              q = fmaf(d, d, q);
            }
            *reinterpret_cast<float2*>(s.part_row.slot(tok_of(w, g, i), n)) = make_float2(q, 0.f);
          }
          wave_lds_sync();
          var = reduce_pairs(s.part_row.half(t_red, hf), hf).x * inv128;
        }
        rho_t += 0.5f * lg2(fmaf(var, rf_t * rf_t, kNormEps));
        rf_t = ex2(-rho_t) * kInvSqrt128;
        (hf ? s.rfl2 : s.rfl)[t_red] = hf ? rf_t * rf_t : rf_t;
      }
      wave_lds_sync();
      {
        const float4 a = *reinterpret_cast<const float4*>(&s.rfl[32 * w + 4 * g]);
        const float4 b = *reinterpret_cast<const float4*>(&s.rfl[32 * w + 16 + 4 * g]);
        rf[0] = a.x; rf[1] = a.y; rf[2] = a.z; rf[3] = a.w;
        rf[4] = b.x; rf[5] = b.y; rf[6] = b.z; rf[7] = b.w;
        const float4 a2 = *reinterpret_cast<const float4*>(&s.rfl2[32 * w + 4 * g]);
        const float4 b2 = *reinterpret_cast<const float4*>(&s.rfl2[32 * w + 16 + 4 * g]);
        r2[0] = a2.x; r2[1] = a2.y; r2[2] = a2.z; r2[3] = a2.w;
        r2[4] = b2.x; r2[5] = b2.y; r2[6] = b2.z; r2[7] = b2.w;
      }
      // ---------------- column pass: moments over tokens of R' * rf -----------
      {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          float s1 = 0.f, s2 = 0.f;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            s1 = fmaf(R[i][c], rf[i], s1);
            s2 = fmaf(P[i][c], r2[i], s2);
          }
          *reinterpret_cast<float2*>(s.part.slot(chan_of(n, c), col_slot(w, g, n))) = make_float2(s1, s2);
        }
      }
      __syncthreads();
      {
        const float2 m = reduce_pairs(s.part.half(t_red, hf), hf);
        const float mu = m.x * inv128, ey2 = m.y * inv128;
        const float var = fmaf(-mu, mu, ey2);
        const float gam_new = gam_c + 0.5f * lg2(fmaf(var, cf_c * cf_c, kNormEps));
        const float cf_new = ex2(-gam_new);
        (hf ? s.cfl2 : s.cfl)[chan_slot(t_red)] = hf ? cf_new * cf_new : cf_new;
        // any column whose one-sweep variance could have lost digits redoes the pass centred;
        // the flag of the next pass is cleared here (every read of it happened before this
        // pass's first barrier)
        if (!(var >= 0.5f * ey2)) s.recenter[it & 1] = 1;
        if (tid == 0) s.recenter[(it + 1) & 1] = 0;
        __syncthreads();
        if (s.recenter[it & 1]) {
          if (hf == 0) s.mul_c[chan_slot(t_red)] = mu;
          __syncthreads();
          const float4 ma = *reinterpret_cast<const float4*>(&s.mul_c[8 * n]);
          const float4 mb = *reinterpret_cast<const float4*>(&s.mul_c[8 * n + 4]);
          const float mc[8] = {ma.x, ma.y, ma.z, ma.w, mb.x, mb.y, mb.z, mb.w};
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            float q = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const float d = fmaf(R[i][c], rf[i], -mc[c]);
              q = fmaf(d, d, q);
            }
            *reinterpret_cast<float2*>(s.part.slot(chan_of(n, c), col_slot(w, g, n))) = make_float2(q, 0.f);
          }
          __syncthreads();
          const float cvar = reduce_pairs(s.part.half(t_red, hf), hf).x * inv128;
          gam_c += 0.5f * lg2(fmaf(cvar, cf_c * cf_c, kNormEps));
          cf_c = ex2(-gam_c);
          (hf ? s.cfl2 : s.cfl)[chan_slot(t_red)] = hf ? cf_c * cf_c : cf_c;
          __syncthreads();
        } else {
          gam_c = gam_new;
          cf_c = cf_new;
        }
      }
      {
        const float4 a = *reinterpret_cast<const float4*>(&s.cfl[8 * n]);
        const float4 b = *reinterpret_cast<const float4*>(&s.cfl[8 * n + 4]);
        cf[0] = a.x; cf[1] = a.y; cf[2] = a.z; cf[3] = a.w;
        cf[4] = b.x; cf[5] = b.y; cf[6] = b.z; cf[7] = b.w;
        const float4 a2 = *reinterpret_cast<const float4*>(&s.cfl2[8 * n]);
        const float4 b2 = *reinterpret_cast<const float4*>(&s.cfl2[8 * n + 4]);
        c2[0] = a2.x; c2[1] = a2.y; c2[2] = a2.z; c2[3] = a2.w;
        c2[4] = b2.x; c2[5] = b2.y; c2[6] = b2.z; c2[7] = b2.w;
      }
    }

    // normalisers: rho of row t_red from one thread of the pair, gamma of column t_red from the other
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(hf ? gam_c : rho_t), dst,
                                          kCodeBytes + (hf ? Meta::kGamma : Meta::kRho) + 4 * t_red, 0, 0);

    // ---- 3. per-group min/max, fp16 scale and zero, round to nearest, pack ------
    // M = R' times the normaliser across the group axis; N = M times the group's own
    // normaliser (positive), so the group's min and max of N are those of M scaled, and
    // that factor is folded into the rounding FMA.  Codes are round-half-even(clamp(u, 0, L)) by the
    // byte conversion v_cvt_pk_u8_f32, which also places each code in a chosen byte of a dword.
    if constexpr (!kIsV) {
      // key groups: one channel over the 128 tokens, 2^kBits levels
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int c = 0; c < 8; ++c) R[i][c] *= rf[i];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        float a = R[0][c], b = R[0][c];
#pragma unroll
        for (int i = 1; i < 8; ++i) {
          a = fminf(a, R[i][c]);
          b = fmaxf(b, R[i][c]);
        }
        *reinterpret_cast<float2*>(s.part.slot(chan_of(n, c), col_slot(w, g, n))) = make_float2(a, b);
      }
      __syncthreads();
      {
        const float4* p = reinterpret_cast<const float4*>(s.part.half(t_red, hf));
        float mn = INFINITY, mx = -INFINITY;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float4 v = p[k];
          mn = min3_raw(mn, v.x, v.z);
          mx = max3_raw(mx, v.y, v.w);
        }
        // thread hf of the pair holds the partials of token half hf (waves 2hf, 2hf + 1): one group of
        // each half for group size 64, merged into the channel's one group otherwise
        if constexpr (!kHalf) {
          mn = min_raw(mn, dpp_xor1(mn));
          mx = max_raw(mx, dpp_xor1(mx));
        }
        mn = mul_rn(mn, cf_c);
        mx = mul_rn(mx, cf_c);
        const uint32_t sb = float_to_half_bits((mx - mn) / kLevels);
        const uint32_t zb = float_to_half_bits(mn);
        const float sf = half_bits_to_float(sb), zf = half_bits_to_float(zb);
        const float inv = sf > 0.f ? 1.0f / sf : 0.f;
        if constexpr (kHalf) {
          const int gi = 128 * hf + t_red;
          __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(sb), dst, kCodeBytes + Meta::kScale + 2 * gi, 0, 0);
          __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(zb), dst, kCodeBytes + Meta::kZero + 2 * gi, 0, 0);
          s.mul_a[hf][chan_slot(t_red)] = cf_c * inv;
          s.mul_b[hf][chan_slot(t_red)] = -zf * inv;
        } else {
          // scale from one thread of the pair, zero from the other
          __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(hf ? zb : sb), dst,
                                                kCodeBytes + (hf ? Meta::kZero : Meta::kScale) + 2 * t_red, 0, 0);
          // one per-lane address instead of a branch on hf: straight-line code schedules better
          (hf ? s.mul_b[0] : s.mul_a[0])[chan_slot(t_red)] = hf ? -zf * inv : cf_c * inv;
        }
      }
      __syncthreads();
      const int kh = kHalf ? (w >> 1) : 0;  // the groups of this wave's tokens
      const float4 a0 = *reinterpret_cast<const float4*>(&s.mul_a[kh][8 * n]);
      const float4 a1 = *reinterpret_cast<const float4*>(&s.mul_a[kh][8 * n + 4]);
      const float4 b0 = *reinterpret_cast<const float4*>(&s.mul_b[kh][8 * n]);
      const float4 b1 = *reinterpret_cast<const float4*>(&s.mul_b[kh][8 * n + 4]);
      const float qa[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
      const float qb[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
      auto kclamp = [&](int i, int c) { return fminf(fmaxf(fmaf(R[i][c], qa[c], qb[c]), 0.f), kLevels); };
      if constexpr (kBits == 4) {
        // byte (i, h4) = code(c = 2h4) | code(c = 2h4 + 1) << 4 is byte 16*h4 + n of token T(i);
        // a quad transpose gives lane j of quad q the dword at bytes 16*h4 + 4q of token T(4*ih + j).
        // v_cvt_pk_u8_f32 rounds the clamped value to nearest even (as the magic add does) and
        // writes it into byte y, so the even-channel codes of the four tokens fill one dword, the
        // odd-channel codes another, and one shift-or pairs them.
        const int j = n & 3, q = n >> 2;
#pragma unroll
        for (int ih = 0; ih < 2; ++ih) {
#pragma unroll
          for (int h4 = 0; h4 < 4; ++h4) {
            uint32_t ce = 0, co = 0;
#pragma unroll
            for (int y = 0; y < 4; ++y) {
              const int i = 4 * ih + y;
              ce = __builtin_amdgcn_cvt_pk_u8_f32(kclamp(i, 2 * h4), y, ce);
              co = __builtin_amdgcn_cvt_pk_u8_f32(kclamp(i, 2 * h4 + 1), y, co);
            }
            const uint32_t word = quad_transpose(ce | (co << 4), j);
            __builtin_amdgcn_raw_buffer_store_b32(word, dst, tok_of(w, g, 4 * ih + j) * 64 + 16 * h4 + 4 * q, 0, 0);
          }
        }
      } else {
        // one byte per code: halfword (i, h4) = code(2h4) | code(2h4 + 1) << 8 is bytes 32*h4 + 2n of token
        // T(i) (128 bytes per token).  Lanes n and n ^ 1 swap halfwords so that the even lane holds
        // the dword of token T(2k) and the odd lane that of token T(2k + 1), at bytes 32*h4 + 4(n/2).
        const bool odd = n & 1;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
#pragma unroll
          for (int h4 = 0; h4 < 4; ++h4) {
            uint32_t v = __builtin_amdgcn_cvt_pk_u8_f32(kclamp(2 * k, 2 * h4), 0, 0u);
            v = __builtin_amdgcn_cvt_pk_u8_f32(kclamp(2 * k, 2 * h4 + 1), 1, v);
            v = __builtin_amdgcn_cvt_pk_u8_f32(kclamp(2 * k + 1, 2 * h4), 2, v);
            v = __builtin_amdgcn_cvt_pk_u8_f32(kclamp(2 * k + 1, 2 * h4 + 1), 3, v);
            const uint32_t p = dpp_u32(v, 0);  // lane n ^ 1
            const uint32_t word = odd ? ((p >> 16) | (v & 0xFFFF0000u)) : ((v & 0xFFFFu) | (p << 16));
            __builtin_amdgcn_raw_buffer_store_b32(word, dst, tok_of(w, g, 2 * k + (odd ? 1 : 0)) * 128 + 32 * h4 +
                                                                 4 * (n >> 1), 0, 0);
          }
        }
      }
    } else {
      // value groups: one token over the 128 channels, 2^kBits levels
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int c = 0; c < 8; ++c) R[i][c] *= cf[c];
      // the lane's channels c = 0..3 lie in channels 0..63, c = 4..7 in 64..127 (chan_of)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float a = R[i][0], b = R[i][0];
#pragma unroll
        for (int c = 1; c < 4; ++c) {
          a = fminf(a, R[i][c]);
          b = fmaxf(b, R[i][c]);
        }
        if constexpr (kHalf) {
          float a1 = R[i][4], b1 = R[i][4];
#pragma unroll
          for (int c = 5; c < 8; ++c) {
            a1 = fminf(a1, R[i][c]);
            b1 = fmaxf(b1, R[i][c]);
          }
          // channel half 0 in the channel array, half 1 in the (now idle) row array
          *reinterpret_cast<float2*>(s.part.slot(tok_of(w, g, i), n)) = make_float2(a, b);
          *reinterpret_cast<float2*>(s.part_row.slot(tok_of(w, g, i), n)) = make_float2(a1, b1);
        } else {
#pragma unroll
          for (int c = 4; c < 8; ++c) {
            a = fminf(a, R[i][c]);
            b = fmaxf(b, R[i][c]);
          }
          *reinterpret_cast<float2*>(s.part.slot(tok_of(w, g, i), n)) = make_float2(a, b);
        }
      }
      __syncthreads();
      {
        float mn = INFINITY, mx = -INFINITY;
        if constexpr (kHalf) {
          // thread hf of the pair reduces channel half hf of token t_red: all 16 lanes' partials
          PartRows& pr = hf ? s.part_row : s.part;
          const float4* p0 = reinterpret_cast<const float4*>(pr.half(t_red, 0));
          const float4* p1 = reinterpret_cast<const float4*>(pr.half(t_red, 1));
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const float4 v = k < 4 ? p0[k] : p1[k - 4];
            mn = min3_raw(mn, v.x, v.z);
            mx = max3_raw(mx, v.y, v.w);
          }
        } else {
          const float4* p = reinterpret_cast<const float4*>(s.part.half(t_red, hf));
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const float4 v = p[k];
            mn = min3_raw(mn, v.x, v.z);
            mx = max3_raw(mx, v.y, v.w);
          }
          mn = min_raw(mn, dpp_xor1(mn));
          mx = max_raw(mx, dpp_xor1(mx));
        }
        mn = mul_rn(mn, rf_t);
        mx = mul_rn(mx, rf_t);
        const uint32_t sb = float_to_half_bits((mx - mn) / kLevels);
        const uint32_t zb = float_to_half_bits(mn);
        const float sf = half_bits_to_float(sb), zf = half_bits_to_float(zb);
        const float inv = sf > 0.f ? 1.0f / sf : 0.f;
        if constexpr (kHalf) {
          const int gi = 128 * hf + t_red;
          __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(sb), dst, kCodeBytes + Meta::kScale + 2 * gi, 0, 0);
          __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(zb), dst, kCodeBytes + Meta::kZero + 2 * gi, 0, 0);
          s.mul_a[hf][t_red] = rf_t * inv;
          s.mul_b[hf][t_red] = -zf * inv;
        } else {
          __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(hf ? zb : sb), dst,
                                                kCodeBytes + (hf ? Meta::kZero : Meta::kScale) + 2 * t_red, 0, 0);
          (hf ? s.mul_b[0] : s.mul_a[0])[t_red] = hf ? -zf * inv : rf_t * inv;
        }
      }
      __syncthreads();
      float qa[8], qb[8];
      // rounding factors of the lane's 8 tokens for channel half vh (the only half for group size 128)
      auto load_q = [&](int vh) {
        const float4 a0 = *reinterpret_cast<const float4*>(&s.mul_a[vh][32 * w + 4 * g]);
        const float4 a1 = *reinterpret_cast<const float4*>(&s.mul_a[vh][32 * w + 16 + 4 * g]);
        const float4 b0 = *reinterpret_cast<const float4*>(&s.mul_b[vh][32 * w + 4 * g]);
        const float4 b1 = *reinterpret_cast<const float4*>(&s.mul_b[vh][32 * w + 16 + 4 * g]);
        qa[0] = a0.x; qa[1] = a0.y; qa[2] = a0.z; qa[3] = a0.w; qa[4] = a1.x; qa[5] = a1.y; qa[6] = a1.z; qa[7] = a1.w;
        qb[0] = b0.x; qb[1] = b0.y; qb[2] = b0.z; qb[3] = b0.w; qb[4] = b1.x; qb[5] = b1.y; qb[6] = b1.z; qb[7] = b1.w;
      };
      load_q(0);
      auto vclamp = [&](int i, int c) { return fminf(fmaxf(fmaf(R[i][c], qa[i], qb[i]), 0.f), kLevels); };
      if constexpr (kBits == 2) {
        // byte (c, ih) = codes of tokens T(4ih + y), y = 0..3, at bits 2y: byte 8w + 4ih + g of
        // channel C(c).  A row transpose gives row y the dword of combination (c, ih) = (2u + y/2, y%2)
        // of unit u: bytes 8w + 4ih .. +3 of that channel.
        // v_cvt_pk_u8_f32 (round to nearest even, into byte y) gathers the k-th code of the four
        // bytes in one dword per k; shifts by 2k put the four dwords' codes side by side in every byte.
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (kHalf && u == 2) load_q(1);  // channels c = 4..7 from here on
          uint32_t d[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            d[k] = 0;
#pragma unroll
            for (int y = 0; y < 4; ++y) {
              const int c = 2 * u + (y >> 1), ih = y & 1;
              d[k] = __builtin_amdgcn_cvt_pk_u8_f32(vclamp(4 * ih + k, c), y, d[k]);
            }
          }
          const uint32_t word = row_transpose(d[0] | (d[1] << 2) | (d[2] << 4) | (d[3] << 6), g);
          const int c = 2 * u + (g >> 1), ih = g & 1;
          __builtin_amdgcn_raw_buffer_store_b32(word, dst, chan_of(n, c) * 32 + 8 * w + 4 * ih, 0, 0);
        }
      } else {
        // two codes per byte: halfword (c, ih) = codes of tokens T(4ih + k), k = 0..3, at bits 4k is
        // bytes 16w + 8ih + 2g of channel C(c) (64 bytes per channel).  Rows g and g ^ 1 swap
        // halfwords (v_permlane16_swap returns (lower row's value, upper row's value)) so that the
        // even row holds the dword of ih = 0 and the odd row that of ih = 1, at bytes 16w + 8ih + 4(g/2).
        const bool odd = g & 1;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          if (kHalf && c == 4) load_q(1);  // channels c = 4..7 from here on
          // byte 2 ih + kk holds tokens T(4 ih + 2 kk) (low nibble) and T(4 ih + 2 kk + 1) (high nibble)
          uint32_t ce = 0, co = 0;
#pragma unroll
          for (int y = 0; y < 4; ++y) {
            const int i = 4 * (y >> 1) + 2 * (y & 1);
            ce = __builtin_amdgcn_cvt_pk_u8_f32(vclamp(i, c), y, ce);
            co = __builtin_amdgcn_cvt_pk_u8_f32(vclamp(i + 1, c), y, co);
          }
          const uint32_t v = ce | (co << 4);
          const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
          const uint32_t word = odd ? ((r[0] >> 16) | (r[1] & 0xFFFF0000u)) : ((r[0] & 0xFFFFu) | (r[1] << 16));
          __builtin_amdgcn_raw_buffer_store_b32(word, dst, chan_of(n, c) * 64 + 16 * w + 8 * (odd ? 1 : 0) +
                                                                 4 * (g >> 1), 0, 0);
        }
      }
    }
    const int next = tile + stride;
    if constexpr (!kIsV) {
      // xa holds key tile `next`, or the first value tile once the keys are done
      rotate(xa, hb, hbn, R, P, m1, m2, g);
      const bool more = next + stride < tiles;
      const int vt = next < tiles ? first : (first + stride < tiles ? first + stride : first);
      load_tile(xa, more ? in : vin, more ? next + stride : vt, hkv, w, n, g);
    } else {
      // past the last value tile the last one stands in (a uniform branch here measured slower)
      const int nt = next < tiles ? next : tile;
      rotate(xa, hb, hbn, R, P, m1, m2, g);
      load_tile(xa, in, nt + stride < tiles ? nt + stride : nt, hkv, w, n, g);
    }
  }
  if (bad && tid == 0 && flags) atomicOr(flags, kFlagBadPage);
}

}  // namespace

// Persistent quantiser: every workgroup walks the key tiles blockIdx.x, blockIdx.x + gridDim.x, ...
// and then the value tiles with the same stride, so all workgroups carry the same mix of the two
// kinds (a value tile costs more than a key tile).  The input pipeline (xa: the tile in flight;
// R, P, m1, m2: the rotated one) runs on from the keys into the values without a second fill.
template <int kKBits, int kVBits, int kGroup>
__global__ __launch_bounds__(256, 2) void quantize_kernel(const uint16_t* __restrict__ kin,
                                                         const uint16_t* __restrict__ vin, int hkv, int tiles,
                                                         const int32_t* __restrict__ dst_pages,
                                                         uint8_t* __restrict__ k_pool, uint8_t* __restrict__ v_pool,
                                                         int num_pages, uint32_t* __restrict__ flags) {
  __shared__ __align__(16) QuantLds lds;
  f16x8 xa[2][4];         // input in flight
  float R[8][8], P[8][8];  // rotated tile and its squares
  float m1[2], m2[2];      // first row pass's moments of tokens 32w + 16 mt + n
  quantize_tiles<false, kKBits, kGroup>(kin, vin, hkv, tiles, dst_pages, k_pool, num_pages, flags, lds, xa, R, P,
                                        m1, m2);
  quantize_tiles<true, kVBits, kGroup>(vin, vin, hkv, tiles, dst_pages, v_pool, num_pages, flags, lds, xa, R, P,
                                       m1, m2);
}

// Test / inspection export: rebuild fp32 K^ or V^ of one tile in the original basis.
__global__ __launch_bounds__(256) void dequantize_kernel(const uint8_t* __restrict__ k_pool,
                                                         const uint8_t* __restrict__ v_pool, int num_pages,
                                                         const int32_t* __restrict__ pages, int hkv, int kbits,
                                                         int vbits, int group, float* __restrict__ k_out,
                                                         float* __restrict__ v_out, uint32_t* __restrict__ flags) {
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
  const int code_bytes = kBlockTokens * kHeadDim * (is_v ? vbits : kbits) / 8;
  const bool half = group == 64;
  const int meta_bytes = half ? MetaLayout<64>::kBytes : MetaLayout<128>::kBytes;
  const uint8_t* pb = (is_v ? v_pool : k_pool) + (static_cast<size_t>(page) * hkv + head) * (code_bytes + meta_bytes);
  const uint8_t* meta = pb + code_bytes;
  const uint16_t* sc = reinterpret_cast<const uint16_t*>(meta + (half ? MetaLayout<64>::kScale : MetaLayout<128>::kScale));
  const uint16_t* zr = reinterpret_cast<const uint16_t*>(meta + (half ? MetaLayout<64>::kZero : MetaLayout<128>::kZero));
  const float* rho = reinterpret_cast<const float*>(meta + (half ? MetaLayout<64>::kRho : MetaLayout<128>::kRho));
  const float* gam = reinterpret_cast<const float*>(meta + (half ? MetaLayout<64>::kGamma : MetaLayout<128>::kGamma));
  for (int e = threadIdx.x; e < kBlockTokens * kHeadDim; e += blockDim.x) {
    const int t = e >> 7, j = e & 127;
    uint32_t code;
    float s, z;
    if (is_v) {
      code = vbits == 4 ? (pb[64 * j + (t >> 1)] >> (4 * (t & 1))) & 15u : (pb[32 * j + (t >> 2)] >> (2 * (t & 3))) & 3u;
      const int gi = (half ? 128 * (j >> 6) : 0) + t;  // value group: token t, channel half
      s = half_bits_to_float(sc[gi]);
      z = half_bits_to_float(zr[gi]);
    } else {
      code = kbits == 8 ? pb[128 * t + j] : (pb[64 * t + (j >> 1)] >> (4 * (j & 1))) & 15u;
      const int gi = (half ? 128 * (t >> 6) : 0) + j;  // key group: channel j, token half
      s = half_bits_to_float(sc[gi]);
      z = half_bits_to_float(zr[gi]);
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
                           void* k_pool, void* v_pool, int num_pages, int kbits, int vbits, int group,
                           uint32_t* flags, hipStream_t stream) {
  const int tiles = n_blocks * hkv;  // per kind
  if (tiles == 0) return hipSuccess;
  // two persistent workgroups per compute unit
  int device = 0, cus = 0;
  hipError_t e = hipGetDevice(&device);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
  if (e != hipSuccess) return e;
  const int groups = tiles < 2 * cus ? tiles : 2 * cus;
  auto kernel = group == 64
                    ? (kbits == 8 ? (vbits == 4 ? quantize_kernel<8, 4, 64> : quantize_kernel<8, 2, 64>)
                                  : (vbits == 4 ? quantize_kernel<4, 4, 64> : quantize_kernel<4, 2, 64>))
                    : (kbits == 8 ? (vbits == 4 ? quantize_kernel<8, 4, 128> : quantize_kernel<8, 2, 128>)
                                  : (vbits == 4 ? quantize_kernel<4, 4, 128> : quantize_kernel<4, 2, 128>));
  hipLaunchKernelGGL(kernel, dim3(groups), dim3(256), 0, stream, static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), hkv, tiles, dst_pages, static_cast<uint8_t*>(k_pool),
                     static_cast<uint8_t*>(v_pool), num_pages, flags);
  return hipGetLastError();
}

hipError_t launch_dequantize(const void* k_pool, const void* v_pool, int num_pages, const int32_t* pages,
                             int n_blocks, int hkv, int kbits, int vbits, int group, float* k_out, float* v_out,
                             uint32_t* flags, hipStream_t stream) {
  const unsigned tiles = 2u * static_cast<unsigned>(n_blocks) * static_cast<unsigned>(hkv);
  hipLaunchKernelGGL(dequantize_kernel, dim3(tiles), dim3(256), 0, stream, static_cast<const uint8_t*>(k_pool),
                     static_cast<const uint8_t*>(v_pool), num_pages, pages, hkv, kbits, vbits, group, k_out, v_out,
                     flags);
  return hipGetLastError();
}

}  // namespace kvarn
