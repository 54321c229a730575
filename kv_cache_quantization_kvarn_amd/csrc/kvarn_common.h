// Shared device helpers for the libkvarn kernels (gfx950, wave64).
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvarn {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBlockTokens = 128;
constexpr int kHeadDim = 128;
constexpr int kKCodeBytes = 8192;   // token-major nibbles
constexpr int kVCodeBytes = 4096;   // channel-major 2-bit codes
constexpr int kMetaBytes = 1536;    // scale fp16[128], zero fp16[128], rho fp32[128], gamma fp32[128]
constexpr int kKPageBytes = kKCodeBytes + kMetaBytes;  // 9728
constexpr int kVPageBytes = kVCodeBytes + kMetaBytes;  // 5632
constexpr int kNormIters = 4;
constexpr float kNormEps = 1e-6f;
constexpr float kInvSqrt128 = 0.08838834764831845f;  // 2^-3.5, the orthonormal Hadamard scale
constexpr int kMaxGroup = 8;                           // query heads per KV head handled by one decode wave

// Offsets inside a page's metadata block (group size 128).
constexpr int kMetaScale = 0, kMetaZero = 256, kMetaRho = 512, kMetaGamma = 1024;

// Metadata block of a page with groups of kGroup elements: scale fp16[n], zero fp16[n], rho fp32[128
// tokens], gamma fp32[128 channels], with n = 128 groups for group size 128 and 2 x 128 for group
// size 64 (half-major: entry 128*h + j is the group over elements 64h .. 64h+63 of channel / token j).
template <int kGroup>
struct MetaLayout {
  static_assert(kGroup == 128 || kGroup == 64, "group size");
  static constexpr int kHalves = kBlockTokens / kGroup;
  static constexpr int kScale = 0;
  static constexpr int kZero = 2 * 128 * kHalves;
  static constexpr int kRho = 2 * kZero;
  static constexpr int kGamma = kRho + 4 * 128;
  static constexpr int kBytes = kGamma + 4 * 128;
};

constexpr uint32_t kFlagBadPage = 1u;
constexpr uint32_t kFlagBadSeqLen = 2u;

// DPP lane permutations inside a 16-lane row.  Every one is an involution
// (partner of partner is self), so x + dpp(x) is bitwise identical on both
// lanes of a pair.
constexpr int kDppXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppXor3 = 0x1B;   // quad_perm [3,2,1,0]
constexpr int kDppXor7 = 0x141;  // row_half_mirror: lane ^ 7 inside 8 lanes
constexpr int kDppXor8 = 0x128;  // row_ror:8: lane ^ 8 inside 16 lanes
constexpr int kDppRor4 = 0x124;  // row_ror:4: lane +- 4 (mod 16) inside 16 lanes (not an involution)

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Sum / min / max over the 16 lanes of a DPP row; every lane gets the same bits.
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp<kDppXor1>(x);
  x += dpp<kDppXor2>(x);
  x += dpp<kDppXor7>(x);
  x += dpp<kDppXor8>(x);
  return x;
}
__device__ __forceinline__ float row16_min(float x) {
  x = fminf(x, dpp<kDppXor1>(x));
  x = fminf(x, dpp<kDppXor2>(x));
  x = fminf(x, dpp<kDppXor7>(x));
  x = fminf(x, dpp<kDppXor8>(x));
  return x;
}
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp<kDppXor1>(x));
  x = fmaxf(x, dpp<kDppXor2>(x));
  x = fmaxf(x, dpp<kDppXor7>(x));
  x = fmaxf(x, dpp<kDppXor8>(x));
  return x;
}

// Sum / min / max over the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float rows4_sum(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}
__device__ __forceinline__ float rows4_min(float x) {
  x = fminf(x, __shfl_xor(x, 16));
  x = fminf(x, __shfl_xor(x, 32));
  return x;
}
__device__ __forceinline__ float rows4_max(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

__device__ __forceinline__ float wave_max(float x) {
  x = row16_max(x);
  return rows4_max(x);
}

__device__ __forceinline__ f32x4 mfma16x16x32(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float half_bits_to_float(uint32_t bits16) {
  return __half2float(__ushort_as_half(static_cast<unsigned short>(bits16)));
}
__device__ __forceinline__ uint32_t float_to_half_bits(float x) {
  return __half_as_ushort(__float2half_rn(x));
}

// 2^e for an integer e in the normal fp32 range.
__device__ __forceinline__ float pow2i(int e) { return __int_as_float((e + 127) << 23); }

}  // namespace kvarn
