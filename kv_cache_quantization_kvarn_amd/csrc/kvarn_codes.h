// Packed codes to exact fp16 matrix-core operands, shared by the decode kernels.
//
// A code c enters a v_mfma_f32_16x16x32_f16 product as the fp16 number off + c: a mask-and-or places
// it in the mantissa under a fixed exponent (the exponent fixes the offset), so a pair of codes costs
// one v_and_or_b32 and at most one shift.  The offsets are removed by the callers with sums of the
// coefficients the products used.  Element orders and offsets per format:
//   4-bit keys   (key_codes):   channels 0,4,1,5,2,6,3,7 of a dword; offset 64 for 1 and 5, else 16
//   8-bit keys   (key_codes8):  channels 0..7 of two dwords in order; offset 1024
//   2-bit values (value_codes): tokens (4hf + j, 4hf + j + 8) of 16 in a dword; offset 4 (even), 16 (odd)
//   4-bit values (value_codes4): the same token pairs from two dwords; offset 64
#pragma once

#include "kvarn_common.h"

namespace kvarn {

// Mask-and-or with the fp16 exponent pattern kept in a vector register (one v_and_or_b32;
// two literal constants would not fit one VOP3 encoding).
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t mask, uint32_t bits) {
  return (x & mask) | bits;
}

// Four fp16 pairs from one dword of 8 key nibbles (channel 8m+i at bits 4i):
// elements (0..7) = nibbles 0,4,1,5,2,6,3,7.  Nibbles 1 and 5 sit at mantissa bits
// 4-7 under `mag64` (fp16 64.0 twice) and read 64 + c; the others are shifted to
// bits 6-9 under `mag16` (16.0) and read 16 + c.
__device__ __forceinline__ f16x8 key_codes(uint32_t x, uint32_t mag16, uint32_t mag64) {
  u32x4 p;
  p[0] = and_or(x << 6, 0x03C003C0u, mag16);
  p[1] = and_or(x, 0x00F000F0u, mag64);
  p[2] = and_or(x >> 2, 0x03C003C0u, mag16);
  p[3] = and_or(x >> 6, 0x03C003C0u, mag16);
  return __builtin_bit_cast(f16x8, p);
}

// Two f16x8 operands from a word of 16 value codes (code k at bits 2k).  Operand hf
// holds pairs j = 0..3 of codes (4hf + j, 4hf + j + 8).  Even codes sit at mantissa
// bits 8-9 under `mag4` (fp16 4.0) and read 4 + c; odd codes at bits 6-7 under
// `mag16` (16.0) and read 16 + c.  Four shifts and eight mask-and-ors for 16 codes.
__device__ __forceinline__ void value_codes(uint32_t w, uint32_t mag4, uint32_t mag16, f16x8& lo, f16x8& hi) {
  const uint32_t r4 = w >> 4, l4 = w << 4, l8 = w << 8, r8 = w >> 8;
  u32x4 a, b;
  a[0] = and_or(l8, 0x03000300u, mag4);    // codes 0, 8
  a[1] = and_or(l4, 0x00C000C0u, mag16);   // codes 1, 9
  a[2] = and_or(l4, 0x03000300u, mag4);    // codes 2, 10
  a[3] = and_or(w, 0x00C000C0u, mag16);    // codes 3, 11
  b[0] = and_or(w, 0x03000300u, mag4);     // codes 4, 12
  b[1] = and_or(r4, 0x00C000C0u, mag16);   // codes 5, 13
  b[2] = and_or(r4, 0x03000300u, mag4);    // codes 6, 14
  b[3] = and_or(r8, 0x00C000C0u, mag16);   // codes 7, 15
  lo = __builtin_bit_cast(f16x8, a);
  hi = __builtin_bit_cast(f16x8, b);
}

// Four fp16 pairs from the 8 byte-wide key codes of channels 8m .. 8m+7 (d0: channels 0-3,
// d1: channels 4-7, channel i at bits 8i of its dword): elements in channel order, each code
// in the low mantissa byte under `mag1024` (fp16 1024.0 twice), reading 1024 + c.
__device__ __forceinline__ f16x8 key_codes8(uint32_t d0, uint32_t d1, uint32_t mag1024) {
  u32x4 p;
  p[0] = (d0 & 0xFFu) | ((d0 << 8) & 0x00FF0000u) | mag1024;          // channels 0, 1
  p[1] = ((d0 >> 16) & 0xFFu) | ((d0 >> 8) & 0x00FF0000u) | mag1024;  // 2, 3
  p[2] = (d1 & 0xFFu) | ((d1 << 8) & 0x00FF0000u) | mag1024;          // 4, 5
  p[3] = ((d1 >> 16) & 0xFFu) | ((d1 >> 8) & 0x00FF0000u) | mag1024;  // 6, 7
  return __builtin_bit_cast(f16x8, p);
}

// The two operands of value_codes from 16 nibble-wide value codes (d0: tokens 0-7, d1: tokens
// 8-15, token i at bits 4i of its dword).  The low halves of d0 and d1 (tokens 0-3 and 8-11)
// and the high halves (4-7 and 12-15) are put side by side, so that nibble j and nibble j + 4
// of each are the pair (4hf + j, 4hf + j + 8); every nibble is moved to mantissa bits 4-7 under
// `mag64` (fp16 64.0) and reads 64 + c.
__device__ __forceinline__ void value_codes4(uint32_t d0, uint32_t d1, uint32_t mag64, f16x8& lo, f16x8& hi) {
  const uint32_t e = (d0 & 0xFFFFu) | (d1 << 16);
  const uint32_t f = (d0 >> 16) | (d1 & 0xFFFF0000u);
  u32x4 a, b;
  a[0] = and_or(e << 4, 0x00F000F0u, mag64);  // tokens 0, 8
  a[1] = and_or(e, 0x00F000F0u, mag64);       // 1, 9
  a[2] = and_or(e >> 4, 0x00F000F0u, mag64);  // 2, 10
  a[3] = and_or(e >> 8, 0x00F000F0u, mag64);  // 3, 11
  b[0] = and_or(f << 4, 0x00F000F0u, mag64);  // 4, 12
  b[1] = and_or(f, 0x00F000F0u, mag64);       // 5, 13
  b[2] = and_or(f >> 4, 0x00F000F0u, mag64);  // 6, 14
  b[3] = and_or(f >> 8, 0x00F000F0u, mag64);  // 7, 15
  lo = __builtin_bit_cast(f16x8, a);
  hi = __builtin_bit_cast(f16x8, b);
}

}  // namespace kvarn
