// Shared device helpers of the gfx950 kernels: bf16 <-> f32, the MXFP8 (E4M3 + E8M0)
// block encoder, wave-level reductions and launch plumbing.
//
// MXFP8 per the OCP Microscaling Formats v1.0 specification (the pages only fix
// "8-bit values with one scale per block of 32 consecutive values"): the shared
// exponent of a block is floor(log2(amax)) - 8 (8 = the largest E4M3 exponent)
// clamped to the E8M0 range, and each element is v / 2^e rounded to the nearest
// E4M3 value (ties to even), saturating at 448.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mge.h"

namespace mge {

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// fp32 -> bf16 round-to-nearest-even (finite inputs; NaN keeps a quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// E8M0 scale byte of a block from its amax (|values| max as fp32):
// s = e + 127 with e = floor(log2 amax) - 8, clamped at 0 below (all-zero and tiny
// blocks).  For a normal fp32 amax, floor(log2 amax) = exponent field - 127, so
// s = field - 8; fp32 subnormals/zero have field 0.
__device__ __forceinline__ uint32_t mx_scale_byte(float amax) {
  int field = int((__float_as_uint(amax) >> 23) & 0xff);
  int s = field - 8;
  return uint32_t(s < 0 ? 0 : s);
}

// 2^-e for the scale byte s (e = s - 127): fp32 with exponent field 254 - s.
__device__ __forceinline__ float mx_inv_scale(uint32_t s) { return __uint_as_float((254u - s) << 23); }

// E4M3 code of w (already divided by the block scale), round-to-nearest-even,
// saturating at 448, signed zero kept.  Works on the fp32 bit pattern: the spacing of
// E4M3 values in the binade b = max(floor(log2|w|), -6) is 2^(b-3); the 24-bit
// significand is shifted right to that spacing with ties to even; the code is then
// 8*(b+7) + (multiple - 8), which also covers subnormals and the carry into the next
// binade.
__device__ __forceinline__ uint32_t e4m3_rne(float w) {
  uint32_t b = __float_as_uint(w);
  uint32_t sign = (b >> 24) & 0x80u;
  uint32_t a = b & 0x7fffffffu;
  if (a >= 0x43e00000u) return sign | 0x7eu;   // |w| >= 448
  if (a <= 0x3a800000u) return sign;           // |w| <= 2^-10 rounds to zero
  int E = int(a >> 23) - 127;                  // >= -10 here
  int bin = E < -6 ? -6 : E;
  uint32_t sig = (a & 0x7fffffu) | 0x800000u;
  int sh = bin - E + 20;                       // 20..24
  uint32_t q = sig >> sh;
  uint32_t rem = sig & ((1u << sh) - 1u);
  uint32_t half = 1u << (sh - 1);
  q += (rem > half) | ((rem == half) & (q & 1u));
  return sign | uint32_t(8 * (bin + 7) + int(q) - 8);
}

__device__ __forceinline__ float wave_max_xor(float v, int lanes) {
  // max over groups of `lanes` consecutive lanes (lanes = power of two <= 64)
  for (int o = 1; o < lanes; o <<= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_sum_xor(float v, int lanes) {
  for (int o = 1; o < lanes; o <<= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + __expf(-z)); }
__device__ __forceinline__ float sigmoid_f(float z) { return 1.0f / (1.0f + __expf(-z)); }

}  // namespace mge

// ---------------------------------------------------------------- host side plumbing
namespace mge {
void set_error(const char* fmt, ...);
mge_status hip_check(const char* what);
}  // namespace mge

#define MGE_REQUIRE(cond, ...)               \
  do {                                       \
    if (!(cond)) {                           \
      ::mge::set_error(__VA_ARGS__);         \
      return MGE_ERR_INVALID_ARG;            \
    }                                        \
  } while (0)
