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

// fp32 -> bf16 round-to-nearest-even (NaN stays NaN): gfx950's v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f)); }

// Two bf16 in one dword: lo in bits 0..15, hi in bits 16..31 (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
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

// E4M3 codes of values already divided by their block scale: round to the nearest
// E4M3 value, ties to even, saturating at +-448, signed zero kept.  gfx950's
// v_cvt_pk_fp8_f32 rounds to nearest even into the OCP E4M3 format; clamping the input
// to +-448 first makes it saturate (448 is the largest finite E4M3 value and every
// |w| in (448, 464) rounds to it anyway).  Over all 2^32 fp32 inputs this equals the
// bit-level definition: the spacing of E4M3 values in binade b = max(floor(log2|w|), -6)
// is 2^(b-3), the significand is rounded to that spacing with ties to even, and results
// beyond 448 become 448.
__device__ __forceinline__ float e4m3_clamp(float w) { return __builtin_amdgcn_fmed3f(w, -448.f, 448.f); }

// codes of a, b in bytes 0, 1
__device__ __forceinline__ uint32_t e4m3x2(float a, float b) {
  return uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(a), e4m3_clamp(b), 0, false)) & 0xffffu;
}

// codes of a, b, c, d in bytes 0..3
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  int v = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(a), e4m3_clamp(b), 0, false);
  v = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(c), e4m3_clamp(d), v, true);
  return uint32_t(v);
}

__device__ __forceinline__ uint32_t e4m3_rne(float w) {
  return uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(w), 0.f, 0, false)) & 0xffu;
}

// Max over the 32 lanes of each half-wave, returned in every lane: DPP exchanges
// within 16-lane rows (xor 1, xor 2, mirror in 8, mirror in 16), then a swizzle that
// swaps the two 16-lane rows of each half.  Needs all 64 lanes active.
__device__ __forceinline__ float max_half_wave(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xf, 0xf, false)));    // quad_perm 1,0,3,2
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xf, 0xf, false)));    // quad_perm 2,3,0,1
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xf, 0xf, false)));   // row_half_mirror
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xf, 0xf, false)));   // row_mirror
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F)));                // swap 16-lane rows
  return v;
}

// v_permlane32_swap_b32: lanes 32..63 of a trade places with lanes 0..31 of b.  Returns
// the new (a, b): lane i < 32 then holds (a[i], a[i + 32]) and lane i + 32 holds
// (b[i], b[i + 32]).
struct U32Pair {
  uint32_t a, b;
};
__device__ __forceinline__ U32Pair permlane32_swap(uint32_t a, uint32_t b) {
  const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
  return U32Pair{uint32_t(r[0]), uint32_t(r[1])};
}

// max of v over lanes i and i ^ 32
__device__ __forceinline__ float max_xor32(float v) {
  const U32Pair r = permlane32_swap(__float_as_uint(v), __float_as_uint(v));
  return fmaxf(__uint_as_float(r.a), __uint_as_float(r.b));
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
