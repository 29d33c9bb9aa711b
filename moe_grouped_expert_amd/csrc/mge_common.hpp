// Shared device helpers of the gfx950 kernels: bf16 <-> f32, the MXFP8 (E4M3 + E8M0)
// block encoder, wave-level reductions and launch plumbing.
//
// MXFP8 per the OCP Microscaling Formats v1.0 specification (the pages fix only 8-bit
// values sharing one scale per 32 consecutive values): the shared
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

// codes of a, b in bytes 0, 1.  The conversion writes one 16-bit half of its destination
// and keeps the other from its third operand; that half is masked off (or, in e4m3x4,
// overwritten), so the clamped a itself serves as that operand and no zero is loaded.
__device__ __forceinline__ uint32_t e4m3x2(float a, float b) {
  const float ca = e4m3_clamp(a);
  return uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(ca, e4m3_clamp(b), __float_as_int(ca), false)) & 0xffffu;
}

// codes of a, b, c, d in bytes 0..3
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  const float ca = e4m3_clamp(a);
  int v = __builtin_amdgcn_cvt_pk_fp8_f32(ca, e4m3_clamp(b), __float_as_int(ca), false);
  v = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(c), e4m3_clamp(d), v, true);
  return uint32_t(v);
}

__device__ __forceinline__ uint32_t e4m3_rne(float w) {
  const float cw = e4m3_clamp(w);
  return uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(cw, 0.f, __float_as_int(cw), false)) & 0xffu;
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

// v_permlane16_swap_b32: lanes 16..31 of a trade places with lanes 0..15 of b (and
// lanes 48..63 of a with lanes 32..47 of b).  Returns the new (a, b): a lane in rows 0, 2
// then holds (its a, the a of the lane 16 above), a lane in rows 1, 3 (the b of the lane
// 16 below, its b) (measured on MI355X).
__device__ __forceinline__ U32Pair permlane16_swap(uint32_t a, uint32_t b) {
  const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
  return U32Pair{uint32_t(r[0]), uint32_t(r[1])};
}

// Workgroup barrier for LDS data: this wave's LDS accesses have completed, then all waves
// meet.  Unlike __syncthreads(), whose fence also waits for every outstanding global
// load and store, it lets stores (and loads meant to stay in flight) continue across the
// barrier; the asm "memory" clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// The scale bytes of the 4 lanes of a quad, lane 4q + i in byte i (every lane of the quad
// gets the dword; all four lanes must be active)
__device__ __forceinline__ uint32_t quad_bytes(uint32_t s) {
  const uint32_t s0 = uint32_t(__builtin_amdgcn_mov_dpp(int(s), 0x00, 0xf, 0xf, false));   // quad_perm 0,0,0,0
  const uint32_t s1 = uint32_t(__builtin_amdgcn_mov_dpp(int(s), 0x55, 0xf, 0xf, false));   // 1,1,1,1
  const uint32_t s2 = uint32_t(__builtin_amdgcn_mov_dpp(int(s), 0xAA, 0xf, 0xf, false));   // 2,2,2,2
  const uint32_t s3 = uint32_t(__builtin_amdgcn_mov_dpp(int(s), 0xFF, 0xf, 0xf, false));   // 3,3,3,3
  return (s0 & 0xffu) | ((s1 & 0xffu) << 8) | ((s2 & 0xffu) << 16) | (s3 << 24);
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}

// max(|a|, |b|) of two fp32 bit patterns as one VOP3 max with abs modifiers.  Written as
// asm because the compiler otherwise canonicalizes each bit-cast operand first (one more
// max per operand) and clears the sign bits with separate ands; the result for NaN inputs
// is not defined here.
__device__ __forceinline__ uint32_t max_abs_bits(uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_max_f32_e64 %0, |%1|, |%2|" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return uint32_t(__builtin_amdgcn_mov_dpp(int(v), CTRL, 0xf, 0xf, true));
}

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

// Row blocks of a 32-column tile held column-wise: in each half-wave, lane c (= l32)
// holds v[0..15], the values of 16 rows in column c.  Computes, for each of the 16 rows,
// the E8M0 scale of its 32 values (their amax over the half-wave) and returns in inv[r]
// the reciprocal scale of row r in every lane, and in the result the scale byte of row
// l32 / 2.  A reduce-scatter (each exchange halves the rows a lane keeps: 16-lane swap,
// lane ^ 8 by row_ror:8, mirror in 8, lane ^ 2, lane ^ 1) leaves the amax of row l32 / 2
// in lanes 2r, 2r + 1.  After the first step the values are non-negative, and
// non-negative fp32 values order as their bit patterns: the later steps are integer maxes,
// which take the DPP exchange as an operand.  The 16 reciprocals return through `slot`,
// 16 floats of LDS per half-wave (lanes 2r, 2r + 1 write row r's, every lane reads all
// 16 back): one wave's LDS accesses are performed in issue order, and a wave barrier keeps
// the compiler from moving the reads above the write.  Needs all 64 lanes.
__device__ __forceinline__ uint32_t row_block_inv16(const float* v, int l32, float* inv, float* slot) {
  const bool b3 = (l32 & 8) != 0, b2 = (l32 & 4) != 0, b1 = (l32 & 2) != 0;
  // m1[i]: row i + 8*b4, amax over lanes c, c ^ 16
  uint32_t m1[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const U32Pair x = permlane16_swap(__float_as_uint(v[i]), __float_as_uint(v[i + 8]));
    m1[i] = max_abs_bits(x.a, x.b);
  }
  // m2[i]: row i + 4*b3 + 8*b4 (partner: lane ^ 8)
  uint32_t m2[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) m2[i] = umax(b3 ? m1[i + 4] : m1[i], dpp_u<0x128>(b3 ? m1[i] : m1[i + 4]));
  // m3[i]: row i + 2*b2 + 4*b3 + 8*b4 (partner: lane 7 - c within 8; same b3, b4)
  uint32_t m3[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) m3[i] = umax(b2 ? m2[i + 2] : m2[i], dpp_u<0x141>(b2 ? m2[i] : m2[i + 2]));
  // m4: row b1 + 2*b2 + 4*b3 + 8*b4 = l32 / 2 (partner: lane ^ 2); then lane ^ 1 holds the same row
  uint32_t m4 = umax(b1 ? m3[1] : m3[0], dpp_u<0x4E>(b1 ? m3[0] : m3[1]));
  m4 = umax(m4, dpp_u<0xB1>(m4));
  const uint32_t sc = mx_scale_byte(__uint_as_float(m4));
  slot[l32 >> 1] = mx_inv_scale(sc);
  __builtin_amdgcn_wave_barrier();   // the other lanes' writes before the reads (no instruction)
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const float4 q = *reinterpret_cast<const float4*>(slot + 4 * g);
    inv[4 * g] = q.x; inv[4 * g + 1] = q.y; inv[4 * g + 2] = q.z; inv[4 * g + 3] = q.w;
  }
  return sc;
}

// The row sums of the same layout (v[r]: row r, one column per lane of the half-wave):
// the reduce-scatter half of row_block_inv16 with sums, in a fixed order; returns the sum
// of row l32 / 2 (in lanes 2r and 2r + 1).
__device__ __forceinline__ float row_block_sum16(const float* v, int l32) {
  const bool b4 = (l32 & 16) != 0, b3 = (l32 & 8) != 0, b2 = (l32 & 4) != 0, b1 = (l32 & 2) != 0;
  float m1[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const U32Pair x = permlane16_swap(__float_as_uint(v[i]), __float_as_uint(v[i + 8]));
    m1[i] = __uint_as_float(x.a) + __uint_as_float(x.b);
  }
  float m2[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) m2[i] = (b3 ? m1[i + 4] : m1[i]) + dpp_f<0x128>(b3 ? m1[i] : m1[i + 4]);
  float m3[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) m3[i] = (b2 ? m2[i + 2] : m2[i]) + dpp_f<0x141>(b2 ? m2[i] : m2[i + 2]);
  const float m4 = (b1 ? m3[1] : m3[0]) + dpp_f<0x4E>(b1 ? m3[0] : m3[1]);
  return m4 + dpp_f<0xB1>(m4);
}

// max of a non-negative v over lanes i and i ^ 32 (an integer max of the bit patterns)
__device__ __forceinline__ float max_xor32(float v) {
  const U32Pair r = permlane32_swap(__float_as_uint(v), __float_as_uint(v));
  return __uint_as_float(umax(r.a, r.b));
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
