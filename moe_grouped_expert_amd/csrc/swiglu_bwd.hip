// Backward of the probability-scaled SwiGLU, between the dh GEMM and the dX / dW_gate_up
// GEMMs.  Per permuted row m (token assignment with probability p) and ffn column f,
// with G, U the gate and up pre-activations saved by the forward and dh = dY W_down:
//   dU = dh * p * silu(G)
//   dG = dh * p * U * silu'(G),   silu'(z) = sig(z) * (1 + z * (1 - sig(z)))
//   d_prob[m] = sum_f dh * silu(G) * U
// dG and dU are written as the gradient of [G U] in row form (blocks of 32 along 2F)
// and column form (blocks of 32 rows, i.e. along tokens), MXFP8 or bf16, for the two
// GEMMs that consume them.  Padding rows (perm_src = -1) produce zeros.
//
// One workgroup owns 32 rows and walks the ffn columns in chunks of 256.  Each thread
// handles one 32-column block of one row (8 threads per row): it reads its dh (fp32),
// G and U (bf16) with 16-byte loads, quantizes its two row blocks (dG and dU) entirely
// in registers, and accumulates its part of the d_prob row sum.  The column form goes
// through LDS: the 32 x 256 dG and dU values are transposed so that a thread owns one
// column's 32 rows.  HBM-bound: 12 B per (row, column) at MXFP8
// (4 dh + 4 G,U read, 2 + 2 codes written).
#include "mge_common.hpp"
#include "mge_internal.hpp"

namespace mge {

constexpr int SB_ROWS = 32;
constexpr int SB_COLS = 256;
constexpr int SB_LDS_STRIDE = SB_COLS + 1;   // floats per LDS row (breaks column-read bank conflicts)

template <bool MX>
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(SwigluBwdParams p) {
  __shared__ float sv[SB_ROWS * SB_LDS_STRIDE];
  const int tid = threadIdx.x;
  const int rloc = tid >> 3;                 // row within the 32-row block
  const int blk = tid & 7;                   // 32-column block within the chunk
  const int r0 = blockIdx.x * SB_ROWS;
  const int row = r0 + rloc;
  const int F = p.F, F2 = 2 * F;
  const bool rok = row < p.R && p.perm_src[row] >= 0;
  const float pr = rok ? p.prob[row] : 0.f;
  const float* __restrict__ dhrow = p.dh + int64_t(row) * F;
  const uint16_t* __restrict__ gurow = p.gu + int64_t(row) * F2;
  float dps = 0.f;

  for (int c0 = 0; c0 < F; c0 += SB_COLS) {
    const int f0 = c0 + blk * 32;             // first column of this thread's block
    const bool bok = rok && f0 < F;           // F is a multiple of 32
    float dg[32], du[32];
    if (bok) {
      float4 d4[8];
      uint4 g4[4], u4[4];
#pragma unroll
      for (int i = 0; i < 8; ++i) d4[i] = reinterpret_cast<const float4*>(dhrow + f0)[i];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        g4[i] = reinterpret_cast<const uint4*>(gurow + f0)[i];
        u4[i] = reinterpret_cast<const uint4*>(gurow + F + f0)[i];
      }
      const float* dv = reinterpret_cast<const float*>(d4);
      const uint32_t* gw = reinterpret_cast<const uint32_t*>(g4);
      const uint32_t* uw = reinterpret_cast<const uint32_t*>(u4);
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const uint32_t gb = (j & 1) ? (gw[j >> 1] & 0xffff0000u) : (gw[j >> 1] << 16);
        const uint32_t ub = (j & 1) ? (uw[j >> 1] & 0xffff0000u) : (uw[j >> 1] << 16);
        const float G = __uint_as_float(gb), U = __uint_as_float(ub), dh = dv[j];
        const float sg = sigmoid_f(G);
        const float sl = G * sg;
        dps += dh * sl * U;
        du[j] = dh * pr * sl;
        dg[j] = dh * pr * U * sg * (1.f + G * (1.f - sg));
      }
    } else {
#pragma unroll
      for (int j = 0; j < 32; ++j) { dg[j] = 0.f; du[j] = 0.f; }
    }
    // ---- row form: blocks of 32 along 2F (dG at column f, dU at F + f)
    if (row < p.R && f0 < F) {
      if (MX) {
        for (int h = 0; h < 2; ++h) {
          const float* v = h == 0 ? dg : du;
          float amax = 0.f;
#pragma unroll
          for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(v[j]));
          const uint32_t s = mx_scale_byte(amax);
          const float inv = mx_inv_scale(s);
          uint32_t w[8];
#pragma unroll
          for (int q = 0; q < 8; ++q)
            w[q] = e4m3_rne(v[4 * q] * inv) | (e4m3_rne(v[4 * q + 1] * inv) << 8) | (e4m3_rne(v[4 * q + 2] * inv) << 16) |
                   (e4m3_rne(v[4 * q + 3] * inv) << 24);
          const int col = h * F + f0;
          uint4* dst = reinterpret_cast<uint4*>(p.row_codes + int64_t(row) * F2 + col);
          dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
          dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
          p.row_scales[int64_t(row) * (F2 / 32) + col / 32] = uint8_t(s);
        }
      } else {
        for (int h = 0; h < 2; ++h) {
          const float* v = h == 0 ? dg : du;
          uint32_t w[16];
#pragma unroll
          for (int q = 0; q < 16; ++q) w[q] = uint32_t(f32_to_bf16(v[2 * q])) | (uint32_t(f32_to_bf16(v[2 * q + 1])) << 16);
          uint4* dst = reinterpret_cast<uint4*>(p.row_bf16 + int64_t(row) * F2 + h * F + f0);
#pragma unroll
          for (int q = 0; q < 4; ++q) dst[q] = make_uint4(w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]);
        }
      }
    }
    // ---- column form through LDS (dG, then dU): thread c owns column c0 + c of the
    // chunk, all 32 rows
    const int c = tid;                        // column within the chunk
    const int f = c0 + c;
    for (int h = 0; h < 2; ++h) {
      const float* src = h == 0 ? dg : du;
      __syncthreads();   // previous readers of sv are done
#pragma unroll
      for (int j = 0; j < 32; ++j) sv[rloc * SB_LDS_STRIDE + blk * 32 + j] = src[j];
      __syncthreads();
      if (f < F && r0 < p.Rp) {
        float v[32];
#pragma unroll
        for (int j = 0; j < 32; ++j) v[j] = sv[j * SB_LDS_STRIDE + c];
        const int col = h * F + f;
        if (MX) {
          float amax = 0.f;
#pragma unroll
          for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(v[j]));
          const uint32_t s = mx_scale_byte(amax);
          const float inv = mx_inv_scale(s);
          uint32_t w[8];
#pragma unroll
          for (int q = 0; q < 8; ++q)
            w[q] = e4m3_rne(v[4 * q] * inv) | (e4m3_rne(v[4 * q + 1] * inv) << 8) | (e4m3_rne(v[4 * q + 2] * inv) << 16) |
                   (e4m3_rne(v[4 * q + 3] * inv) << 24);
          uint4* dst = reinterpret_cast<uint4*>(p.col_codes + int64_t(col) * p.Rp + r0);
          dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
          dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
          p.col_scales[int64_t(col) * (p.Rp / 32) + r0 / 32] = uint8_t(s);
        } else {
          uint32_t w[16];
#pragma unroll
          for (int q = 0; q < 16; ++q) w[q] = uint32_t(f32_to_bf16(v[2 * q])) | (uint32_t(f32_to_bf16(v[2 * q + 1])) << 16);
          uint4* dst = reinterpret_cast<uint4*>(p.col_bf16 + int64_t(col) * p.Rp + r0);
#pragma unroll
          for (int q = 0; q < 4; ++q) dst[q] = make_uint4(w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]);
        }
      }
    }
  }
  // ---- d_prob of the row: the 8 threads of a row are 8 consecutive lanes
  dps += __shfl_xor(dps, 1);
  dps += __shfl_xor(dps, 2);
  dps += __shfl_xor(dps, 4);
  if (blk == 0 && rok) p.dprob_row[row] = dps;
}

mge_status launch_swiglu_bwd(const SwigluBwdParams& p, bool mx, hipStream_t s) {
  if (p.R <= 0) return MGE_OK;
  dim3 grid((p.R + SB_ROWS - 1) / SB_ROWS);
  ProfScope prof(s, mx ? "swiglu_bwd_mx" : "swiglu_bwd_bf16");
  if (mx)
    hipLaunchKernelGGL(swiglu_bwd_kernel<true>, grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(swiglu_bwd_kernel<false>, grid, dim3(256), 0, s, p);
  return hip_check("swiglu_bwd_kernel");
}

}  // namespace mge
