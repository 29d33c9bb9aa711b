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
// A workgroup owns a tile of 128 rows x 256 ffn columns and walks it in sub-tiles of 64
// columns (the grid, rows x column groups, has thousands of workgroups: HBM-bound work
// needs many waves in flight).  In a sub-tile, thread t takes row t/2 and the 32-column
// block t%2: it reads its dh (fp32), G and U (bf16) with 16-byte loads, quantizes its
// dG and dU row blocks in registers and adds to its share of the row's d_prob.  The
// column form goes through LDS one array at a time (dG, then dU).  There, thread t takes
// column t/4 and rows 32*(t%4)..+31, so the 4 lanes of a column write its 128 rows as
// one 128-byte piece of one store instruction.  The 128 x 64 values are stored with a
// row stride of 65 floats plus 16 floats per 32-row group, so that both the row-wise
// stores and the column-wise reads hit 64 distinct banks.
// d_prob leaves as one partial sum per (row, column group), summed in a fixed order by
// the d_prob reduction.  HBM-bound: 12 B per (row, column) at MXFP8 (4 dh + 4 G,U read,
// 2 + 2 codes written).
#include "mge_common.hpp"
#include "mge_internal.hpp"

namespace mge {

constexpr int SB_ROWS = 128;                 // rows of a workgroup tile
constexpr int SB_COLS = 256;                 // ffn columns of a workgroup tile
constexpr int SB_SUB = 64;                   // columns of a sub-tile (one LDS round)
constexpr int SB_LD = SB_SUB + 1;            // LDS row stride in floats
constexpr int SB_GRP = 16;                   // extra floats per 32-row group
__device__ __forceinline__ int sb_at(int row, int col) { return row * SB_LD + (row >> 5) * SB_GRP + col; }

int swiglu_bwd_nparts(int F) { return (F + SB_COLS - 1) / SB_COLS; }

// One block of 32 consecutive values: MXFP8 codes (32 B) + E8M0 scale, or bf16 (64 B).
__device__ __forceinline__ void store_mx32(const float* v, uint8_t* codes, uint8_t* scale) {
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(v[j]));
  const uint32_t s = mx_scale_byte(amax);
  const float inv = mx_inv_scale(s);
  uint32_t w[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) w[q] = e4m3x4(v[4 * q] * inv, v[4 * q + 1] * inv, v[4 * q + 2] * inv, v[4 * q + 3] * inv);
  uint4* dst = reinterpret_cast<uint4*>(codes);
  dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
  dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
  *scale = uint8_t(s);
}

__device__ __forceinline__ void store_bf16x32(const float* v, uint16_t* dst16) {
  uint32_t w[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) w[q] = bf16x2(v[2 * q], v[2 * q + 1]);
  uint4* dst = reinterpret_cast<uint4*>(dst16);
#pragma unroll
  for (int q = 0; q < 4; ++q) dst[q] = make_uint4(w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]);
}

template <bool MX>
__global__ __launch_bounds__(256, 4) void swiglu_bwd_kernel(SwigluBwdParams p) {
  __shared__ float sv[SB_ROWS * SB_LD + (SB_ROWS / 32) * SB_GRP];
  const int tid = threadIdx.x;
  const int r0 = blockIdx.x * SB_ROWS;
  const int cg = blockIdx.y;                 // column group
  const int F = p.F, F2 = 2 * F;
  // row-wise mapping
  const int rl = tid >> 1, hh = tid & 1;
  const int row = r0 + rl;
  const bool rin = row < p.R;
  const bool rok = rin && p.perm_src[row] >= 0;
  const float pr = rok ? p.prob[row] : 0.f;
  // column-wise mapping
  const int c = tid >> 2, rb = tid & 3;
  const int rr = r0 + rb * 32;               // first row of this thread's column block
  float dps = 0.f;

  for (int sub = 0; sub < SB_COLS / SB_SUB; ++sub) {
    const int f0 = cg * SB_COLS + sub * SB_SUB;
    if (f0 >= F) break;                      // workgroup-uniform
    const int fb = f0 + hh * 32;             // this thread's row block (F is a multiple of 32)
    const bool bok = fb < F;
    float dg[32], du[32];
    if (rok && bok) {
      const float* dhp = p.dh + int64_t(row) * F + fb;
      const uint16_t* gp = p.gu + int64_t(row) * F2 + fb;
      float4 d4[8];
      uint4 g4[4], u4[4];
#pragma unroll
      for (int i = 0; i < 8; ++i) d4[i] = reinterpret_cast<const float4*>(dhp)[i];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        g4[i] = reinterpret_cast<const uint4*>(gp)[i];
        u4[i] = reinterpret_cast<const uint4*>(gp + F)[i];
      }
      const float* dv = reinterpret_cast<const float*>(d4);
      const uint32_t* gw = reinterpret_cast<const uint32_t*>(g4);
      const uint32_t* uw = reinterpret_cast<const uint32_t*>(u4);
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const uint32_t gb = (j & 1) ? (gw[j >> 1] & 0xffff0000u) : (gw[j >> 1] << 16);
        const uint32_t ub = (j & 1) ? (uw[j >> 1] & 0xffff0000u) : (uw[j >> 1] << 16);
        const float G = __uint_as_float(gb), U = __uint_as_float(ub), dh = dv[j];
        const float sg = __builtin_amdgcn_rcpf(1.f + __expf(-G));
        const float sl = G * sg;
        dps += dh * sl * U;
        du[j] = dh * pr * sl;
        dg[j] = dh * pr * U * sg * (1.f + G * (1.f - sg));
      }
    } else {
#pragma unroll
      for (int j = 0; j < 32; ++j) { dg[j] = 0.f; du[j] = 0.f; }
    }
    // ---- row form: dG at column fb, dU at F + fb
    if (rin && bok) {
      const int64_t o = int64_t(row) * F2 + fb;
      if constexpr (MX) {
        const int64_t so = int64_t(row) * (F2 / 32) + fb / 32;
        store_mx32(dg, p.row_codes + o, p.row_scales + so);
        store_mx32(du, p.row_codes + o + F, p.row_scales + so + F / 32);
      } else {
        store_bf16x32(dg, p.row_bf16 + o);
        store_bf16x32(du, p.row_bf16 + o + F);
      }
    }
    // ---- column form through LDS, dG then dU
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float* src = h == 0 ? dg : du;
      lds_barrier();                         // the previous readers of sv are done
#pragma unroll
      for (int j = 0; j < 32; ++j) sv[sb_at(rl, hh * 32 + j)] = src[j];
      lds_barrier();                         // (stores in flight may stay so)
      const int fc = f0 + c;
      if (fc < F && rr < p.R) {              // R is a multiple of 32: the block's rows exist
        float v[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) v[i] = sv[sb_at(rb * 32 + i, c)];
        const int64_t col = int64_t(h) * F + fc;
        if constexpr (MX)
          store_mx32(v, p.col_codes + col * p.Rp + rr, p.col_scales + col * (p.Rp / 32) + rr / 32);
        else
          store_bf16x32(v, p.col_bf16 + col * p.Rp + rr);
      }
    }
  }
  // ---- d_prob partial of the row over this column group (the two threads of a row are
  // neighbouring lanes)
  dps += __shfl_xor(dps, 1);
  if (hh == 0 && rin) p.dprob_part[int64_t(row) * p.nparts + cg] = dps;
}

mge_status launch_swiglu_bwd(const SwigluBwdParams& p, bool mx, hipStream_t s) {
  if (p.R <= 0) return MGE_OK;
  MGE_REQUIRE(p.nparts == swiglu_bwd_nparts(p.F), "d_prob partial count mismatch");
  dim3 grid((p.R + SB_ROWS - 1) / SB_ROWS, p.nparts);
  ProfScope prof(s, mx ? "swiglu_bwd_mx" : "swiglu_bwd_bf16");
  if (mx)
    hipLaunchKernelGGL(swiglu_bwd_kernel<true>, grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(swiglu_bwd_kernel<false>, grid, dim3(256), 0, s, p);
  return hip_check("swiglu_bwd_kernel");
}

}  // namespace mge
