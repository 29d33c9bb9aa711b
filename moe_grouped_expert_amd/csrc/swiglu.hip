// Standalone SwiGLU x prob of the unfused forward, the structure the fused gate-up
// epilogue replaces ("Accelerating MoE Training ..." [P5], "How it works"; the
// Transformer Engine report [P4], paragraph on the Sequential fusion): the gate-up GEMM
// has written [G U] to HBM in bf16, and this kernel reads it back to form
//   h[r][f] = p[r] * silu(G[r][f]) * U[r][f],  silu(z) = z / (1 + e^-z)   [GLU]
// in fp32, rounded to bf16 (the MXFP8 pipeline then quantizes h in a pass of its own).
// Rows with p = 0 (the padding rows between expert groups, which the GEMM never
// writes) get h = 0 without reading [G U].  HBM-bound: 4 B read and 2 B written per
// (row, ffn column); each thread moves 8 columns as 16-byte loads and one 16-byte store.
#include "mge_common.hpp"
#include "mge_internal.hpp"

namespace mge {

constexpr int SW_THREADS = 256;
typedef uint32_t sw_u32x4 __attribute__((ext_vector_type(4)));
constexpr int64_t SW_MAX_BLOCKS = 8192;

__global__ __launch_bounds__(SW_THREADS) void swiglu_prob_kernel(int R, int F, const uint16_t* __restrict__ gu,
                                                                 const float* __restrict__ prob,
                                                                 uint16_t* __restrict__ h) {
  const int nv = F / 8;
  const int64_t total = int64_t(R) * nv;
  for (int64_t i = int64_t(blockIdx.x) * SW_THREADS + threadIdx.x; i < total;
       i += int64_t(gridDim.x) * SW_THREADS) {
    const int r = int(i / nv);
    const int c = int(i - int64_t(r) * nv) * 8;
    const float p = prob[r];
    uint4 out = make_uint4(0u, 0u, 0u, 0u);
    if (p != 0.f) {
      const uint16_t* row = gu + int64_t(r) * 2 * F;
      // [G U] is read once: non-temporal, so it does not displace other lines in L2
      const sw_u32x4 gv = __builtin_nontemporal_load(reinterpret_cast<const sw_u32x4*>(row + c));
      const sw_u32x4 uv = __builtin_nontemporal_load(reinterpret_cast<const sw_u32x4*>(row + F + c));
      const uint32_t* g = reinterpret_cast<const uint32_t*>(&gv);
      const uint32_t* u = reinterpret_cast<const uint32_t*>(&uv);
      uint32_t* o = reinterpret_cast<uint32_t*>(&out);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float g0 = __uint_as_float(g[j] << 16), g1 = __uint_as_float(g[j] & 0xffff0000u);
        const float u0 = __uint_as_float(u[j] << 16), u1 = __uint_as_float(u[j] & 0xffff0000u);
        o[j] = bf16x2(p * silu_f(g0) * u0, p * silu_f(g1) * u1);
      }
    }
    *reinterpret_cast<uint4*>(h + int64_t(r) * F + c) = out;
  }
}

mge_status launch_swiglu_prob(int R, int F, const uint16_t* gu, const float* prob, uint16_t* h, hipStream_t s) {
  if (R <= 0) return MGE_OK;
  const int64_t total = int64_t(R) * (F / 8);
  int64_t blocks = (total + SW_THREADS - 1) / SW_THREADS;
  if (blocks > SW_MAX_BLOCKS) blocks = SW_MAX_BLOCKS;
  ProfScope prof(s, "swiglu_prob");
  hipLaunchKernelGGL(swiglu_prob_kernel, dim3(unsigned(blocks)), dim3(SW_THREADS), 0, s, R, F, gu, prob, h);
  return hip_check("swiglu_prob_kernel");
}

// Padding rows of a permuted bf16 [R][C] matrix (perm_src[r] < 0, the rows between and
// after the expert groups that no GEMM tile writes) set to zero, so that a pass over all
// R rows (a tensor's amax, the column form's 32-row blocks) reads zeros there.  A
// workgroup per row, grid-stride; rows of the groups are left untouched (one 4-byte read).
__global__ __launch_bounds__(SW_THREADS) void zero_pad_rows_kernel(int R, int C, const int32_t* __restrict__ perm_src,
                                                                   uint16_t* __restrict__ m) {
  for (int r = blockIdx.x; r < R; r += gridDim.x) {
    if (perm_src[r] >= 0) continue;   // uniform over the workgroup
    uint4* row = reinterpret_cast<uint4*>(m + int64_t(r) * C);
    for (int c = threadIdx.x; c < C / 8; c += SW_THREADS) row[c] = make_uint4(0u, 0u, 0u, 0u);
  }
}

mge_status launch_zero_pad_rows(int R, int C, const int32_t* perm_src, uint16_t* m, hipStream_t s) {
  if (R <= 0 || C <= 0) return MGE_OK;
  const int blocks = R < 4096 ? R : 4096;
  ProfScope prof(s, "zero_pad_rows");
  hipLaunchKernelGGL(zero_pad_rows_kernel, dim3(unsigned(blocks)), dim3(SW_THREADS), 0, s, R, C, perm_src, m);
  return hip_check("zero_pad_rows_kernel");
}

}  // namespace mge
