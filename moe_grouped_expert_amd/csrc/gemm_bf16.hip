// The six grouped-GEMM kernels of the BF16 path (BF16 MFMA), one symbol per
// role so that traces and per-kernel timings tell the GEMMs of a training step apart.
#include "gemm_impl.hpp"

namespace mge {

#define MGE_GEMM_KERNEL(name, EPI, MODE) \
  __global__ __launch_bounds__(G_THREADS, 1) void name(GemmParams p) { gemm_body<false, EPI, MODE>(p); }

MGE_GEMM_KERNEL(gemm_gateup_swiglu_bf16, EPI_SWIGLU, RAGGED_M)
MGE_GEMM_KERNEL(gemm_down_bf16, EPI_STORE, RAGGED_M)
MGE_GEMM_KERNEL(gemm_dh_bf16, EPI_STORE, RAGGED_M)
MGE_GEMM_KERNEL(gemm_dx_bf16, EPI_STORE, RAGGED_M)
MGE_GEMM_KERNEL(gemm_dw_down_bf16, EPI_STORE, RAGGED_K)
MGE_GEMM_KERNEL(gemm_dw_gateup_bf16, EPI_STORE, RAGGED_K)

#undef MGE_GEMM_KERNEL

mge_status launch_gemm_bf16(const GemmParams& p, hipStream_t s) {
  switch (p.role) {
    case GEMM_GATEUP: return launch_gemm_kernel(gemm_gateup_swiglu_bf16, "gemm_gateup_swiglu_bf16", p, s);
    case GEMM_DOWN: return launch_gemm_kernel(gemm_down_bf16, "gemm_down_bf16", p, s);
    case GEMM_DH: return launch_gemm_kernel(gemm_dh_bf16, "gemm_dh_bf16", p, s);
    case GEMM_DX: return launch_gemm_kernel(gemm_dx_bf16, "gemm_dx_bf16", p, s);
    case GEMM_DW_DOWN: return launch_gemm_kernel(gemm_dw_down_bf16, "gemm_dw_down_bf16", p, s);
    case GEMM_DW_GATEUP: return launch_gemm_kernel(gemm_dw_gateup_bf16, "gemm_dw_gateup_bf16", p, s);
  }
  set_error("unknown GEMM role %d", p.role);
  return MGE_ERR_INVALID_ARG;
}

}  // namespace mge
