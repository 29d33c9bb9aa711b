// The grouped-GEMM kernels of the BF16 path (BF16 MFMA): one symbol per role (and
// output form) so that traces and per-kernel timings tell the GEMMs of a training step
// apart, and each kernel carries only its own epilogue.
#include "gemm_impl.hpp"

namespace mge {

#define MGE_GEMM_KERNEL(name, EPI, MODE, OUT) \
  __global__ __launch_bounds__(G_THREADS, 1) void name(GemmParams p) { gemm_body<false, EPI, MODE, OUT>(p); }

MGE_GEMM_KERNEL(gemm_gateup_swiglu_bf16, EPI_SWIGLU, RAGGED_M, OUT_NONE)
MGE_GEMM_KERNEL(gemm_down_bf16, EPI_STORE, RAGGED_M, OUT_BF16)
MGE_GEMM_KERNEL(gemm_down_f32_bf16, EPI_STORE, RAGGED_M, OUT_F32)
MGE_GEMM_KERNEL(gemm_dh_swiglu_bf16, EPI_SWIGLU_BWD, RAGGED_M, OUT_NONE)
MGE_GEMM_KERNEL(gemm_dx_bf16, EPI_STORE, RAGGED_M, OUT_BF16)
MGE_GEMM_KERNEL(gemm_gateup_store_bf16, EPI_STORE, RAGGED_M, OUT_BF16)
MGE_GEMM_KERNEL(gemm_dw_down_bf16, EPI_STORE, RAGGED_K, OUT_F32)
MGE_GEMM_KERNEL(gemm_dw_down_acc_bf16, EPI_STORE, RAGGED_K, OUT_F32_ACC)
MGE_GEMM_KERNEL(gemm_dw_gateup_bf16, EPI_STORE, RAGGED_K, OUT_F32)
MGE_GEMM_KERNEL(gemm_dw_gateup_acc_bf16, EPI_STORE, RAGGED_K, OUT_F32_ACC)
MGE_GEMM_KERNEL(gemm_dw_down_bf16out_bf16, EPI_STORE, RAGGED_K, OUT_BF16)
MGE_GEMM_KERNEL(gemm_dw_gateup_bf16out_bf16, EPI_STORE, RAGGED_K, OUT_BF16)

// the quarter-width tail launches of the plain-store ragged-M GEMMs (see gemm_body)
#define MGE_GEMM_TAIL_KERNEL(name, OUT) \
  __global__ __launch_bounds__(G_THREADS, 1) void name(GemmParams p) { gemm_body<false, EPI_STORE, RAGGED_M, OUT, 1>(p); }

MGE_GEMM_TAIL_KERNEL(gemm_down_tail_bf16, OUT_BF16)
MGE_GEMM_TAIL_KERNEL(gemm_down_f32_tail_bf16, OUT_F32)
MGE_GEMM_TAIL_KERNEL(gemm_dx_tail_bf16, OUT_BF16)
MGE_GEMM_TAIL_KERNEL(gemm_gateup_store_tail_bf16, OUT_BF16)

#undef MGE_GEMM_TAIL_KERNEL
#undef MGE_GEMM_KERNEL

// Kernel of a role; the output dtype and the accumulate flag were checked by
// launch_gemm (DOWN, DW: bf16 or f32, accumulate only f32; DH: the SwiGLU-backward
// epilogue's outputs; DX, GATEUP_STORE: bf16).
mge_status launch_gemm_bf16(const GemmParams& p, hipStream_t s) {
  const bool f32 = p.out_dtype == MGE_DTYPE_F32;
  switch (p.role) {
    case GEMM_GATEUP: return launch_gemm_kernel(gemm_gateup_swiglu_bf16, "gemm_gateup_swiglu_bf16", p, s);
    case GEMM_DOWN:
      return f32 ? launch_gemm_split(gemm_down_f32_bf16, gemm_down_f32_tail_bf16, "gemm_down_bf16", p, s)
                 : launch_gemm_split(gemm_down_bf16, gemm_down_tail_bf16, "gemm_down_bf16", p, s);
    case GEMM_DH: return launch_gemm_kernel(gemm_dh_swiglu_bf16, "gemm_dh_swiglu_bf16", p, s);
    case GEMM_DX: return launch_gemm_split(gemm_dx_bf16, gemm_dx_tail_bf16, "gemm_dx_bf16", p, s);
    case GEMM_GATEUP_STORE:
      return launch_gemm_split(gemm_gateup_store_bf16, gemm_gateup_store_tail_bf16, "gemm_gateup_store_bf16", p, s);
    case GEMM_DW_DOWN:
      if (!f32) return launch_gemm_kernel(gemm_dw_down_bf16out_bf16, "gemm_dw_down_bf16", p, s);
      return p.accumulate ? launch_gemm_kernel(gemm_dw_down_acc_bf16, "gemm_dw_down_bf16", p, s)
                          : launch_gemm_kernel(gemm_dw_down_bf16, "gemm_dw_down_bf16", p, s);
    case GEMM_DW_GATEUP:
      if (!f32) return launch_gemm_kernel(gemm_dw_gateup_bf16out_bf16, "gemm_dw_gateup_bf16", p, s);
      return p.accumulate ? launch_gemm_kernel(gemm_dw_gateup_acc_bf16, "gemm_dw_gateup_bf16", p, s)
                          : launch_gemm_kernel(gemm_dw_gateup_bf16, "gemm_dw_gateup_bf16", p, s);
  }
  set_error("unknown GEMM role %d", p.role);
  return MGE_ERR_INVALID_ARG;
}

}  // namespace mge
