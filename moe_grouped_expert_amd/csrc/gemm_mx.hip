// The grouped-GEMM kernels of the MXFP8 path (block-scaled FP8 MFMA): one symbol per role (and
// output form) so that traces and per-kernel timings tell the GEMMs of a training step
// apart, and each kernel carries only its own epilogue.
#include "gemm_impl.hpp"

namespace mge {

#define MGE_GEMM_KERNEL(name, EPI, MODE, OUT) \
  __global__ __launch_bounds__(G_THREADS, 1) void name(GemmParams p) { gemm_body<true, EPI, MODE, OUT>(p); }

MGE_GEMM_KERNEL(gemm_gateup_swiglu_mx, EPI_SWIGLU, RAGGED_M, OUT_NONE)
MGE_GEMM_KERNEL(gemm_down_mx, EPI_STORE, RAGGED_M, OUT_BF16)
MGE_GEMM_KERNEL(gemm_down_f32_mx, EPI_STORE, RAGGED_M, OUT_F32)
MGE_GEMM_KERNEL(gemm_dh_swiglu_mx, EPI_SWIGLU_BWD, RAGGED_M, OUT_NONE)
MGE_GEMM_KERNEL(gemm_dh_swiglu_bf16out_mx, EPI_SWIGLU_BWD, RAGGED_M, OUT_BF16)   // [dG dU] in bf16
MGE_GEMM_KERNEL(gemm_dx_mx, EPI_STORE, RAGGED_M, OUT_BF16)
MGE_GEMM_KERNEL(gemm_gateup_store_mx, EPI_STORE, RAGGED_M, OUT_BF16)
MGE_GEMM_KERNEL(gemm_dw_down_mx, EPI_STORE, RAGGED_K, OUT_F32)
MGE_GEMM_KERNEL(gemm_dw_down_acc_mx, EPI_STORE, RAGGED_K, OUT_F32_ACC)
MGE_GEMM_KERNEL(gemm_dw_gateup_mx, EPI_STORE, RAGGED_K, OUT_F32)
MGE_GEMM_KERNEL(gemm_dw_gateup_acc_mx, EPI_STORE, RAGGED_K, OUT_F32_ACC)
MGE_GEMM_KERNEL(gemm_dw_down_bf16out_mx, EPI_STORE, RAGGED_K, OUT_BF16)
MGE_GEMM_KERNEL(gemm_dw_gateup_bf16out_mx, EPI_STORE, RAGGED_K, OUT_BF16)

// the quarter-width tail launches of the plain-store ragged-M GEMMs (see gemm_body)
#define MGE_GEMM_TAIL_KERNEL(name, OUT) \
  __global__ __launch_bounds__(G_THREADS, 1) void name(GemmParams p) { gemm_body<true, EPI_STORE, RAGGED_M, OUT, 1>(p); }

MGE_GEMM_TAIL_KERNEL(gemm_down_tail_mx, OUT_BF16)
MGE_GEMM_TAIL_KERNEL(gemm_down_f32_tail_mx, OUT_F32)
MGE_GEMM_TAIL_KERNEL(gemm_dx_tail_mx, OUT_BF16)
MGE_GEMM_TAIL_KERNEL(gemm_gateup_store_tail_mx, OUT_BF16)

#undef MGE_GEMM_TAIL_KERNEL
#undef MGE_GEMM_KERNEL

// Kernel of a role; the output dtype and the accumulate flag were checked by
// launch_gemm (DOWN, DW: bf16 or f32, accumulate only f32; DH: the SwiGLU-backward
// epilogue's outputs, MXFP8 or (out_dtype BF16) bf16; DX, GATEUP_STORE: bf16).
mge_status launch_gemm_mx(const GemmParams& p, hipStream_t s) {
  const bool f32 = p.out_dtype == MGE_DTYPE_F32;
  switch (p.role) {
    case GEMM_GATEUP: return launch_gemm_kernel(gemm_gateup_swiglu_mx, "gemm_gateup_swiglu_mx", p, s);
    case GEMM_DOWN:
      return f32 ? launch_gemm_split(gemm_down_f32_mx, gemm_down_f32_tail_mx, "gemm_down_mx", p, s)
                 : launch_gemm_split(gemm_down_mx, gemm_down_tail_mx, "gemm_down_mx", p, s);
    case GEMM_DH:
      // bf16 [dG dU] (FP8 with one scale per tensor quantizes it afterwards, with its amax)
      return p.out_dtype == MGE_DTYPE_BF16 ? launch_gemm_kernel(gemm_dh_swiglu_bf16out_mx, "gemm_dh_swiglu_bf16out_mx", p, s)
                                           : launch_gemm_kernel(gemm_dh_swiglu_mx, "gemm_dh_swiglu_mx", p, s);
    case GEMM_DX: return launch_gemm_split(gemm_dx_mx, gemm_dx_tail_mx, "gemm_dx_mx", p, s);
    case GEMM_GATEUP_STORE:
      return launch_gemm_split(gemm_gateup_store_mx, gemm_gateup_store_tail_mx, "gemm_gateup_store_mx", p, s);
    case GEMM_DW_DOWN:
      if (!f32) return launch_gemm_kernel(gemm_dw_down_bf16out_mx, "gemm_dw_down_mx", p, s);
      return p.accumulate ? launch_gemm_kernel(gemm_dw_down_acc_mx, "gemm_dw_down_mx", p, s)
                          : launch_gemm_kernel(gemm_dw_down_mx, "gemm_dw_down_mx", p, s);
    case GEMM_DW_GATEUP:
      if (!f32) return launch_gemm_kernel(gemm_dw_gateup_bf16out_mx, "gemm_dw_gateup_mx", p, s);
      return p.accumulate ? launch_gemm_kernel(gemm_dw_gateup_acc_mx, "gemm_dw_gateup_mx", p, s)
                          : launch_gemm_kernel(gemm_dw_gateup_mx, "gemm_dw_gateup_mx", p, s);
  }
  set_error("unknown GEMM role %d", p.role);
  return MGE_ERR_INVALID_ARG;
}

}  // namespace mge
