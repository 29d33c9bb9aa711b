// Host side of the grouped GEMM: tile-count bounds for grid sizing, the checks of a
// role's mode and output form, and the dispatch to the per-precision kernel sets.
#include "gemm_impl.hpp"

namespace mge {

mge_status launch_gemm_mx(const GemmParams& p, hipStream_t s);
mge_status launch_gemm_bf16(const GemmParams& p, hipStream_t s);

int gemm_tiles_upper(const GemmParams& p, int64_t total_rows_bound) {
  int64_t nt = (int64_t(p.N) + G_BN - 1) / G_BN;
  if (p.mode == RAGGED_M) {
    int64_t mt = (total_rows_bound + G_BM - 1) / G_BM + p.E;
    return int(mt * nt);
  }
  int64_t mt = (int64_t(p.M) + G_BM - 1) / G_BM;
  return int(mt * nt * p.E);
}

mge_status launch_gemm(const GemmParams& p, int prec, hipStream_t s) {
  const bool k_mode = p.role == GEMM_DW_DOWN || p.role == GEMM_DW_GATEUP;
  if ((p.mode == RAGGED_K) != k_mode) {
    set_error("GEMM role %d does not match mode %d", p.role, p.mode);
    return MGE_ERR_INVALID_ARG;
  }
  if (p.role == GEMM_DH) {
    // SwiGLU-backward epilogue: N is F; a wave's 128 rows of [G U] and [dG dU] are
    // addressed with 32-bit offsets
    if (p.gu_in == nullptr || p.N != p.F || int64_t(p.F) * 4 * 2 * G_BM >= (int64_t(1) << 31) || p.F % 32 != 0 ||
        p.Rp % 32 != 0 || p.prob == nullptr || p.dprob_part == nullptr || p.dprob_nparts != dh_swiglu_nparts(p.F) ||
        (prec == MGE_PREC_MXFP8 && p.out_dtype != MGE_DTYPE_BF16
             ? (!p.dgu_row_codes || !p.dgu_row_scales || !p.dgu_col_codes || !p.dgu_col_scales)
             : (!p.dgu_row_bf16 || (prec != MGE_PREC_MXFP8 && !p.dgu_col_bf16)))) {
      set_error("dh GEMM with the SwiGLU-backward epilogue: inconsistent parameters (F %d, N %d)", p.F, p.N);
      return MGE_ERR_INVALID_ARG;
    }
  } else if (p.role != GEMM_GATEUP) {
    const bool ok = (p.role == GEMM_DOWN || k_mode) ? (p.out_dtype == MGE_DTYPE_BF16 || p.out_dtype == MGE_DTYPE_F32)
                                                    : p.out_dtype == MGE_DTYPE_BF16;   // DX
    if (!ok || (p.accumulate && (!k_mode || p.out_dtype != MGE_DTYPE_F32))) {
      set_error("GEMM role %d: output dtype %d / accumulate %d not supported", p.role, p.out_dtype, p.accumulate);
      return MGE_ERR_INVALID_ARG;
    }
    // the store epilogue addresses a wave's 128 output rows with 32-bit offsets
    if (int64_t(p.ldc) * 4 * G_BM >= (int64_t(1) << 31)) {
      set_error("GEMM output row stride %lld too large", static_cast<long long>(p.ldc));
      return MGE_ERR_INVALID_ARG;
    }
  } else if (int64_t(p.F) * 4 * 2 * G_BM >= (int64_t(1) << 31)) {
    set_error("F = %d too large for the SwiGLU epilogue", p.F);
    return MGE_ERR_INVALID_ARG;
  }
  return prec == MGE_PREC_MXFP8 ? launch_gemm_mx(p, s) : launch_gemm_bf16(p, s);
}

}  // namespace mge
