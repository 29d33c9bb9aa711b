// Kernel parameter blocks and launchers shared between the library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mge.h"

namespace mge {

// ------------------------------------------------------------ block quantize / gather
struct QuantTileParams {
  const uint16_t* in;
  int64_t in_batch_stride, in_row_stride;   // elements
  const int32_t* gather;                    // optional: source row of each output row (-1 = zero row)
  int batch, R, C, Rp;                      // output rows R (row form), padded rows Rp (column form)
  uint8_t* row_codes;  uint8_t* row_scales;  // MX row form  [b][R][C], [b][R][C/32]
  uint16_t* row_bf16;                        // bf16 row copy [b][R][C]
  uint8_t* col_codes;  uint8_t* col_scales;  // MX column form [b][C][Rp], [b][C][Rp/32]
  uint16_t* col_bf16;                        // bf16 transpose [b][C][Rp]
};
mge_status launch_quant_tile(const QuantTileParams& p, bool mx, hipStream_t s);

// ------------------------------------------------------------ routing / permutation
struct RouteParams {
  int T, E, k, align, nblk, nbits;
  uint32_t flags;
  const float* logits;
  int32_t* topk_idx;
  float* topk_prob;
  int32_t* split_sizes;
  int32_t* group_offsets;
  int32_t* perm_src;
  int32_t* perm_pos;
  float* prob_perm;
  int32_t* err_flag;        // workspace
  int32_t* block_counts;    // workspace [nblk][E]
  int R;
};
mge_status launch_route(const RouteParams& p, hipStream_t s);

// ------------------------------------------------------------ combine / reductions
mge_status launch_combine(int T, int k, int H, int in_dtype, int out_dtype, const void* in,
                          const int32_t* perm_pos, const float* weights, void* out, hipStream_t s);
mge_status launch_dprob_reduce(int T, int k, int nparts, const float* partial, const int32_t* perm_pos,
                               float* d_prob, hipStream_t s);
mge_status launch_upload_ptrs(const void* const* host_ptrs, int n, void** dev_table, hipStream_t s);

// ------------------------------------------------------------ grouped GEMM
enum GemmMode { RAGGED_M = 0, RAGGED_K = 1 };
enum Epi { EPI_STORE = 0, EPI_SWIGLU = 1, EPI_SWIGLU_BWD = 2 };

struct GemmParams {
  int mode;              // RAGGED_M: group e = rows [off[e], off[e]+sizes[e]) of A; RAGGED_K: K span of group e
  int E;
  const int32_t* sizes;
  const int32_t* offs;
  // A: RAGGED_M -> shared [R][K] (row stride lda bytes); RAGGED_K -> shared [M][R] (row stride lda bytes)
  const uint8_t* A;  int64_t lda;
  const uint8_t* As; int64_t ldas;        // MX scales of A (bytes per row)
  // B: RAGGED_M -> per-expert tables Bt[e] ([N][K], row stride ldb bytes); RAGGED_K -> shared [N][R]
  const uint8_t* const* Bt; const uint8_t* const* Bst;
  const uint8_t* B;  const uint8_t* Bs;
  int64_t ldb, ldbs;
  int M, N, K;           // M used in RAGGED_K; K used in RAGGED_M (elements)
  // outputs
  int out_dtype;         // MGE_DTYPE_*
  void* C; int64_t ldc;  // RAGGED_M: shared [R][N]; elements per row
  void* const* Ct;       // RAGGED_K: per-expert outputs [M][N]
  int accumulate;
  // SwiGLU epilogue (forward): N is 2F, tile covers BN/2 columns of gate and of up
  int F;
  const float* prob;                       // prob_perm [R]
  uint8_t* h_codes; uint8_t* h_scales;     // MX h row [R][F], [R][F/32]
  uint16_t* h_bf16;                        // bf16 h row [R][F]
  uint16_t* saved_gu;                      // [R][2F] bf16 (training)
  uint8_t* hc_codes; uint8_t* hc_scales;   // MX h column [F][Rp], [F][Rp/32] (training)
  uint16_t* hc_bf16;                       // bf16 h transpose [F][Rp] (training)
  int Rp;
  // SwiGLU backward epilogue: N is F
  const uint16_t* gu;                      // saved [R][2F]
  uint8_t* dgu_codes; uint8_t* dgu_scales; // MX dGU row [R][2F], [R][2F/32]
  uint16_t* dgu_bf16;                      // bf16 dGU row [R][2F]
  uint8_t* dguc_codes; uint8_t* dguc_scales;  // MX dGU column [2F][Rp], [2F][Rp/32]
  uint16_t* dguc_bf16;                     // bf16 dGU transpose [2F][Rp]
  float* dprob_part; int nparts;           // [R][nparts]
  int tiles_upper;                         // host bound on the number of tiles (grid sizing)
};

// Number of d_prob partial sums per row written by the SwiGLU-backward epilogue.
int gemm_swiglu_bwd_nparts(int F);
// Upper bound of tiles for a RAGGED_M GEMM (host-side, from T*k and E).
int gemm_tiles_upper(const GemmParams& p, int64_t total_rows_bound);
mge_status launch_gemm(const GemmParams& p, int prec, int epi, hipStream_t s);

}  // namespace mge
