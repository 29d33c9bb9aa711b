// Kernel parameter blocks and launchers shared between the library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mge.h"

namespace mge {

// ------------------------------------------------------------ per-kernel timing
// While mge_profile_start() is in effect, a ProfScope records a HIP event on the
// launch stream when it is constructed and another when it is destroyed, so each
// kernel launched inside the scope gets its own start/stop pair.  Otherwise it does
// nothing (one relaxed atomic load).
struct ProfScope {
  ProfScope(hipStream_t s, const char* name);
  ~ProfScope();
  ProfScope(const ProfScope&) = delete;
  ProfScope& operator=(const ProfScope&) = delete;
  hipStream_t stream;
  int slot;
};

// ------------------------------------------------------------ block quantize / gather
struct QuantTileParams {
  const uint16_t* in;
  int64_t in_batch_stride, in_row_stride;   // elements
  const int32_t* gather;                    // optional: source row of each output row (-1 = zero row)
  int64_t src_rows;                         // with gather: rows of `in`; a source row outside [0, src_rows) reads as zero
  int batch, R, C, Rp;                      // output rows R (row form), padded rows Rp (column form)
  uint8_t* row_codes;  uint8_t* row_scales;  // MX row form  [b][R][C], [b][R][C/32]
  uint16_t* row_bf16;                        // bf16 row copy [b][R][C]
  uint8_t* col_codes;  uint8_t* col_scales;  // MX column form [b][C][Rp], [b][C][Rp/32]
  uint16_t* col_bf16;                        // bf16 transpose [b][C][Rp]
  const uint8_t* tensor_scale;               // optional [b]: one E8M0 scale per batch entry for every block
};
// timing_name: the launch's name for per-kernel timing (NULL: by form)
mge_status launch_quant_tile(const QuantTileParams& p, bool mx, hipStream_t s, const char* timing_name = nullptr);

// Segmented row map: output row o of the padded order (segment s of input rows
// [seg[s], seg[s+1]) starting at a multiple of 32) -> input row, or -1; S <= SEG_MAX.
constexpr int SEG_MAX = 1024;
mge_status launch_seg_map(const int32_t* seg, int S, int R, int Rp, int32_t* map, hipStream_t s);

// One E8M0 scale per tensor (FP8 with one scale per tensor): amax of each of `batch`
// bf16 tensors of n elements (batch stride bstride elements) -> scale[b] by the block
// rule.  part: tensor_scale_parts(n) * batch floats of workspace.
int tensor_scale_parts(int64_t n);
mge_status launch_tensor_scale(const uint16_t* in, int batch, int64_t n, int64_t bstride, float* part,
                               uint8_t* scale, hipStream_t s);

// E8M0 scales [rows][kb] (kb bytes per row, row stride ld bytes) -> the packed layout
// the GEMM reads: dst[b][j][r] = bytes 4j..4j+3 of row r as one dword (j < ceil(kb/4)).
// Bytes at block index >= kb, or >= *kb_valid/32 when kb_valid is given (a device
// count of valid rows along K: blocks past it hold no data), become 127 (scale 1).
struct ScalePackParams {
  const uint8_t* src;             // batch b at src + b * src_bstride ...
  const uint8_t* const* src_tab;  // ... or at src_tab[b] (device table) when non-NULL
  int64_t src_bstride, ld;
  int batch, rows, kb;
  const int32_t* kb_valid;        // optional
  uint32_t* dst;                  // [batch][ceil(kb/4)][rows]
};
mge_status launch_scale_pack(const ScalePackParams& p, hipStream_t s);
constexpr int SP_MAXD = 8;   // scale packs per batched launch
mge_status launch_scale_pack_batch(const ScalePackParams* list, int n, hipStream_t s);
inline int64_t scale_pack_dwords(int rows, int kb) { return int64_t(rows) * ((kb + 3) / 4); }

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
// moe_route_permute_noalloc's workspace: a fixed device array of kRouteScratchBytes (one
// per GPU); *ptr = its device address on the current device
constexpr size_t kRouteScratchBytes = size_t(1) << 20;
mge_status route_scratch(void** ptr);
mge_status launch_router_bwd(int T, int E, int k, const int32_t* idx, const float* prob, const float* dprob,
                             float* dlogits, hipStream_t s);

// ------------------------------------------------------------ combine / reductions
// entries of perm_pos outside [0, in_rows) add nothing
mge_status launch_combine(int T, int k, int H, int in_dtype, int out_dtype, const void* in, int64_t in_rows,
                          const int32_t* perm_pos, const float* weights, void* out, hipStream_t s);
// h = p * silu(G) * U from the bf16 [G U] rows (stride 2F) into bf16 h [R][F] (the
// unfused forward's standalone SwiGLU x prob; rows with p = 0 get 0)
mge_status launch_swiglu_prob(int R, int F, const uint16_t* gu, const float* prob, uint16_t* h, hipStream_t s);
// rows r of a bf16 [R][C] matrix with perm_src[r] < 0 (padding) set to zero (C % 8 == 0)
mge_status launch_zero_pad_rows(int R, int C, const int32_t* perm_src, uint16_t* m, hipStream_t s);
// d_prob partials per row written by the dh GEMM's SwiGLU-backward epilogue (one per
// 128-column span of F: two per 256-column tile)
inline int dh_swiglu_nparts(int F) { return 2 * ((F + 255) / 256); }
// (an entry of perm_pos outside [0, rows) gives 0)
mge_status launch_dprob_reduce(int T, int k, int nparts, const float* partial, int64_t rows, const int32_t* perm_pos,
                               float* d_prob, hipStream_t s);
// tables[t] (n host pointers each; null tables are skipped) -> dev_table[t * n + i], in as
// few launches as the kernel argument space allows
mge_status launch_upload_tables(const void* const* const* tables, int ntab, int n, void** dev_table, hipStream_t s);

// ------------------------------------------------------------ grouped GEMM
enum GemmMode { RAGGED_M = 0, RAGGED_K = 1 };
enum Epi { EPI_STORE = 0, EPI_SWIGLU = 1, EPI_SWIGLU_BWD = 2 };
// What a plain-store epilogue writes (a kernel template parameter, so that each kernel
// carries one store path): none (SwiGLU), bf16, f32, or f32 added to the output.
enum OutForm { OUT_NONE = 0, OUT_BF16 = 1, OUT_F32 = 2, OUT_F32_ACC = 3 };
// The six GEMMs of the layer; each is its own kernel symbol (traces, per-kernel timing).
enum GemmRole {
  GEMM_GATEUP = 0,      // [G U] = X W_gate_up^T, SwiGLU x p epilogue       (RAGGED_M)
  GEMM_DOWN = 1,        // Y = h W_down^T                                   (RAGGED_M)
  GEMM_DH = 2,          // dh = dY W_down, SwiGLU-backward epilogue           (RAGGED_M)
  GEMM_DX = 3,          // dX = dGU W_gate_up                               (RAGGED_M)
  GEMM_DW_DOWN = 4,     // dW_down = dY^T h                                 (RAGGED_K)
  GEMM_DW_GATEUP = 5,   // dW_gate_up = dGU^T X                             (RAGGED_K)
  GEMM_GATEUP_STORE = 6 // [G U] = X W_gate_up^T stored in bf16 (unfused)  (RAGGED_M)
};

struct GemmParams {
  int role;              // GemmRole
  int mode;              // RAGGED_M: group e = rows [off[e], off[e]+sizes[e]) of A; RAGGED_K: K span of group e
  int E;
  const int32_t* sizes;
  const int32_t* offs;
  int rows;              // R, the permuted rows: every group's span is clamped into [0, R)
  // A: RAGGED_M -> shared [R][K] (row stride lda bytes); RAGGED_K -> shared [M][R] (row stride lda bytes)
  const uint8_t* A;  int64_t lda;
  // B: RAGGED_M -> per-expert table Bt[e] ([N][K], row stride ldb bytes); RAGGED_K -> shared [N][R]
  const uint8_t* const* Bt;
  const uint8_t* B;
  int64_t ldb;
  // MX scales, packed (launch_scale_pack): dword j of a row holds the E8M0 bytes of K
  // blocks 4j..4j+3; the dwords of one j are contiguous over rows.
  //   A: RAGGED_M -> [K/128][R] over the permuted rows (asp_ld = R);
  //      RAGGED_K -> [R/128][M] (asp_ld = M)
  //   B: RAGGED_M -> expert e at Bsp + e*bsp_estride, [K/128][N] (bsp_ld = N);
  //      RAGGED_K -> [R/128][N] (bsp_ld = N)
  const uint32_t* Asp; int64_t asp_ld; uint32_t asp_bytes;
  const uint32_t* Bsp; int64_t bsp_ld, bsp_estride; uint32_t bsp_bytes;
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
  // SwiGLU-backward epilogue (dh GEMM, N = F): G, U from gu_in; dG (columns f) and dU
  // (columns F + f) of [dG dU] in row and column forms; d_prob partial sums
  const uint16_t* gu_in;                                                  // saved [R][2F] bf16
  uint8_t* dgu_row_codes; uint8_t* dgu_row_scales; uint16_t* dgu_row_bf16; // [R][2F], [R][2F/32]
  uint8_t* dgu_col_codes; uint8_t* dgu_col_scales; uint16_t* dgu_col_bf16; // [2F][Rp], [2F][Rp/32]
  float* dprob_part; int dprob_nparts;   // [R][nparts]: one sum per (row, 128-column span of F)
  int tiles_upper;                         // host bound on the number of tiles (grid sizing)
  int group_m;                             // 1: a short last raster band joins the one before
  int band_m;                              // M-tiles per raster band (0: the default, 8)
  int tail_split;                          // plain-store ragged M: tiles past the last whole round go to the tail launch
  int grid_main;                           // workgroups of the main launch (set by the launcher; both launches read it)
};

// Upper bound of tiles for a RAGGED_M GEMM (host-side, from T*k and E).
int gemm_tiles_upper(const GemmParams& p, int64_t total_rows_bound);
mge_status launch_gemm(const GemmParams& p, int prec, hipStream_t s);

}  // namespace mge
