/*
 * mge.h — C ABI of the MI355X (gfx950) grouped expert MLP library.
 *
 * The routed mixture-of-experts SwiGLU MLP, forward and backward, in BF16 and in
 * MXFP8, as five stream-ordered calls plus helpers:
 *
 *   moe_route_permute   top-k routing, per-expert counts (split_sizes), stable
 *                       permutation of the tokens by expert, gather of x
 *                       (optionally quantized to MXFP8 on load)
 *   mxfp8_quantize      16-bit master weights -> MXFP8 codes + E8M0 scales, in row
 *                       and/or column orientation
 *   grouped_mlp_fwd     grouped gate-up GEMM over all experts in one launch, fused
 *                       SwiGLU x routing probability (+ MXFP8 quantize of h), grouped
 *                       down GEMM
 *   grouped_mlp_bwd     dy permute (+quantize), dh GEMM with fused SwiGLU backward and
 *                       d_prob, dW_down, dX and dW_gate_up grouped GEMMs
 *   unpermute_combine   out[t] = sum over the k slots of in[perm_pos[t][i]]
 * and the router backward (moe_router_bwd: d_logits from d_prob), the forward without
 * the fusion (grouped_mlp_fwd_unfused, the baseline the fusion is measured against) and
 * the one scale of FP8 with one scale per tensor (mge_tensor_scale; the quantizers then
 * take it through their tensor_scale / x_tensor_scale fields).
 *
 * Sources: "NVIDIA Shows an Efficient MoE Training Path for Biological Foundation
 * Models" (sections "Grouped experts instead of a Python loop" and "Memory and
 * quantization overhead"), the BioNeMo recipe report (sections "Fragmented Expert
 * Kernels", "Quantization Overhead") and the ai4snews report (paragraphs on
 * GroupedLinear, on FP8/MXFP8 and on the Sequential fusion).  MXFP8 follows the OCP
 * Microscaling Formats v1.0 specification: E4M3 elements, one E8M0 (power of two)
 * scale per 32 consecutive values along the reduction dimension.
 *
 * Conventions (all calls):
 *   - Every pointer is a device pointer unless marked [host].  The caller allocates
 *     and frees every buffer; the library never allocates device memory.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues work on it and returns; nothing synchronizes except
 *     mge_check_device_errors.  split_sizes stays on the device.
 *   - Arguments are checked on the host first; on a bad argument no kernel is
 *     launched and an error code is returned (details in mge_last_error()).
 *   - bf16 tensors are raw 16-bit patterns (uint16_t).  MXFP8 tensors are a pair:
 *     uint8 E4M3 codes and uint8 E8M0 scales (value 2^(s-127)), one scale per 32
 *     consecutive elements along the stated axis.
 *   - Permuted layout: rows of all experts in expert order; expert e occupies rows
 *     [group_offsets[e], group_offsets[e] + split_sizes[e]); group_offsets are
 *     multiples of `align`; the rows in between are padding (perm_src = -1).  The
 *     total row count is R = mge_perm_rows(T, k, E, align), a multiple of 32.
 *   - "Column form" of a [rows][C] matrix is stored transposed, [C][R], with blocks
 *     of 32 consecutive rows; rows of an expert's 32-row padding hold zeros.  With
 *     align % 32 == 0 no block straddles two experts.  The column form of h written
 *     by the forward's gate-up epilogue covers rows [0, group_offsets[E]) only; those
 *     written by moe_route_permute, the dy permute and the SwiGLU backward (dgu_col)
 *     cover all R rows.
 *   - Limits: 1 <= k <= min(E, 8); 1 <= E <= 256; H and F multiples of 32;
 *     align a power of two in [1, 256]; column forms (training, backward) need
 *     align % 32 == 0.
 *     T = 0 is a no-op.  NaN/Inf inputs give undefined (but memory-safe) results.
 *   - The routing maps the grouped calls take are those moe_route_permute wrote for
 *     the same T, k, E and align.  They stay on the device, where the host cannot
 *     check them, so the kernels bound what they read through them: the grouped GEMMs
 *     clamp each group's span into the R permuted rows, the gathers take a source row
 *     outside [0, T) as zeros, and the combine and the d_prob reduction skip an entry
 *     outside the permuted rows.  Other maps give wrong results, but no access outside
 *     the buffers.
 *   - Calls are thread-safe and re-entrant; each is deterministic, so two identical
 *     calls give bit-identical outputs: no floating-point value is accumulated with
 *     atomics (the only atomics are the integer LDS adds of the routing histogram,
 *     whose counts do not depend on their order).
 */
#ifndef MGE_H
#define MGE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mge_status {
  MGE_OK = 0,
  MGE_ERR_INVALID_ARG = 1,   /* bad size, NULL pointer, misaligned pointer */
  MGE_ERR_UNSUPPORTED = 2,   /* valid request the library does not implement */
  MGE_ERR_WORKSPACE = 3,     /* workspace missing or smaller than the query says */
  MGE_ERR_HIP = 4,           /* a HIP launch failed (hipGetLastError text in mge_last_error) */
  MGE_ERR_DEVICE_CHECK = 5   /* a kernel flagged bad data (see mge_check_device_errors) */
} mge_status;

enum { MGE_PREC_BF16 = 0, MGE_PREC_MXFP8 = 1 };
enum { MGE_DTYPE_BF16 = 0, MGE_DTYPE_F32 = 1 };
enum { MGE_ORIENT_ROW = 1, MGE_ORIENT_COL = 2 };
enum {
  MGE_ROUTE_WANT_COL = 1,     /* also write the column form of the permuted x */
  MGE_ROUTE_PROB_GIVEN = 2    /* topk_idx / topk_prob are inputs (router skipped) */
};

/* Rows of every permuted buffer: T*k + E*(align-1), rounded up to 32. */
int64_t mge_perm_rows(int32_t T, int32_t k, int32_t E, int32_t align);

/* ------------------------------------------------------------------------------
 * moe_route_permute — top-k routing and the stable permutation by expert.
 *
 * Routing (each token is sent to a small number k of the E experts): per token the k
 * largest fp32 logits, ordered by (logit descending, expert index ascending);
 * topk_prob = softmax over the k selected logits (the full softmax renormalised over
 * the top-k).  split_sizes[e] = number of (t, i) with topk_idx[t][i] == e (the
 * per-expert counts the grouped call takes); group_offsets = exclusive prefix sum of
 * split_sizes rounded up to align (E+1 entries).  The row of assignment (t, i) is
 * group_offsets[e] + the number of assignments to e that come before (t, i) in
 * (t, i) order (a stable counting sort, so indices are unique and bit-exact).
 * perm_src[row] = t (-1 on padding), perm_pos[t][i] = row, prob_perm[row] = p (0 on
 * padding).  If x != NULL the permuted x is written: prec BF16 -> x_perm bf16 [R][H];
 * prec MXFP8 -> x_perm u8 codes [R][H] + x_perm_scale u8 [R][H/32] (blocks along H).
 * With MGE_ROUTE_WANT_COL also the column form x_col ([H][R] bf16, or codes [H][R] +
 * x_col_scale [H][R/32]); padding rows are zero in every permuted buffer.
 * With MGE_ROUTE_PROB_GIVEN, logits is ignored and topk_idx/topk_prob are read; an
 * index outside [0, E) sets the device error flag (read by mge_check_device_errors)
 * and is clamped.  A token may name one expert in several slots (given, or after the
 * clamp): each slot is still its own assignment with its own row, in (t, i) order, so
 * perm_src is fully defined (every row in [-1, T)).
 * Workspace: mge_route_workspace_bytes(T, E) bytes, 256-byte aligned.
 * ---------------------------------------------------------------------------- */
typedef struct mge_route_args {
  uint32_t struct_size;      /* sizeof(mge_route_args) */
  int32_t T, E, k, H, align;
  int32_t prec;              /* format of x_perm / x_col */
  uint32_t flags;
  const float* logits;       /* [T][E] */
  const uint16_t* x;         /* [T][H] bf16, or NULL (maps only) */
  int32_t* topk_idx;         /* [T][k] */
  float* topk_prob;          /* [T][k] */
  int32_t* split_sizes;      /* [E] */
  int32_t* group_offsets;    /* [E+1] */
  int32_t* perm_src;         /* [R] */
  int32_t* perm_pos;         /* [T][k] */
  float* prob_perm;          /* [R] */
  void* x_perm;              /* [R][H] bf16 or u8 */
  uint8_t* x_perm_scale;     /* [R][H/32] (MXFP8) */
  void* x_col;               /* [H][R] bf16 or u8 (MGE_ROUTE_WANT_COL) */
  uint8_t* x_col_scale;      /* [H][R/32] (MXFP8, MGE_ROUTE_WANT_COL) */
  void* workspace;
  size_t workspace_bytes;
  /* Added field (a struct_size that ends before it means NULL): optional, MXFP8 only —
   * one E8M0 scale byte for all of x (FP8 with one scale per tensor, e.g. from
   * mge_tensor_scale): every block of x_perm / x_col then takes it, and the scale
   * arrays hold it on every row, padding rows included. */
  const uint8_t* x_tensor_scale;
} mge_route_args;

size_t mge_route_workspace_bytes(int32_t T, int32_t E);
mge_status moe_route_permute(const mge_route_args* args, void* stream);

/* ------------------------------------------------------------------------------
 * moe_route_permute_noalloc — moe_route_permute for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): the same computation, kernels and outputs, with its workspace
 * (the device error flag and the per-block expert counts) in a fixed scratch array
 * the library holds on every GPU it runs on, 1 MiB per GPU, kept until the process
 * ends.  The caller still passes every input and output; args->workspace must be
 * NULL and args->workspace_bytes 0.  Nothing is allocated: no hipMalloc, no hipFree.
 * Limit: mge_route_workspace_bytes(T, E) <= 1 MiB, i.e. 256 + ceil(T/256)*E*4 bytes
 * (each part rounded up to 256): about 8.3 M tokens at E = 8, 262 144 at E = 256.
 * Every call on one GPU shares that GPU's scratch, which keeps the last call's
 * contents (each call clears the flag and rewrites the counts before reading them):
 * calls that overlap on one GPU (two streams, two threads) race and must be
 * serialized by the caller.  The device error flag of an out-of-range given index is
 * not reported (indices are still clamped); check such inputs with
 * moe_route_permute and its workspace.
 * Errors: those of moe_route_permute; MGE_ERR_INVALID_ARG for a workspace given;
 * MGE_ERR_UNSUPPORTED for T, E beyond the scratch (the message gives the sizes);
 * MGE_ERR_HIP if the scratch's device address cannot be obtained.
 * ---------------------------------------------------------------------------- */
mge_status moe_route_permute_noalloc(const mge_route_args* args, void* stream);

/* ------------------------------------------------------------------------------
 * mxfp8_quantize — BF16 -> MXFP8 (E4M3 + E8M0 per 32), the per-step quantization of
 * the 16-bit master weights.
 *
 * in: `batch` matrices of [R][C] bf16; element (b, r, c) at in[b*in_batch_stride +
 * r*in_row_stride + c] (strides in elements).  Per block of 32 values the shared
 * exponent is e = floor(log2(amax)) - 8 clamped to [-127, 127] (all-zero block:
 * -127); scale byte = e + 127; element = E4M3 round-to-nearest-even of v / 2^e,
 * saturating at 448 (OCP MX v1.0).
 * ROW: blocks along C: row_codes [b][R][C], row_scales [b][R][C/32].  Needs C % 32 == 0.
 * COL: blocks along R, stored transposed and K-contiguous: col_codes [b][C][Rp],
 * col_scales [b][C][Rp/32], Rp = R rounded up to 32 (zero padded) — by definition the
 * ROW quantization of the transpose.
 * Errors: MGE_ERR_INVALID_ARG for a struct_size other than the full size or one that ends
 * before an added field, negative sizes, C % 32 != 0, an unknown orientation, missing or
 * misaligned (16-byte) input (NULL allowed when R = 0) / code pointers, strides too small, or num_segments outside
 * [1, 1024] with seg_offsets; MGE_ERR_WORKSPACE for a missing or short workspace with
 * seg_offsets.  batch, C or (without segments) R = 0 is a no-op.
 * ---------------------------------------------------------------------------- */
typedef struct mge_quant_args {
  uint32_t struct_size;
  int32_t batch, R, C;
  int64_t in_batch_stride, in_row_stride;
  const uint16_t* in;
  uint32_t orient;           /* MGE_ORIENT_ROW | MGE_ORIENT_COL */
  uint8_t* row_codes;
  uint8_t* row_scales;
  uint8_t* col_codes;
  uint8_t* col_scales;
  /* Added field (a struct_size that ends before it means NULL): optional [batch] E8M0
   * bytes, one per matrix — FP8 with one scale per tensor: every block of matrix b
   * takes tensor_scale[b] instead of its own, and the scale arrays hold it replicated,
   * so the block-scaled GEMMs read the result unchanged. */
  const uint8_t* tensor_scale;
  /* Added fields (a struct_size that ends before them means no segments): optional
   * segments along R, for tensors already grouped (e.g. by expert) whose groups do not
   * start at multiples of 32.  seg_offsets: device int32 [num_segments + 1], non-decreasing
   * in [0, R] (otherwise undefined but memory-safe results), 1 <= num_segments <= 1024.
   * Segment s (rows seg_offsets[s] .. seg_offsets[s+1]) is placed at a multiple of 32
   * rows, padded with zero rows, in Rs = mge_perm_rows(R, 1, num_segments, 32) output
   * rows: ROW codes [b][Rs][C], scales [b][Rs][C/32]; COL codes [b][C][Rs], scales
   * [b][C][Rs/32], whose 32-row blocks thus restart at every segment.  Rows past the
   * padded segments are zero.  workspace: mge_quant_workspace_bytes(args) bytes. */
  const int32_t* seg_offsets;
  int32_t num_segments;
  void* workspace;
  size_t workspace_bytes;
} mge_quant_args;

size_t mge_quant_workspace_bytes(const mge_quant_args* args);
mge_status mxfp8_quantize(const mge_quant_args* args, void* stream);

/* ------------------------------------------------------------------------------
 * mge_tensor_scale — the one scale of FP8 with one scale per tensor.  The pages name
 * FP8 beside MXFP8 (both 8-bit, MXFP8 adding a scale per block of 32: "NVIDIA Shows
 * an Efficient MoE Training Path ..." section "Memory and quantization overhead"; the
 * ai4snews report's paragraph on FP8/MXFP8) without the FP8 scale rule; this library
 * takes the block rule above with the whole tensor as the block: for each of `batch`
 * bf16 tensors of n elements (tensor b at in + b*batch_stride elements),
 *   scale[b] = clamp(floor(log2(max |v|)) - 8, -127, 127) + 127   (all-zero: 0).
 * Feed it to mxfp8_quantize / moe_route_permute as tensor_scale / x_tensor_scale.
 * Workspace: mge_tensor_scale_workspace_bytes(batch, n).  n = 0 gives scale 0.
 * Errors: MGE_ERR_INVALID_ARG for NULL in/scale (batch > 0), batch outside [0, 65535],
 * n < 0 or batch_stride < n (batch > 1).
 * ---------------------------------------------------------------------------- */
typedef struct mge_tensor_scale_args {
  uint32_t struct_size;
  int32_t batch;
  int64_t n, batch_stride;
  const uint16_t* in;
  uint8_t* scale;                        /* [batch] */
  void* workspace;
  size_t workspace_bytes;
} mge_tensor_scale_args;

size_t mge_tensor_scale_workspace_bytes(int32_t batch, int64_t n);
mge_status mge_tensor_scale(const mge_tensor_scale_args* args, void* stream);

/* ------------------------------------------------------------------------------
 * grouped_mlp_fwd — GroupedLinear(gate_up) -> ScaledSwiGLU -> GroupedLinear(down)
 * over all experts, each projection one persistent grouped launch.
 *
 * Per expert e with rows X_e of the permuted x (split_sizes[e] rows, possibly 0):
 *   [G U] = X_e W_gate_up[e]^T   (W_gate_up[e] is [2F][H]: gate rows 0..F-1, up rows F..2F-1)
 *   h     = p * silu(G) * U      (p = prob_perm of the row; fp32, never stored unquantized)
 *   Y_e   = h W_down[e]^T        (W_down[e] is [H][F])
 * BF16: operands bf16, fp32 accumulate, h rounded to bf16.  MXFP8: x_perm, W_gate_up
 * (blocks along H), h (blocks along F, quantized after the p scaling) and W_down
 * (blocks along F) are MXFP8; fp32 accumulate on block-scaled MFMA.
 * w_gate_up, w_down: [host] arrays of E device pointers (each expert keeps its own
 * weight tensor); *_scale arrays only for MXFP8.
 * Outputs: y_perm [R][H] (bf16 or f32, rows outside the groups untouched); h row form
 * (bf16 [R][F], or codes [R][F] + h_scale [R][F/32]) — if h is NULL it lives in the
 * workspace.  Training (saved_gu != NULL): saved_gu bf16 [R][2F] (G then U) and the
 * column form of h (h_col [F][R] bf16, or codes + h_col_scale [F][R/32]) for dW_down.
 * Workspace: mge_fwd_workspace_bytes(args).
 * ---------------------------------------------------------------------------- */
typedef struct mge_fwd_args {
  uint32_t struct_size;
  int32_t prec, E, H, F, T, k, align;
  const int32_t* split_sizes;
  const int32_t* group_offsets;
  const float* prob_perm;
  const void* x_perm;
  const uint8_t* x_perm_scale;
  const void* const* w_gate_up;          /* [host] E pointers */
  const uint8_t* const* w_gate_up_scale; /* [host] E pointers (MXFP8) */
  const void* const* w_down;             /* [host] E pointers */
  const uint8_t* const* w_down_scale;    /* [host] E pointers (MXFP8) */
  int32_t y_dtype;                       /* MGE_DTYPE_BF16 or MGE_DTYPE_F32 */
  void* y_perm;
  void* h;                               /* optional */
  uint8_t* h_scale;                      /* optional (MXFP8) */
  uint16_t* saved_gu;                    /* training: [R][2F] bf16, else NULL */
  void* h_col;                           /* training */
  uint8_t* h_col_scale;                  /* training, MXFP8 */
  void* workspace;
  size_t workspace_bytes;
} mge_fwd_args;

size_t mge_fwd_workspace_bytes(const mge_fwd_args* args);
mge_status grouped_mlp_fwd(const mge_fwd_args* args, void* stream);

/* ------------------------------------------------------------------------------
 * mge_fwd_saved_bytes — sizes of the activations a training forward saves for the
 * backward.  The fused forward keeps the SwiGLU input and output out of HBM only in
 * part ("some" intermediates are not materialised: the ai4snews report, paragraph on
 * the Sequential fusion); this library saves G and U in bf16 (so the backward does
 * not recompute the gate-up GEMM) and h in column form (the dW_down operand).
 * For prec, T, k, E, F, align as grouped_mlp_fwd takes them (align % 32 == 0), fills
 *   rows        R = mge_perm_rows(T, k, E, align)
 *   saved_gu    bf16 [R][2F]                        (saved_gu)
 *   h_col       MXFP8 codes [F][R] or bf16 [F][R]   (h_col)
 *   h_col_scale E8M0 [F][R/32] (MXFP8), 0 for BF16  (h_col_scale)
 *   total       their sum
 * in bytes.  out->struct_size must be set by the caller.  Pure host arithmetic: no
 * device call.  Errors: MGE_ERR_INVALID_ARG for a NULL or mis-sized out, or for
 * sizes grouped_mlp_fwd's training mode rejects.
 * ---------------------------------------------------------------------------- */
typedef struct mge_fwd_saved_sizes {
  uint32_t struct_size;      /* sizeof(mge_fwd_saved_sizes) */
  int64_t rows;
  size_t saved_gu, h_col, h_col_scale, total;
} mge_fwd_saved_sizes;

mge_status mge_fwd_saved_bytes(int32_t prec, int32_t T, int32_t k, int32_t E, int32_t F, int32_t align,
                               mge_fwd_saved_sizes* out);

/* ------------------------------------------------------------------------------
 * grouped_mlp_fwd_unfused — the same forward without the fusion:
 * the structure the pages' fused GroupedLinear -> ScaledSwiGLU -> GroupedLinear
 * replaces ("Accelerating MoE Training ..." "How it works"; the ai4snews report,
 * paragraph on the Sequential fusion; the BioNeMo recipe report, "Quantization
 * Overhead"), kept to measure what the fusion saves:
 *   1. grouped gate-up GEMM, [G U] written to HBM in bf16 ([R][2F], gate columns
 *      0..F-1, up columns F..2F-1);
 *   2. a standalone SwiGLU x prob kernel: h = p * silu(G) * U in fp32 from the bf16
 *      G, U, rounded to bf16 ([R][F]; rows with p = 0 get 0);
 *   3. MXFP8 only: a standalone quantize of that bf16 h along F (the row form
 *      mxfp8_quantize writes) into h / h_scale, by blocks, or with one scale for all
 *      of h when h_tensor_scale is given;
 *   4. the grouped down GEMM, as in grouped_mlp_fwd.
 * fwd: grouped_mlp_fwd's arguments.  Its workspace fields carry this call's workspace.
 * Training (fwd.saved_gu != NULL; align % 32 == 0): step 1 writes [G U] into saved_gu
 * (the backward's saved G, U; gu must then be NULL or equal to it), and step 3 also
 * writes the column form of the bf16 h into fwd.h_col (+ h_col_scale), with h's one
 * scale when h_tensor_scale is given, by blocks of 32 rows otherwise (BF16: the bf16
 * transpose); it covers all R rows (padding rows zero).
 * gu: optional [R][2F] bf16 output of step 1 (NULL: in the workspace).
 * h_bf16: MXFP8 only, optional [R][F] bf16 output of step 2 (NULL: in the
 * workspace); in BF16 step 2 writes fwd.h (or the workspace) directly.
 * Rows outside the groups: gu untouched, h_bf16 and h zero (MXFP8 codes 0, scales
 * 0 for an all-zero block), y_perm untouched.
 * Errors: those of grouped_mlp_fwd; MGE_ERR_INVALID_ARG for a misaligned gu / h_bf16,
 * or a gu other than saved_gu in training.
 * ---------------------------------------------------------------------------- */
typedef struct mge_fwd_unfused_args {
  uint32_t struct_size;
  mge_fwd_args fwd;
  uint16_t* gu;                          /* optional [R][2F] bf16 */
  uint16_t* h_bf16;                      /* optional [R][F] bf16 (MXFP8) */
  uint8_t* h_tensor_scale;               /* optional (MXFP8): FP8 with one scale per tensor for h —
                                            step 3 first takes h's one scale (as mge_tensor_scale
                                            over [R][F]; padding rows are 0) into this byte, then
                                            quantizes every block of h with it */
} mge_fwd_unfused_args;

size_t mge_fwd_unfused_workspace_bytes(const mge_fwd_unfused_args* args);
mge_status grouped_mlp_fwd_unfused(const mge_fwd_unfused_args* args, void* stream);

/* ------------------------------------------------------------------------------
 * grouped_mlp_bwd — the matching backward of grouped_mlp_fwd (the fused forward comes
 * with a fused backward: "NVIDIA Shows an Efficient MoE Training Path ..." section
 * "Memory and quantization overhead"; the ai4snews report, paragraph on the Sequential
 * fusion), for L = <dy, y> with y = unpermute_combine(y_perm):
 *   dY = dy gathered by perm_src; dh = dY W_down (K = H)
 *   d_prob[t][i] = sum_f dh * silu(G) * U        (row perm_pos[t][i])
 *   dU = dh * p * silu(G);  dG = dh * p * U * silu'(G)   (G, U from saved_gu)
 *   dW_down[e]    = dY_e^T h_e          (K = the expert's tokens)
 *   dX            = [dG dU] W_gate_up   (K = 2F) -> dx_perm; dx = combine(dx_perm)
 *   dW_gate_up[e] = [dG dU]_e^T X_e     (K = the expert's tokens)
 * MXFP8: dY is quantized along H (row form) and along tokens (column form, blocks
 * start at each expert's first row); [dG dU] along 2F and along tokens; the weights
 * come in column form (w_gate_up_col[e]: codes [H][2F] + scales [H][2F/32], i.e.
 * mxfp8_quantize COL of W_gate_up[e]; w_down_col[e]: codes [F][H] + scales [F][H/32]);
 * h_col and x_col are the column forms written by the forward and by
 * moe_route_permute.  BF16: the weights are the bf16 masters (w_gate_up[e] [2F][H],
 * w_down[e] [H][F]); h_col/x_col are the bf16 transposes.
 * Outputs: dx_perm bf16 [R][H] (valid rows), dw_gate_up[e] [2F][H] and dw_down[e]
 * [H][F], fp32 (dw_bf16 = 0, the default) or bf16 (dw_bf16 = 1: rounded to nearest even
 * from the fp32 sums); accumulate != 0 adds to fp32 outputs instead of overwriting and is
 * rejected with bf16 ones; experts with no tokens get zeros; d_prob f32 [T][k].  The intermediates (dY row/col, dGU row/col)
 * go to the optional buffers when given, else to the workspace; dh never leaves the dh
 * GEMM (the SwiGLU backward is its epilogue), and the d_prob partial sums (one per row
 * and 128-column span of F, summed in a fixed order) always live in the workspace.
 * ---------------------------------------------------------------------------- */
typedef struct mge_bwd_args {
  uint32_t struct_size;
  int32_t prec, E, H, F, T, k, align;
  const uint16_t* dy;                    /* [T][H] bf16 */
  const int32_t* split_sizes;
  const int32_t* group_offsets;
  const int32_t* perm_src;
  const int32_t* perm_pos;
  const float* prob_perm;
  const uint16_t* saved_gu;              /* [R][2F] */
  const void* h_col;  const uint8_t* h_col_scale;
  const void* x_col;  const uint8_t* x_col_scale;
  const void* const* w_gate_up;          /* [host] E: MXFP8 col codes [H][2F] / BF16 masters [2F][H] */
  const uint8_t* const* w_gate_up_scale; /* [host] E: [H][2F/32] (MXFP8) */
  const void* const* w_down;             /* [host] E: MXFP8 col codes [F][H] / BF16 masters [H][F] */
  const uint8_t* const* w_down_scale;    /* [host] E: [F][H/32] (MXFP8) */
  uint16_t* dx_perm;                     /* [R][H] bf16 */
  void* const* dw_gate_up;               /* [host] E pointers, [2F][H] f32 (bf16 with dw_bf16) */
  void* const* dw_down;                  /* [host] E pointers, [H][F] f32 (bf16 with dw_bf16) */
  float* d_prob;                         /* [T][k] */
  int32_t accumulate;
  /* optional intermediates (NULL -> workspace) */
  void* dy_row;  uint8_t* dy_row_scale;  /* [R][H] */
  void* dy_col;  uint8_t* dy_col_scale;  /* [H][R] */
  void* dgu_row; uint8_t* dgu_row_scale; /* [R][2F] */
  void* dgu_col; uint8_t* dgu_col_scale; /* [2F][R] */
  void* workspace;
  size_t workspace_bytes;
  /* added after the first version of the struct: a struct_size that ends before it
     means 0 */
  int32_t dw_bf16;                       /* 0: dW in fp32; 1: dW in bf16 (no accumulate) */
  /* Added fields (a struct_size that ends before them means NULL): FP8 with one scale per
   * tensor, MXFP8 only, the two scale pointers together.  dY and [dG dU] then each take
   * one E8M0 scale from their amax (the rule of mge_tensor_scale), written to these
   * bytes, and every block of both their forms is quantized with it (the scale arrays hold
   * it replicated, so the block-scaled GEMMs run unchanged).  A single scale for [dG dU]
   * needs its amax before any code is written, so the SwiGLU backward then writes
   * [dG dU] in bf16 ([R][2F], into dgu_bf16 when given, else the workspace; padding rows
   * zero), a pass takes its amax and a quantize pass writes both forms.  The weights and
   * the column forms of h and x must come quantized the same way (mxfp8_quantize and
   * moe_route_permute with a tensor scale; grouped_mlp_fwd_unfused in training).  The
   * pages name FP8 beside MXFP8 ("NVIDIA Shows an Efficient MoE Training Path ..."
   * section "Memory and quantization overhead"; the ai4snews report's paragraph on
   * FP8/MXFP8) and the recipe trains in either. */
  uint8_t* dy_tensor_scale;              /* [1] written */
  uint8_t* dgu_tensor_scale;             /* [1] written */
  uint16_t* dgu_bf16;                    /* optional [R][2F] bf16 (per-tensor mode only) */
} mge_bwd_args;

size_t mge_bwd_workspace_bytes(const mge_bwd_args* args);
mge_status grouped_mlp_bwd(const mge_bwd_args* args, void* stream);

/* ------------------------------------------------------------------------------
 * unpermute_combine — out[t][:] = sum_{i<k} w[t][i] * in[perm_pos[t][i]][:]
 * (w = 1 when weights == NULL), summed in fp32 in slot order i = 0..k-1, no atomics.
 * It undoes the gather of every expert's tokens that grouped execution starts with
 * ("NVIDIA Shows an Efficient MoE Training Path ..." section "Grouped experts instead
 * of a Python loop"): each token's k expert outputs return to its row and add up.
 * The probability is already applied inside the forward, in the scaled SwiGLU between
 * the two grouped linears (the ai4snews report, paragraph on the Sequential fusion),
 * so the forward's combine is unweighted.
 * Errors: MGE_ERR_INVALID_ARG for T < 0, k outside [1, 8], H not a positive multiple
 * of 32, dtypes other than BF16/F32, or a NULL / misaligned (16-byte) in, out or
 * perm_pos, or in_rows < 0.  Rows of in that no perm_pos entry names are not read; an
 * entry outside [0, in_rows) names no row, and its slot adds nothing (so a caller may
 * drop a slot by setting its entry to -1).
 * ---------------------------------------------------------------------------- */
typedef struct mge_combine_args {
  uint32_t struct_size;
  int32_t T, k, H;
  int32_t in_dtype, out_dtype;           /* MGE_DTYPE_* */
  const void* in;                        /* [in_rows][H] */
  const int32_t* perm_pos;               /* [T][k] */
  const float* weights;                  /* [T][k] or NULL */
  void* out;                             /* [T][H] */
  int64_t in_rows;                       /* rows of in (R for the permuted buffers) */
} mge_combine_args;

mge_status unpermute_combine(const mge_combine_args* args, void* stream);

/* ------------------------------------------------------------------------------
 * moe_router_bwd — gradient of the routing probabilities with respect to the router
 * logits, the step upstream of grouped_mlp_bwd's d_prob.  moe_route_permute gives
 * token t's k slots the softmax of its selected logits (z_i = logits[t][topk_idx[t][i]]),
 * so with s_t = sum_j topk_prob[t][j] * d_prob[t][j] (fp32, slot order):
 *   d_logits[t][e] = sum over the slots i with topk_idx[t][i] == e of
 *                    topk_prob[t][i] * (d_prob[t][i] - s_t)
 * and 0 for the experts no slot selected (the renormalised probabilities do not depend
 * on their logits).  Sources: the routing of "NVIDIA Shows an Efficient MoE Training
 * Path for Biological Foundation Models" (introduction: each token is sent to only a
 * few experts), the routing-probability scaling the fused path folds in (the BioNeMo
 * recipe report, section "Quantization Overhead"; the ai4snews report, paragraph on the
 * Sequential fusion), and the chain rule through that softmax.
 * Layout: topk_idx int32 [T][k], topk_prob and d_prob fp32 [T][k] (as moe_route_permute
 * and grouped_mlp_bwd write them), d_logits fp32 [T][E], every element written.
 * Indices outside [0, E) take part in s_t but add to no output.  T = 0 is a no-op.
 * Errors: MGE_ERR_INVALID_ARG for a NULL pointer (T > 0), E outside [1, 256] or k
 * outside [1, min(E, 8)].
 * ---------------------------------------------------------------------------- */
typedef struct mge_router_bwd_args {
  uint32_t struct_size;
  int32_t T, E, k;
  const int32_t* topk_idx;               /* [T][k] */
  const float* topk_prob;                /* [T][k] */
  const float* d_prob;                   /* [T][k] */
  float* d_logits;                       /* [T][E] */
} mge_router_bwd_args;

mge_status moe_router_bwd(const mge_router_bwd_args* args, void* stream);

/* ------------------------------------------------------------------------------ helpers */
const char* mge_status_string(mge_status s);
/* Detail of the last error on the calling thread ("" if none). */
const char* mge_last_error(void);
/* Synchronizes `stream`, then reads and clears the device error flag kept at the
 * start of a moe_route_permute workspace.  Tests and debugging only. */
mge_status mge_check_device_errors(void* route_workspace, void* stream);
/* Library version, e.g. "0.1.0". */
const char* mge_version(void);

/* ------------------------------------------------------------------------------
 * Per-kernel timing — a measuring aid, not part of the computation (the pages give
 * no per-operator breakdown of the grouped MLP; this provides one).
 * Between mge_profile_start() and mge_profile_stop(), every kernel the library
 * launches, from any thread and on any stream, is bracketed by two HIP events
 * recorded on its own stream.  mge_profile_stop() ends recording, waits for the
 * recorded events, writes up to max_records records (launch order: kernel name and
 * elapsed milliseconds; -1 if an event could not be read, detail in
 * mge_last_error) to out (may be NULL), and returns the number of launches recorded.
 * The events are created once and reused; no device memory is allocated.  Starting
 * again discards the previous records.
 * ---------------------------------------------------------------------------- */
typedef struct mge_kernel_time {
  char name[56];
  float ms;
} mge_kernel_time;

mge_status mge_profile_start(void);
int32_t mge_profile_stop(mge_kernel_time* out, int32_t max_records);

#ifdef __cplusplus
}
#endif

#endif /* MGE_H */
