// Host-side driver of the C ABI for the sanitizer build (AddressSanitizer +
// UndefinedBehaviorSanitizer on the host code of the library; no GPU needed).
//
// It runs every entry point's argument checks, the workspace and saved-buffer size
// queries and the T = 0 paths, the parts of the library that are plain host code, with
// inputs at and past the documented limits.  Pointers stand in for device buffers only as
// values that the checks inspect (NULL or not, 16-byte aligned or not): every call here
// returns before a kernel would be launched.  Exit code 0 and "abi_driver ok" when every
// call returned the documented status; any sanitizer report aborts the run.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "../../include/mge.h"

static int g_fail = 0;

#define EXPECT(expr, code)                                                                      \
  do {                                                                                          \
    const int got_ = int(expr);                                                                 \
    if (got_ != int(code)) {                                                                    \
      fprintf(stderr, "%s:%d: %s returned %d, expected %d (%s)\n", __FILE__, __LINE__, #expr, \
              got_, int(code), mge_last_error());                                               \
      ++g_fail;                                                                                 \
    }                                                                                           \
  } while (0)

// Stand-in addresses: aligned and misaligned, never dereferenced by the checks.
static void* const A16 = reinterpret_cast<void*>(uintptr_t(0x10000));
static void* const A8 = reinterpret_cast<void*>(uintptr_t(0x10008));

int main() {
  // ------------------------------------------------------------ helpers
  for (int s = 0; s <= 6; ++s) {
    const char* t = mge_status_string(mge_status(s));
    if (!t || strncmp(t, "MGE_", 4) != 0) ++g_fail;
  }
  if (strlen(mge_version()) < 5) ++g_fail;
  const int32_t Ts[] = {0, 1, 31, 8192, 1 << 20, 1 << 24};
  for (int32_t T : Ts)
    for (int32_t E : {1, 8, 256})
      for (int32_t k : {1, 2, 8})
        for (int32_t al : {1, 32, 256}) {
          const int64_t r = mge_perm_rows(T, k, E, al);
          if (r % 32 != 0 || r < int64_t(T) * k) ++g_fail;
          (void)mge_route_workspace_bytes(T, E);
        }
  (void)mge_route_workspace_bytes(-1, 8);
  (void)mge_tensor_scale_workspace_bytes(3, int64_t(1) << 40);
  (void)mge_tensor_scale_workspace_bytes(-1, 10);

  // ------------------------------------------------------------ saved-buffer sizes
  mge_fwd_saved_sizes sz{};
  sz.struct_size = sizeof(sz);
  EXPECT(mge_fwd_saved_bytes(MGE_PREC_MXFP8, 8192, 2, 8, 14336, 32, &sz), MGE_OK);
  if (sz.total != sz.saved_gu + sz.h_col + sz.h_col_scale || sz.rows != mge_perm_rows(8192, 2, 8, 32)) ++g_fail;
  EXPECT(mge_fwd_saved_bytes(MGE_PREC_BF16, 1 << 24, 8, 256, 1 << 16, 256, &sz), MGE_OK);
  EXPECT(mge_fwd_saved_bytes(MGE_PREC_MXFP8, 10, 2, 8, 48, 32, &sz), MGE_ERR_INVALID_ARG);
  EXPECT(mge_fwd_saved_bytes(MGE_PREC_MXFP8, 10, 9, 8, 64, 32, &sz), MGE_ERR_INVALID_ARG);
  EXPECT(mge_fwd_saved_bytes(MGE_PREC_MXFP8, 10, 2, 8, 64, 8, &sz), MGE_ERR_INVALID_ARG);
  EXPECT(mge_fwd_saved_bytes(MGE_PREC_MXFP8, 10, 2, 8, 64, 32, nullptr), MGE_ERR_INVALID_ARG);

  // ------------------------------------------------------------ moe_route_permute
  EXPECT(moe_route_permute(nullptr, nullptr), MGE_ERR_INVALID_ARG);
  {
    mge_route_args a{};
    a.struct_size = sizeof(a) - 4;
    EXPECT(moe_route_permute(&a, nullptr), MGE_ERR_INVALID_ARG);
    a = mge_route_args{};
    a.struct_size = sizeof(a);
    a.T = 100; a.E = 8; a.k = 2; a.H = 64; a.align = 32; a.prec = MGE_PREC_MXFP8;
    EXPECT(moe_route_permute(&a, nullptr), MGE_ERR_INVALID_ARG);   // logits NULL
    a.logits = static_cast<const float*>(A16);
    a.topk_idx = static_cast<int32_t*>(A16); a.topk_prob = static_cast<float*>(A16);
    a.split_sizes = static_cast<int32_t*>(A16); a.group_offsets = static_cast<int32_t*>(A16);
    a.perm_src = static_cast<int32_t*>(A16); a.perm_pos = static_cast<int32_t*>(A16);
    a.prob_perm = static_cast<float*>(A16);
    EXPECT(moe_route_permute(&a, nullptr), MGE_ERR_WORKSPACE);      // no workspace
    for (int k : {0, 9}) { mge_route_args b = a; b.k = k; EXPECT(moe_route_permute(&b, nullptr), MGE_ERR_INVALID_ARG); }
    for (int E : {0, 257}) { mge_route_args b = a; b.E = E; EXPECT(moe_route_permute(&b, nullptr), MGE_ERR_INVALID_ARG); }
    for (int al : {0, 3, 512}) { mge_route_args b = a; b.align = al; EXPECT(moe_route_permute(&b, nullptr), MGE_ERR_INVALID_ARG); }
    { mge_route_args b = a; b.H = 48; EXPECT(moe_route_permute(&b, nullptr), MGE_ERR_INVALID_ARG); }
    { mge_route_args b = a; b.flags = 0x80; EXPECT(moe_route_permute(&b, nullptr), MGE_ERR_INVALID_ARG); }
    { mge_route_args b = a; b.x = static_cast<const uint16_t*>(A8); EXPECT(moe_route_permute(&b, nullptr), MGE_ERR_INVALID_ARG); }
    { mge_route_args b = a; b.x = static_cast<const uint16_t*>(A16); b.x_perm = A16;
      EXPECT(moe_route_permute(&b, nullptr), MGE_ERR_INVALID_ARG); }   // x_perm_scale NULL
    { mge_route_args b = a; b.x = static_cast<const uint16_t*>(A16); b.x_perm = A16; b.x_perm_scale = static_cast<uint8_t*>(A16);
      b.flags = MGE_ROUTE_WANT_COL; b.x_col = A16; b.x_col_scale = static_cast<uint8_t*>(A16); b.align = 8;
      EXPECT(moe_route_permute(&b, nullptr), MGE_ERR_INVALID_ARG); }   // MXFP8 column form needs align % 32
    // T = 0 with a workspace: a no-op
    std::vector<uint8_t> ws(mge_route_workspace_bytes(0, 8) + 256);
    mge_route_args z = a; z.T = 0; z.workspace = ws.data(); z.workspace_bytes = ws.size();
    EXPECT(moe_route_permute(&z, nullptr), MGE_OK);
  }

  // ------------------------------------------------------------ mxfp8_quantize
  EXPECT(mxfp8_quantize(nullptr, nullptr), MGE_ERR_INVALID_ARG);
  {
    mge_quant_args q{};
    q.struct_size = sizeof(q);
    q.batch = 1; q.R = 64; q.C = 48; q.in_row_stride = 48; q.orient = MGE_ORIENT_ROW;
    q.in = static_cast<const uint16_t*>(A16); q.row_codes = static_cast<uint8_t*>(A16); q.row_scales = static_cast<uint8_t*>(A16);
    EXPECT(mxfp8_quantize(&q, nullptr), MGE_ERR_INVALID_ARG);        // C % 32
    q.C = 64; q.in_row_stride = 64;
    { mge_quant_args b = q; b.orient = 4; EXPECT(mxfp8_quantize(&b, nullptr), MGE_ERR_INVALID_ARG); }
    { mge_quant_args b = q; b.in_row_stride = 32; EXPECT(mxfp8_quantize(&b, nullptr), MGE_ERR_INVALID_ARG); }
    { mge_quant_args b = q; b.in = static_cast<const uint16_t*>(A8); EXPECT(mxfp8_quantize(&b, nullptr), MGE_ERR_INVALID_ARG); }
    { mge_quant_args b = q; b.batch = 2; b.in_batch_stride = 8; EXPECT(mxfp8_quantize(&b, nullptr), MGE_ERR_INVALID_ARG); }
    { mge_quant_args b = q; b.orient = MGE_ORIENT_COL; EXPECT(mxfp8_quantize(&b, nullptr), MGE_ERR_INVALID_ARG); }
    { mge_quant_args b = q; b.R = -1; EXPECT(mxfp8_quantize(&b, nullptr), MGE_ERR_INVALID_ARG); }
    { mge_quant_args b = q; b.R = 0; EXPECT(mxfp8_quantize(&b, nullptr), MGE_OK); }
    { mge_quant_args b = q; b.batch = 0; EXPECT(mxfp8_quantize(&b, nullptr), MGE_OK); }
    { mge_quant_args b = q; b.seg_offsets = static_cast<const int32_t*>(A16); b.num_segments = 0;
      EXPECT(mxfp8_quantize(&b, nullptr), MGE_ERR_INVALID_ARG); }
    { mge_quant_args b = q; b.seg_offsets = static_cast<const int32_t*>(A16); b.num_segments = 4;
      EXPECT(mxfp8_quantize(&b, nullptr), MGE_ERR_WORKSPACE);
      (void)mge_quant_workspace_bytes(&b); }
    { mge_quant_args b = q; b.struct_size = 8; EXPECT(mxfp8_quantize(&b, nullptr), MGE_ERR_INVALID_ARG); }
  }

  // ------------------------------------------------------------ mge_tensor_scale
  EXPECT(mge_tensor_scale(nullptr, nullptr), MGE_ERR_INVALID_ARG);
  {
    mge_tensor_scale_args t{};
    t.struct_size = sizeof(t);
    t.batch = 2; t.n = 100; t.batch_stride = 50;
    t.in = static_cast<const uint16_t*>(A16); t.scale = static_cast<uint8_t*>(A16);
    EXPECT(mge_tensor_scale(&t, nullptr), MGE_ERR_INVALID_ARG);       // batch_stride < n
    t.batch = 70000; t.batch_stride = 100;
    EXPECT(mge_tensor_scale(&t, nullptr), MGE_ERR_INVALID_ARG);
  }

  // ------------------------------------------------------------ grouped_mlp_fwd / _unfused
  const int E = 8;
  std::vector<const void*> wp(E, A16), wp_bad(E, A16);
  std::vector<const uint8_t*> sp(E, static_cast<const uint8_t*>(A16));
  wp_bad[E - 1] = A8;
  EXPECT(grouped_mlp_fwd(nullptr, nullptr), MGE_ERR_INVALID_ARG);
  {
    mge_fwd_args f{};
    f.struct_size = sizeof(f);
    f.prec = MGE_PREC_MXFP8; f.E = E; f.H = 4096; f.F = 14336; f.T = 8192; f.k = 2; f.align = 32;
    f.split_sizes = static_cast<const int32_t*>(A16); f.group_offsets = static_cast<const int32_t*>(A16);
    f.prob_perm = static_cast<const float*>(A16); f.x_perm = A16; f.x_perm_scale = static_cast<const uint8_t*>(A16);
    f.w_gate_up = wp.data(); f.w_down = wp.data(); f.w_gate_up_scale = sp.data(); f.w_down_scale = sp.data();
    f.y_dtype = MGE_DTYPE_BF16; f.y_perm = A16;
    const size_t need = mge_fwd_workspace_bytes(&f);
    if (need == 0) ++g_fail;
    EXPECT(grouped_mlp_fwd(&f, nullptr), MGE_ERR_WORKSPACE);
    { mge_fwd_args b = f; b.w_down = wp_bad.data(); EXPECT(grouped_mlp_fwd(&b, nullptr), MGE_ERR_INVALID_ARG); }
    { mge_fwd_args b = f; b.y_dtype = 7; EXPECT(grouped_mlp_fwd(&b, nullptr), MGE_ERR_INVALID_ARG); }
    { mge_fwd_args b = f; b.F = 100; EXPECT(grouped_mlp_fwd(&b, nullptr), MGE_ERR_INVALID_ARG); }
    { mge_fwd_args b = f; b.saved_gu = static_cast<uint16_t*>(A16); EXPECT(grouped_mlp_fwd(&b, nullptr), MGE_ERR_INVALID_ARG); }
    { mge_fwd_args b = f; b.w_gate_up_scale = nullptr; EXPECT(grouped_mlp_fwd(&b, nullptr), MGE_ERR_INVALID_ARG); }
    { mge_fwd_args b = f; b.struct_size = 4; EXPECT(grouped_mlp_fwd(&b, nullptr), MGE_ERR_INVALID_ARG); }
    // T = 0 with a (host) workspace of the queried size: a no-op
    mge_fwd_args z = f; z.T = 0; z.H = 64; z.F = 64;
    std::vector<uint8_t> ws(mge_fwd_workspace_bytes(&z) + 256);
    z.workspace = ws.data(); z.workspace_bytes = ws.size();
    EXPECT(grouped_mlp_fwd(&z, nullptr), MGE_OK);
    mge_fwd_unfused_args u{};
    u.struct_size = sizeof(u);
    u.fwd = f;
    if (mge_fwd_unfused_workspace_bytes(&u) <= need) ++g_fail;           // [G U] and h in the workspace
    EXPECT(grouped_mlp_fwd_unfused(&u, nullptr), MGE_ERR_WORKSPACE);
    u.fwd.saved_gu = static_cast<uint16_t*>(A16); u.fwd.h_col = A16; u.fwd.h_col_scale = static_cast<uint8_t*>(A16);
    EXPECT(grouped_mlp_fwd_unfused(&u, nullptr), MGE_ERR_WORKSPACE);     // training: [G U] is saved_gu
    { mge_fwd_unfused_args v = u; v.gu = static_cast<uint16_t*>(A16) + 8; EXPECT(grouped_mlp_fwd_unfused(&v, nullptr), MGE_ERR_INVALID_ARG); }
    { mge_fwd_unfused_args v = u; v.fwd.h_col = nullptr; EXPECT(grouped_mlp_fwd_unfused(&v, nullptr), MGE_ERR_INVALID_ARG); }
    { mge_fwd_unfused_args v = u; v.fwd.saved_gu = nullptr; EXPECT(grouped_mlp_fwd_unfused(&v, nullptr), MGE_ERR_INVALID_ARG); }
    EXPECT(grouped_mlp_fwd_unfused(nullptr, nullptr), MGE_ERR_INVALID_ARG);
  }

  // ------------------------------------------------------------ grouped_mlp_bwd
  EXPECT(grouped_mlp_bwd(nullptr, nullptr), MGE_ERR_INVALID_ARG);
  {
    std::vector<void*> dw(E, A16);
    mge_bwd_args b{};
    b.struct_size = sizeof(b);
    b.prec = MGE_PREC_MXFP8; b.E = E; b.H = 4096; b.F = 14336; b.T = 8192; b.k = 2; b.align = 32;
    b.dy = static_cast<const uint16_t*>(A16);
    b.split_sizes = static_cast<const int32_t*>(A16); b.group_offsets = static_cast<const int32_t*>(A16);
    b.perm_src = static_cast<const int32_t*>(A16); b.perm_pos = static_cast<const int32_t*>(A16);
    b.prob_perm = static_cast<const float*>(A16); b.saved_gu = static_cast<const uint16_t*>(A16);
    b.h_col = A16; b.h_col_scale = static_cast<const uint8_t*>(A16); b.x_col = A16; b.x_col_scale = static_cast<const uint8_t*>(A16);
    b.w_gate_up = wp.data(); b.w_down = wp.data(); b.w_gate_up_scale = sp.data(); b.w_down_scale = sp.data();
    b.dx_perm = static_cast<uint16_t*>(A16); b.dw_gate_up = dw.data(); b.dw_down = dw.data(); b.d_prob = static_cast<float*>(A16);
    if (mge_bwd_workspace_bytes(&b) == 0) ++g_fail;
    EXPECT(grouped_mlp_bwd(&b, nullptr), MGE_ERR_WORKSPACE);
    { mge_bwd_args c = b; c.align = 8; EXPECT(grouped_mlp_bwd(&c, nullptr), MGE_ERR_INVALID_ARG); }
    { mge_bwd_args c = b; c.dw_bf16 = 1; c.accumulate = 1; EXPECT(grouped_mlp_bwd(&c, nullptr), MGE_ERR_INVALID_ARG); }
    { mge_bwd_args c = b; c.dw_bf16 = 2; EXPECT(grouped_mlp_bwd(&c, nullptr), MGE_ERR_INVALID_ARG); }
    { mge_bwd_args c = b; c.dgu_row = A8; EXPECT(grouped_mlp_bwd(&c, nullptr), MGE_ERR_INVALID_ARG); }
    { mge_bwd_args c = b; c.w_gate_up = wp_bad.data(); EXPECT(grouped_mlp_bwd(&c, nullptr), MGE_ERR_INVALID_ARG); }
    { mge_bwd_args c = b; c.struct_size = offsetof(mge_bwd_args, dw_bf16); EXPECT(grouped_mlp_bwd(&c, nullptr), MGE_ERR_WORKSPACE); }
    mge_bwd_args z = b; z.T = 0; z.H = 64; z.F = 64;
    std::vector<uint8_t> ws(mge_bwd_workspace_bytes(&z) + 256);
    z.workspace = ws.data(); z.workspace_bytes = ws.size();
    EXPECT(grouped_mlp_bwd(&z, nullptr), MGE_OK);
  }

  // ------------------------------------------------------------ combine / router backward
  EXPECT(unpermute_combine(nullptr, nullptr), MGE_ERR_INVALID_ARG);
  {
    mge_combine_args c{};
    c.struct_size = sizeof(c);
    c.T = 10; c.k = 9; c.H = 64; c.in = A16; c.out = A16; c.perm_pos = static_cast<const int32_t*>(A16);
    EXPECT(unpermute_combine(&c, nullptr), MGE_ERR_INVALID_ARG);
    c.k = 2; c.in_dtype = 5;
    EXPECT(unpermute_combine(&c, nullptr), MGE_ERR_INVALID_ARG);
    c.in_dtype = MGE_DTYPE_BF16; c.out = A8;
    EXPECT(unpermute_combine(&c, nullptr), MGE_ERR_INVALID_ARG);
    c.out = A16; c.in_rows = -1;
    EXPECT(unpermute_combine(&c, nullptr), MGE_ERR_INVALID_ARG);
  }
  EXPECT(moe_router_bwd(nullptr, nullptr), MGE_ERR_INVALID_ARG);
  {
    mge_router_bwd_args r{};
    r.struct_size = sizeof(r);
    r.T = 0; r.E = 8; r.k = 2;
    EXPECT(moe_router_bwd(&r, nullptr), MGE_OK);
    r.T = 5;
    EXPECT(moe_router_bwd(&r, nullptr), MGE_ERR_INVALID_ARG);   // NULL pointers
    r.E = 300;
    EXPECT(moe_router_bwd(&r, nullptr), MGE_ERR_INVALID_ARG);
  }
  EXPECT(mge_check_device_errors(nullptr, nullptr), MGE_ERR_INVALID_ARG);

  if (g_fail) {
    fprintf(stderr, "abi_driver: %d failures\n", g_fail);
    return 1;
  }
  printf("abi_driver ok\n");
  return 0;
}
