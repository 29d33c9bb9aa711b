// C ABI entry points: argument checks, workspace carving and the launch sequence of
// each call.  Every check runs before the first launch; nothing here synchronizes
// except mge_check_device_errors.
#include <cstddef>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <vector>

#include "mge_common.hpp"
#include "mge_internal.hpp"

namespace mge {

static thread_local char g_err[512] = "";

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

mge_status hip_check(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("%s: %s", what, hipGetErrorString(e));
    return MGE_ERR_HIP;
  }
  return MGE_OK;
}

// ------------------------------------------------------------------ per-kernel timing
struct ProfRecord {
  const char* name;
  hipEvent_t start, stop;
};
static std::atomic<bool> g_prof_on{false};
static std::mutex g_prof_mu;
static std::vector<ProfRecord> g_prof_rec;     // this session's launches, in order
static std::vector<hipEvent_t> g_prof_pool;    // events kept for reuse across sessions

static hipEvent_t prof_event() {
  if (!g_prof_pool.empty()) {
    hipEvent_t e = g_prof_pool.back();
    g_prof_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

ProfScope::ProfScope(hipStream_t s, const char* name) : stream(s), slot(-1) {
  if (!g_prof_on.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  ProfRecord r{name, prof_event(), prof_event()};
  if (!r.start || !r.stop) return;
  hipEventRecord(r.start, s);
  slot = int(g_prof_rec.size());
  g_prof_rec.push_back(r);
}

ProfScope::~ProfScope() {
  if (slot < 0) return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (slot < int(g_prof_rec.size())) hipEventRecord(g_prof_rec[slot].stop, stream);
}

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
static bool pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }
static size_t up256(size_t v) { return (v + 255) & ~size_t(255); }

// Gate-up (SwiGLU) GEMM: an expert's M-tile remainder under 4 joins its last raster band.
// Two same-job A/B pairs on the Mixtral-shaped training step: gate-up 1.97 -> 1.93 and
// 2.02 -> 1.95 ms, with 3.61 -> 3.51 GB fetched per launch.  The same rule on dh fetched
// 2.75 -> 3.07 GB for a time change within run-to-run noise, so dh does not use it (the
// weight-gradient GEMMs' band heights are kBandDwDown and kBandDwGateUp below).
constexpr int kMergeShortBand = 1;
// M-tiles per raster band of the weight-gradient GEMMs (the others take 8).  Same-job A/B on
// the Mixtral-shaped training step, each time over the dX GEMM's of the same run (two runs
// of bands 1, 2, 4, 8, 16): dW_down is fastest with 4 (0.62 -> 0.61; 16: 0.69); dW_gate_up
// with 16 by about 1% (1.26 -> 1.25 and 1.24; 1, 2, 4: 1.28-1.34) while its counter traffic
// grows from 3.0 to 4.6 GB per launch, so it keeps 8.
constexpr int kBandDwDown = 4;
constexpr int kBandDwGateUp = 8;

// Bump allocator over the caller's workspace.
struct Carve {
  uint8_t* base;
  size_t used = 0;
  explicit Carve(void* b) : base(static_cast<uint8_t*>(b)) {}
  void* take(size_t bytes) {
    void* p = base ? base + used : nullptr;
    used += up256(bytes);
    return p;
  }
};

static mge_status check_common(int T, int E, int k, int H, int align) {
  MGE_REQUIRE(T >= 0, "T must be >= 0 (got %d)", T);
  MGE_REQUIRE(E >= 1 && E <= 256, "E must be in [1, 256] (got %d)", E);
  MGE_REQUIRE(k >= 1 && k <= 8 && k <= E, "k must be in [1, min(E, 8)] (got k=%d, E=%d)", k, E);
  MGE_REQUIRE(H >= 32 && H % 32 == 0, "H must be a positive multiple of 32 (got %d)", H);
  MGE_REQUIRE(pow2(align) && align <= 256, "align must be a power of two in [1, 256] (got %d)", align);
  return MGE_OK;
}

}  // namespace mge

using namespace mge;

extern "C" {

int64_t mge_perm_rows(int32_t T, int32_t k, int32_t E, int32_t align) {
  int64_t n = int64_t(T) * k + int64_t(E) * (align - 1);
  return (n + 31) / 32 * 32;
}

const char* mge_status_string(mge_status s) {
  switch (s) {
    case MGE_OK: return "MGE_OK";
    case MGE_ERR_INVALID_ARG: return "MGE_ERR_INVALID_ARG";
    case MGE_ERR_UNSUPPORTED: return "MGE_ERR_UNSUPPORTED";
    case MGE_ERR_WORKSPACE: return "MGE_ERR_WORKSPACE";
    case MGE_ERR_HIP: return "MGE_ERR_HIP";
    case MGE_ERR_DEVICE_CHECK: return "MGE_ERR_DEVICE_CHECK";
  }
  return "MGE_ERR_UNKNOWN";
}

const char* mge_last_error(void) { return g_err; }

const char* mge_version(void) { return "0.1.0"; }

mge_status mge_profile_start(void) {
  g_err[0] = 0;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (auto& r : g_prof_rec) {
    g_prof_pool.push_back(r.start);
    g_prof_pool.push_back(r.stop);
  }
  g_prof_rec.clear();
  g_prof_on.store(true);
  return MGE_OK;
}

int32_t mge_profile_stop(mge_kernel_time* out, int32_t max_records) {
  g_err[0] = 0;
  g_prof_on.store(false);
  std::lock_guard<std::mutex> lk(g_prof_mu);
  const int32_t n = int32_t(g_prof_rec.size());
  for (int32_t i = 0; i < n; ++i) {
    ProfRecord& r = g_prof_rec[i];
    float ms = -1.f;
    if (hipEventSynchronize(r.stop) != hipSuccess || hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) {
      set_error("reading the events of launch %d (%s) failed", i, r.name);
      ms = -1.f;
    }
    if (out && i < max_records) {
      snprintf(out[i].name, sizeof(out[i].name), "%s", r.name);
      out[i].ms = ms;
    }
  }
  return n;
}

// ------------------------------------------------------------------ routing
static int route_nblk(int T) { return (T + 255) / 256; }

size_t mge_route_workspace_bytes(int32_t T, int32_t E) {
  if (T < 0 || E < 1) return 0;
  return up256(256) + up256(size_t(route_nblk(T)) * E * sizeof(int32_t));
}

// moe_route_permute with the workspace `ws` of `ws_bytes` (the caller's, or the fixed
// scratch of the no-allocation variant).
static mge_status route_impl(const mge_route_args* a, void* ws_base, size_t ws_bytes, void* stream) {
  // the struct may end before its added last field (x_tensor_scale: then NULL)
  MGE_REQUIRE(a->struct_size == sizeof(mge_route_args) || a->struct_size == offsetof(mge_route_args, x_tensor_scale),
              "struct_size mismatch (%u vs %zu)", a->struct_size, sizeof(mge_route_args));
  const uint8_t* x_ts = a->struct_size == sizeof(mge_route_args) ? a->x_tensor_scale : nullptr;
  MGE_REQUIRE(!x_ts || (a->x && a->prec == MGE_PREC_MXFP8), "x_tensor_scale needs x and prec MXFP8");
  mge_status st = check_common(a->T, a->E, a->k, a->H, a->align);
  if (st != MGE_OK) return st;
  MGE_REQUIRE(a->prec == MGE_PREC_BF16 || a->prec == MGE_PREC_MXFP8, "prec must be BF16 or MXFP8");
  const bool given = (a->flags & MGE_ROUTE_PROB_GIVEN) != 0;
  const bool want_col = (a->flags & MGE_ROUTE_WANT_COL) != 0;
  MGE_REQUIRE((a->flags & ~uint32_t(MGE_ROUTE_PROB_GIVEN | MGE_ROUTE_WANT_COL)) == 0, "unknown flags 0x%x", a->flags);
  MGE_REQUIRE(given || a->logits, "logits is NULL");
  MGE_REQUIRE(a->topk_idx && a->topk_prob && a->split_sizes && a->group_offsets && a->perm_src && a->perm_pos &&
                  a->prob_perm,
              "an output map pointer is NULL");
  if (a->x) {
    MGE_REQUIRE(aligned16(a->x), "x must be 16-byte aligned");
    MGE_REQUIRE(a->x_perm && aligned16(a->x_perm), "x_perm must be non-NULL and 16-byte aligned");
    if (a->prec == MGE_PREC_MXFP8) MGE_REQUIRE(a->x_perm_scale, "x_perm_scale is NULL");
    if (want_col) {
      MGE_REQUIRE(a->x_col && aligned16(a->x_col), "x_col must be non-NULL and 16-byte aligned");
      if (a->prec == MGE_PREC_MXFP8) {
        MGE_REQUIRE(a->x_col_scale, "x_col_scale is NULL");
        MGE_REQUIRE(a->align % 32 == 0, "the MXFP8 column form needs align %% 32 == 0 (got %d)", a->align);
      }
    }
  }
  const size_t need = mge_route_workspace_bytes(a->T, a->E);
  if (!ws_base || ws_bytes < need) {
    set_error("route workspace needs %zu bytes (got %zu)", need, ws_bytes);
    return MGE_ERR_WORKSPACE;
  }
  if (a->T == 0) return MGE_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int R = int(mge_perm_rows(a->T, a->k, a->E, a->align));
  Carve ws(ws_base);
  RouteParams p{};
  p.T = a->T; p.E = a->E; p.k = a->k; p.align = a->align;
  p.nblk = route_nblk(a->T);
  int nb = 1;
  while ((1 << nb) <= a->E) ++nb;   // bits to tell the E experts and the sentinel E apart
  p.nbits = nb;
  p.flags = a->flags;
  p.logits = a->logits;
  p.topk_idx = a->topk_idx; p.topk_prob = a->topk_prob;
  p.split_sizes = a->split_sizes; p.group_offsets = a->group_offsets;
  p.perm_src = a->perm_src; p.perm_pos = a->perm_pos; p.prob_perm = a->prob_perm;
  p.err_flag = static_cast<int32_t*>(ws.take(256));
  p.block_counts = static_cast<int32_t*>(ws.take(size_t(p.nblk) * a->E * 4));
  p.R = R;
  st = launch_route(p, s);
  if (st != MGE_OK || !a->x) return st;
  QuantTileParams q{};
  q.in = a->x; q.in_batch_stride = 0; q.in_row_stride = a->H;
  q.gather = a->perm_src; q.src_rows = a->T;
  q.batch = 1; q.R = R; q.C = a->H; q.Rp = R;
  q.tensor_scale = x_ts;
  if (a->prec == MGE_PREC_MXFP8) {
    q.row_codes = static_cast<uint8_t*>(a->x_perm);
    q.row_scales = a->x_perm_scale;
    if (want_col) { q.col_codes = static_cast<uint8_t*>(a->x_col); q.col_scales = a->x_col_scale; }
  } else {
    q.row_bf16 = static_cast<uint16_t*>(a->x_perm);
    if (want_col) q.col_bf16 = static_cast<uint16_t*>(a->x_col);
  }
  return launch_quant_tile(q, a->prec == MGE_PREC_MXFP8, s);
}

mge_status moe_route_permute(const mge_route_args* a, void* stream) {
  g_err[0] = 0;
  MGE_REQUIRE(a != nullptr, "args is NULL");
  return route_impl(a, a->struct_size >= offsetof(mge_route_args, x_tensor_scale) ? a->workspace : nullptr,
                    a->struct_size >= offsetof(mge_route_args, x_tensor_scale) ? a->workspace_bytes : 0, stream);
}

mge_status moe_route_permute_noalloc(const mge_route_args* a, void* stream) {
  g_err[0] = 0;
  MGE_REQUIRE(a != nullptr, "args is NULL");
  MGE_REQUIRE(a->struct_size >= offsetof(mge_route_args, x_tensor_scale), "struct_size mismatch");
  MGE_REQUIRE(a->workspace == nullptr && a->workspace_bytes == 0,
              "moe_route_permute_noalloc takes no workspace (workspace NULL, workspace_bytes 0)");
  const mge_status chk = check_common(a->T, a->E, a->k, a->H, a->align);
  if (chk != MGE_OK) return chk;
  const size_t need = mge_route_workspace_bytes(a->T, a->E);
  if (need > kRouteScratchBytes) {
    set_error("moe_route_permute_noalloc: T=%d, E=%d need %zu bytes of scratch, above its fixed %zu "
              "(256 + ceil(T/256)*E*4, rounded to 256, must fit); use moe_route_permute with a workspace",
              a->T, a->E, need, kRouteScratchBytes);
    return MGE_ERR_UNSUPPORTED;
  }
  void* ws = nullptr;
  const mge_status st = route_scratch(&ws);
  if (st != MGE_OK) return st;
  return route_impl(a, ws, kRouteScratchBytes, stream);
}

// ------------------------------------------------------------------ quantize
mge_status mxfp8_quantize(const mge_quant_args* a, void* stream) {
  g_err[0] = 0;
  MGE_REQUIRE(a != nullptr, "args is NULL");
  // the struct may end before its added fields (tensor_scale; the segments): then absent
  MGE_REQUIRE(a->struct_size == sizeof(mge_quant_args) || a->struct_size == offsetof(mge_quant_args, tensor_scale) ||
                  a->struct_size == offsetof(mge_quant_args, seg_offsets),
              "struct_size mismatch");
  const uint8_t* ts = a->struct_size > offsetof(mge_quant_args, tensor_scale) ? a->tensor_scale : nullptr;
  const bool seg = a->struct_size == sizeof(mge_quant_args) && a->seg_offsets != nullptr;
  if (seg) {
    MGE_REQUIRE(a->num_segments >= 1 && a->num_segments <= SEG_MAX, "num_segments must be in [1, %d] (got %d)",
                SEG_MAX, a->num_segments);
    const size_t need = mge_quant_workspace_bytes(a);
    if (!a->workspace || a->workspace_bytes < need) {
      set_error("segmented quantize workspace needs %zu bytes (got %zu)", need, a->workspace_bytes);
      return MGE_ERR_WORKSPACE;
    }
  }
  MGE_REQUIRE(a->batch >= 0 && a->R >= 0 && a->C >= 0, "negative size");
  MGE_REQUIRE(a->C % 32 == 0, "C must be a multiple of 32 (got %d)", a->C);
  MGE_REQUIRE(a->orient != 0 && (a->orient & ~3u) == 0, "orient must be ROW, COL or ROW|COL");
  MGE_REQUIRE((a->in || a->R == 0 || a->batch == 0) && aligned16(a->in), "in must be non-NULL (R > 0) and 16-byte aligned");
  MGE_REQUIRE(a->in_row_stride >= a->C && a->in_row_stride % 8 == 0, "in_row_stride must be >= C and a multiple of 8");
  MGE_REQUIRE(a->batch <= 1 || (a->in_batch_stride % 8 == 0 && a->in_batch_stride >= int64_t(a->R) * a->in_row_stride),
              "in_batch_stride too small or not a multiple of 8");
  if (a->orient & MGE_ORIENT_ROW)
    MGE_REQUIRE(a->row_codes && a->row_scales && aligned16(a->row_codes), "row outputs missing or misaligned");
  if (a->orient & MGE_ORIENT_COL)
    MGE_REQUIRE(a->col_codes && a->col_scales && aligned16(a->col_codes), "column outputs missing or misaligned");
  if (a->batch == 0 || a->C == 0 || (a->R == 0 && !seg)) return MGE_OK;
  if (seg) MGE_REQUIRE(a->R < (1 << 30), "R too large for segments");
  hipStream_t s = static_cast<hipStream_t>(stream);
  QuantTileParams q{};
  q.in = a->in; q.in_batch_stride = a->in_batch_stride; q.in_row_stride = a->in_row_stride;
  q.batch = a->batch; q.R = a->R; q.C = a->C; q.Rp = (a->R + 31) / 32 * 32;
  if (seg) {   // rows in the padded segment order: gathered through the row map
    const int Rs = int(mge_perm_rows(a->R, 1, a->num_segments, 32));
    int32_t* map = static_cast<int32_t*>(a->workspace);
    const mge_status st = launch_seg_map(a->seg_offsets, a->num_segments, a->R, Rs, map, s);
    if (st != MGE_OK) return st;
    q.gather = map; q.src_rows = a->R;
    q.R = Rs; q.Rp = Rs;
  }
  if (a->orient & MGE_ORIENT_ROW) { q.row_codes = a->row_codes; q.row_scales = a->row_scales; }
  if (a->orient & MGE_ORIENT_COL) { q.col_codes = a->col_codes; q.col_scales = a->col_scales; }
  q.tensor_scale = ts;
  return launch_quant_tile(q, true, s);
}

size_t mge_quant_workspace_bytes(const mge_quant_args* a) {
  if (!a || a->struct_size != sizeof(mge_quant_args) || !a->seg_offsets || a->R < 0 || a->num_segments < 1) return 0;
  return up256(size_t(mge_perm_rows(a->R, 1, a->num_segments, 32)) * sizeof(int32_t));
}

// ------------------------------------------------------------------ per-tensor scale
size_t mge_tensor_scale_workspace_bytes(int32_t batch, int64_t n) {
  if (batch < 0 || n < 0) return 0;
  return up256(size_t(tensor_scale_parts(n)) * size_t(batch) * sizeof(float));
}

mge_status mge_tensor_scale(const mge_tensor_scale_args* a, void* stream) {
  g_err[0] = 0;
  MGE_REQUIRE(a != nullptr, "args is NULL");
  MGE_REQUIRE(a->struct_size == sizeof(mge_tensor_scale_args), "struct_size mismatch");
  MGE_REQUIRE(a->batch >= 0 && a->batch <= 65535, "batch must be in [0, 65535] (got %d)", a->batch);
  MGE_REQUIRE(a->n >= 0, "n must be >= 0");
  MGE_REQUIRE(a->batch <= 1 || a->batch_stride >= a->n, "batch_stride must be >= n");
  if (a->batch == 0) return MGE_OK;
  MGE_REQUIRE(a->in && a->scale, "in / scale is NULL");
  const size_t need = mge_tensor_scale_workspace_bytes(a->batch, a->n);
  if (!a->workspace || a->workspace_bytes < need) {
    set_error("tensor-scale workspace needs %zu bytes (got %zu)", need, a->workspace_bytes);
    return MGE_ERR_WORKSPACE;
  }
  return launch_tensor_scale(a->in, a->batch, a->n, a->batch_stride, static_cast<float*>(a->workspace), a->scale,
                             static_cast<hipStream_t>(stream));
}

// ------------------------------------------------------------------ forward
static mge_status check_mlp_dims(int prec, int E, int H, int F, int T, int k, int align) {
  mge_status st = check_common(T, E, k, H, align);
  if (st != MGE_OK) return st;
  MGE_REQUIRE(prec == MGE_PREC_BF16 || prec == MGE_PREC_MXFP8, "prec must be BF16 or MXFP8");
  MGE_REQUIRE(F >= 32 && F % 32 == 0, "F must be a positive multiple of 32 (got %d)", F);
  return MGE_OK;
}

// Bytes of a packed scale matrix (launch_scale_pack) of `batch` x [rows][kb]: exact, and
// rounded up for carving the workspace.
static uint32_t packed_exact(int batch, int rows, int kb) { return uint32_t(int64_t(batch) * scale_pack_dwords(rows, kb) * 4); }
static size_t packed_bytes(int batch, int rows, int kb) { return up256(packed_exact(batch, rows, kb)); }

static size_t fwd_ws(const mge_fwd_args* a, int R) {
  size_t n = up256(4 * size_t(a->E) * sizeof(void*));
  const bool mx = a->prec == MGE_PREC_MXFP8;
  if (!a->h) {
    if (mx) n += up256(size_t(R) * a->F) + up256(size_t(R) * (a->F / 32));
    else n += up256(size_t(R) * a->F * 2);
  }
  if (mx) {
    n += packed_bytes(1, R, a->H / 32) + packed_bytes(a->E, 2 * a->F, a->H / 32);
    n += packed_bytes(1, R, a->F / 32) + packed_bytes(a->E, a->H, a->F / 32);
  }
  return n;
}

// Every operand the GEMMs address with 32-bit buffer offsets must stay below 2^31 bytes.
static mge_status check_offsets(int R, int H, int F, int elem) {
  const int64_t lim = int64_t(1) << 31;
  const int64_t big = int64_t(R) * 2 * F * elem;            // [R][2F] and [2F][R] forms
  const int64_t w = int64_t(2) * F * H * elem;               // one expert's W_gate_up
  MGE_REQUIRE(big < lim && w < lim && int64_t(R) * H * elem < lim,
              "operand too large for 32-bit offsets (R=%d H=%d F=%d)", R, H, F);
  return MGE_OK;
}

// The unfused forward's extra buffers: [G U] bf16, and in MXFP8 the bf16 h before its
// quantize pass (in BF16 h itself is the bf16 h, counted by fwd_ws).
static size_t fwd_unfused_extra(const mge_fwd_unfused_args* u, int R) {
  const mge_fwd_args* a = &u->fwd;
  size_t n = 0;
  if (!u->gu && !a->saved_gu) n += up256(size_t(R) * 2 * a->F * 2);   // training: [G U] is saved_gu
  if (a->prec == MGE_PREC_MXFP8 && !u->h_bf16) n += up256(size_t(R) * a->F * 2);
  if (u->h_tensor_scale) n += up256(size_t(tensor_scale_parts(int64_t(R) * a->F)) * sizeof(float));
  return n;
}

mge_status mge_fwd_saved_bytes(int32_t prec, int32_t T, int32_t k, int32_t E, int32_t F, int32_t align,
                               mge_fwd_saved_sizes* out) {
  g_err[0] = 0;
  MGE_REQUIRE(out != nullptr, "out is NULL");
  MGE_REQUIRE(out->struct_size == sizeof(mge_fwd_saved_sizes), "struct_size mismatch");
  MGE_REQUIRE(prec == MGE_PREC_BF16 || prec == MGE_PREC_MXFP8, "prec must be BF16 or MXFP8");
  MGE_REQUIRE(T >= 0, "T must be >= 0 (got %d)", T);
  MGE_REQUIRE(E >= 1 && E <= 256, "E must be in [1, 256] (got %d)", E);
  MGE_REQUIRE(k >= 1 && k <= 8 && k <= E, "k must be in [1, min(E, 8)] (got k=%d, E=%d)", k, E);
  MGE_REQUIRE(F >= 32 && F % 32 == 0, "F must be a positive multiple of 32 (got %d)", F);
  MGE_REQUIRE(pow2(align) && align <= 256 && align % 32 == 0, "training needs align a power of two in [32, 256] (got %d)",
              align);
  const size_t R = size_t(mge_perm_rows(T, k, E, align));
  const bool mx = prec == MGE_PREC_MXFP8;
  out->rows = int64_t(R);
  out->saved_gu = R * 2 * size_t(F) * 2;
  out->h_col = size_t(F) * R * (mx ? 1 : 2);
  out->h_col_scale = mx ? size_t(F) * (R / 32) : 0;
  out->total = out->saved_gu + out->h_col + out->h_col_scale;
  return MGE_OK;
}

size_t mge_fwd_workspace_bytes(const mge_fwd_args* a) {
  if (!a || a->E < 1 || a->T < 0 || a->k < 1 || a->align < 1) return 0;
  return fwd_ws(a, int(mge_perm_rows(a->T, a->k, a->E, a->align)));
}

size_t mge_fwd_unfused_workspace_bytes(const mge_fwd_unfused_args* u) {
  if (!u) return 0;
  const mge_fwd_args* a = &u->fwd;
  if (a->E < 1 || a->T < 0 || a->k < 1 || a->align < 1) return 0;
  const int R = int(mge_perm_rows(a->T, a->k, a->E, a->align));
  return fwd_ws(a, R) + fwd_unfused_extra(u, R);
}

// The forward, fused (u == NULL) or unfused (u != NULL, a == &u->fwd).
static mge_status fwd_impl(const mge_fwd_args* a, const mge_fwd_unfused_args* u, void* stream) {
  MGE_REQUIRE(a->struct_size == sizeof(mge_fwd_args), "struct_size mismatch");
  mge_status st = check_mlp_dims(a->prec, a->E, a->H, a->F, a->T, a->k, a->align);
  if (st != MGE_OK) return st;
  const bool mx = a->prec == MGE_PREC_MXFP8;
  const bool train = a->saved_gu != nullptr;
  MGE_REQUIRE(a->split_sizes && a->group_offsets && a->prob_perm, "split_sizes / group_offsets / prob_perm NULL");
  MGE_REQUIRE(a->x_perm && aligned16(a->x_perm), "x_perm must be non-NULL and 16-byte aligned");
  MGE_REQUIRE(!mx || a->x_perm_scale, "x_perm_scale is NULL");
  MGE_REQUIRE(a->w_gate_up && a->w_down, "weight pointer arrays are NULL");
  MGE_REQUIRE(!mx || (a->w_gate_up_scale && a->w_down_scale), "weight scale pointer arrays are NULL");
  for (int e = 0; e < a->E; ++e) {
    MGE_REQUIRE(a->w_gate_up[e] && aligned16(a->w_gate_up[e]), "w_gate_up[%d] NULL or misaligned", e);
    MGE_REQUIRE(a->w_down[e] && aligned16(a->w_down[e]), "w_down[%d] NULL or misaligned", e);
    if (mx) MGE_REQUIRE(a->w_gate_up_scale[e] && a->w_down_scale[e], "weight scales of expert %d NULL", e);
  }
  MGE_REQUIRE(a->y_dtype == MGE_DTYPE_BF16 || a->y_dtype == MGE_DTYPE_F32, "y_dtype must be BF16 or F32");
  MGE_REQUIRE(a->y_perm && aligned16(a->y_perm), "y_perm must be non-NULL and 16-byte aligned");
  if (a->h) MGE_REQUIRE(aligned16(a->h) && (!mx || a->h_scale), "h misaligned or h_scale NULL");
  if (train) {
    MGE_REQUIRE(a->h_col && aligned16(a->h_col), "training needs h_col (16-byte aligned)");
    MGE_REQUIRE(!mx || a->h_col_scale, "h_col_scale is NULL");
    MGE_REQUIRE(a->align % 32 == 0, "training (column form of h) needs align %% 32 == 0 (got %d)", a->align);
  }
  if (u) {
    MGE_REQUIRE(!train || !u->gu || u->gu == a->saved_gu, "training: gu must be NULL or saved_gu ([G U] is saved)");
    MGE_REQUIRE(train || (!a->h_col && !a->h_col_scale), "h_col / h_col_scale without saved_gu");
    MGE_REQUIRE(!train || aligned16(a->saved_gu), "saved_gu must be 16-byte aligned");
    MGE_REQUIRE((!u->gu || aligned16(u->gu)) && (!u->h_bf16 || aligned16(u->h_bf16)), "gu / h_bf16 misaligned");
    MGE_REQUIRE(!u->h_tensor_scale || mx, "h_tensor_scale needs prec MXFP8");
  }
  const int R = int(mge_perm_rows(a->T, a->k, a->E, a->align));
  const size_t need = fwd_ws(a, R) + (u ? fwd_unfused_extra(u, R) : 0);
  if (!a->workspace || a->workspace_bytes < need) {
    set_error("forward workspace needs %zu bytes (got %zu)", need, a->workspace_bytes);
    return MGE_ERR_WORKSPACE;
  }
  if (a->T == 0) return MGE_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Carve ws(a->workspace);
  void** tab = static_cast<void**>(ws.take(4 * size_t(a->E) * sizeof(void*)));
  void* h = a->h;
  uint8_t* hs = a->h_scale;
  if (!h) {
    if (mx) { h = ws.take(size_t(R) * a->F); hs = static_cast<uint8_t*>(ws.take(size_t(R) * (a->F / 32))); }
    else h = ws.take(size_t(R) * a->F * 2);
  }
  uint16_t* gu = nullptr;     // unfused: [G U] bf16 and (MXFP8) the bf16 h
  uint16_t* hb = nullptr;
  if (u) {
    gu = train ? a->saved_gu : u->gu ? u->gu : static_cast<uint16_t*>(ws.take(size_t(R) * 2 * a->F * 2));
    hb = !mx ? static_cast<uint16_t*>(h) : u->h_bf16 ? u->h_bf16 : static_cast<uint16_t*>(ws.take(size_t(R) * a->F * 2));
  }
  float* h_amax_part = (u && u->h_tensor_scale)
                           ? static_cast<float*>(ws.take(size_t(tensor_scale_parts(int64_t(R) * a->F)) * sizeof(float)))
                           : nullptr;
  const int E = a->E;
  {
    const void* const* tabs[4] = {reinterpret_cast<const void* const*>(a->w_gate_up),
                                  reinterpret_cast<const void* const*>(a->w_down),
                                  mx ? reinterpret_cast<const void* const*>(a->w_gate_up_scale) : nullptr,
                                  mx ? reinterpret_cast<const void* const*>(a->w_down_scale) : nullptr};
    st = launch_upload_tables(tabs, 4, E, tab, s);
    if (st != MGE_OK) return st;
  }
  const int64_t rows_bound = int64_t(a->T) * a->k;
  const int elem = mx ? 1 : 2;
  st = check_offsets(R, a->H, a->F, elem);
  if (st != MGE_OK) return st;
  const int H = a->H, F = a->F;
  uint32_t *xs_p = nullptr, *wgu_p = nullptr, *hs_p = nullptr, *wd_p = nullptr;
  if (mx) {
    xs_p = static_cast<uint32_t*>(ws.take(packed_bytes(1, R, H / 32)));
    wgu_p = static_cast<uint32_t*>(ws.take(packed_bytes(E, 2 * F, H / 32)));
    hs_p = static_cast<uint32_t*>(ws.take(packed_bytes(1, R, F / 32)));
    wd_p = static_cast<uint32_t*>(ws.take(packed_bytes(E, H, F / 32)));
    ScalePackParams pk[3] = {};
    pk[0].src = a->x_perm_scale; pk[0].ld = H / 32; pk[0].batch = 1; pk[0].rows = R; pk[0].kb = H / 32; pk[0].dst = xs_p;
    pk[1].src_tab = reinterpret_cast<const uint8_t* const*>(tab + 2 * E); pk[1].ld = H / 32;
    pk[1].batch = E; pk[1].rows = 2 * F; pk[1].kb = H / 32; pk[1].dst = wgu_p;
    pk[2].src_tab = reinterpret_cast<const uint8_t* const*>(tab + 3 * E); pk[2].ld = F / 32;
    pk[2].batch = E; pk[2].rows = H; pk[2].kb = F / 32; pk[2].dst = wd_p;
    st = launch_scale_pack_batch(pk, 3, s);   // one launch for the three
    if (st != MGE_OK) return st;
  }

  GemmParams g{};
  g.mode = RAGGED_M; g.E = E; g.sizes = a->split_sizes; g.offs = a->group_offsets; g.rows = R;
  g.A = static_cast<const uint8_t*>(a->x_perm); g.lda = int64_t(a->H) * elem;
  g.Asp = xs_p; g.asp_ld = R; g.asp_bytes = packed_exact(1, R, H / 32);
  g.Bt = reinterpret_cast<const uint8_t* const*>(tab);
  g.Bsp = wgu_p; g.bsp_ld = 2 * F; g.bsp_estride = scale_pack_dwords(2 * F, H / 32);
  g.bsp_bytes = packed_exact(E, 2 * F, H / 32);
  g.ldb = int64_t(a->H) * elem;
  g.N = 2 * a->F; g.K = a->H; g.F = a->F;
  g.prob = a->prob_perm;
  if (mx) { g.h_codes = static_cast<uint8_t*>(h); g.h_scales = hs; }
  else g.h_bf16 = static_cast<uint16_t*>(h);
  if (train && !u) {
    g.saved_gu = a->saved_gu;
    if (mx) { g.hc_codes = static_cast<uint8_t*>(a->h_col); g.hc_scales = a->h_col_scale; }
    else g.hc_bf16 = static_cast<uint16_t*>(a->h_col);
  }
  g.Rp = R;
  if (!u) {
    g.tiles_upper = gemm_tiles_upper(g, rows_bound);
    g.role = GEMM_GATEUP;
    g.group_m = kMergeShortBand;
    st = launch_gemm(g, a->prec, s);
    if (st != MGE_OK) return st;
  } else {
    // [G U] to HBM in bf16, then SwiGLU x p, then (MXFP8) the quantize of h
    g.h_codes = nullptr; g.h_scales = nullptr; g.h_bf16 = nullptr;
    g.out_dtype = MGE_DTYPE_BF16; g.C = gu; g.ldc = 2 * int64_t(F);
    g.tiles_upper = gemm_tiles_upper(g, rows_bound);
    g.role = GEMM_GATEUP_STORE;
    st = launch_gemm(g, a->prec, s);
    if (st != MGE_OK) return st;
    st = launch_swiglu_prob(R, F, gu, a->prob_perm, hb, s);
    if (st != MGE_OK) return st;
    if (mx) {
      QuantTileParams q{};
      q.in = hb; q.in_batch_stride = int64_t(R) * F; q.in_row_stride = F;
      q.batch = 1; q.R = R; q.C = F; q.Rp = R;
      q.row_codes = static_cast<uint8_t*>(h); q.row_scales = hs;
      if (train) { q.col_codes = static_cast<uint8_t*>(a->h_col); q.col_scales = a->h_col_scale; }
      if (u->h_tensor_scale) {   // one scale for all of h: its amax first
        st = launch_tensor_scale(hb, 1, int64_t(R) * F, 0, h_amax_part, u->h_tensor_scale, s);
        if (st != MGE_OK) return st;
        q.tensor_scale = u->h_tensor_scale;
      }
      st = launch_quant_tile(q, true, s, "quant_h_mx");
      if (st != MGE_OK) return st;
    } else if (train) {   // BF16 training: the transpose of h
      QuantTileParams q{};
      q.in = hb; q.in_row_stride = F;
      q.batch = 1; q.R = R; q.C = F; q.Rp = R;
      q.col_bf16 = static_cast<uint16_t*>(a->h_col);
      st = launch_quant_tile(q, false, s, "transpose_h_bf16");
      if (st != MGE_OK) return st;
    }
  }
  if (mx) {
    ScalePackParams q{};
    q.src = hs; q.ld = F / 32; q.batch = 1; q.rows = R; q.kb = F / 32; q.dst = hs_p;
    st = launch_scale_pack(q, s);
    if (st != MGE_OK) return st;
  }

  GemmParams d{};
  d.mode = RAGGED_M; d.E = E; d.sizes = a->split_sizes; d.offs = a->group_offsets; d.rows = R;
  d.A = static_cast<const uint8_t*>(h); d.lda = int64_t(a->F) * elem;
  d.Asp = hs_p; d.asp_ld = R; d.asp_bytes = packed_exact(1, R, F / 32);
  d.Bt = reinterpret_cast<const uint8_t* const*>(tab + E);
  d.Bsp = wd_p; d.bsp_ld = H; d.bsp_estride = scale_pack_dwords(H, F / 32);
  d.bsp_bytes = packed_exact(E, H, F / 32);
  d.ldb = int64_t(a->F) * elem;
  d.N = a->H; d.K = a->F;
  d.out_dtype = a->y_dtype; d.C = a->y_perm; d.ldc = a->H;
  d.tiles_upper = gemm_tiles_upper(d, rows_bound);
  d.role = GEMM_DOWN;
  return launch_gemm(d, a->prec, s);
}

mge_status grouped_mlp_fwd(const mge_fwd_args* a, void* stream) {
  g_err[0] = 0;
  MGE_REQUIRE(a != nullptr, "args is NULL");
  return fwd_impl(a, nullptr, stream);
}

mge_status grouped_mlp_fwd_unfused(const mge_fwd_unfused_args* u, void* stream) {
  g_err[0] = 0;
  MGE_REQUIRE(u != nullptr, "args is NULL");
  MGE_REQUIRE(u->struct_size == sizeof(mge_fwd_unfused_args), "struct_size mismatch");
  return fwd_impl(&u->fwd, u, stream);
}

// ------------------------------------------------------------------ backward
// The added per-tensor fields of mge_bwd_args, NULL when the struct ends before them.
struct BwdTensorScale {
  uint8_t* dy = nullptr;
  uint8_t* dgu = nullptr;
  uint16_t* dgu_bf16 = nullptr;
};
static BwdTensorScale bwd_tensor_scale(const mge_bwd_args* a) {
  BwdTensorScale t;
  if (a->struct_size == sizeof(mge_bwd_args)) {
    t.dy = a->dy_tensor_scale;
    t.dgu = a->dgu_tensor_scale;
    t.dgu_bf16 = a->dgu_bf16;
  }
  return t;
}

static size_t bwd_ws(const mge_bwd_args* a, int R) {
  const bool mx = a->prec == MGE_PREC_MXFP8;
  const size_t H = a->H, F = a->F, E = a->E, F2 = 2 * F;
  size_t n = up256(6 * E * sizeof(void*));
  const BwdTensorScale ts = bwd_tensor_scale(a);
  if (ts.dy) {   // per-tensor scales: the amax partials, and [dG dU] in bf16 unless given
    const int parts = std::max(tensor_scale_parts(int64_t(a->T) * a->H), tensor_scale_parts(int64_t(R) * F2));
    n += up256(size_t(parts) * sizeof(float));
    if (!ts.dgu_bf16) n += up256(size_t(R) * F2 * 2);
  }
  n += up256(size_t(R) * dh_swiglu_nparts(int(F)) * sizeof(float));   // d_prob partials per permuted row
  auto mat = [&](size_t rows, size_t cols) {
    return mx ? up256(rows * cols) + up256(rows * (cols / 32)) : up256(rows * cols * 2);
  };
  if (!a->dy_row) n += mat(R, H);
  if (!a->dy_col) n += mat(H, R);
  if (!a->dgu_row) n += mat(R, F2);
  if (!a->dgu_col) n += mat(F2, R);
  if (!mx) n += E * (up256(F * H * 2) + up256(H * F2 * 2));   // bf16 transposed weights
  if (mx) {
    const int r = R, h = int(H), f = int(F), f2 = int(F2), e = int(E);
    n += packed_bytes(1, r, h / 32) + packed_bytes(e, f, h / 32);      // dh GEMM: dY row, W_down col
    n += packed_bytes(1, h, r / 32) + packed_bytes(1, f, r / 32);      // dW_down: dY col, h col
    n += packed_bytes(1, r, f2 / 32) + packed_bytes(e, h, f2 / 32);    // dX: dGU row, W_gate_up col
    n += packed_bytes(1, f2, r / 32) + packed_bytes(1, h, r / 32);     // dW_gate_up: dGU col, x col
  }
  return n;
}

size_t mge_bwd_workspace_bytes(const mge_bwd_args* a) {
  if (!a || a->E < 1 || a->T < 0 || a->k < 1 || a->align < 1 || a->F < 32) return 0;
  return bwd_ws(a, int(mge_perm_rows(a->T, a->k, a->E, a->align)));
}

mge_status grouped_mlp_bwd(const mge_bwd_args* a, void* stream) {
  g_err[0] = 0;
  MGE_REQUIRE(a != nullptr, "args is NULL");
  // earlier versions of the struct ended before dw_bf16, and before the per-tensor fields
  MGE_REQUIRE(a->struct_size == sizeof(mge_bwd_args) || a->struct_size == offsetof(mge_bwd_args, dy_tensor_scale) ||
                  a->struct_size == offsetof(mge_bwd_args, dw_bf16),
              "struct_size mismatch");
  const bool has_dw_bf16 = a->struct_size > offsetof(mge_bwd_args, dw_bf16);
  const bool dw_bf16 = has_dw_bf16 && a->dw_bf16 != 0;
  MGE_REQUIRE(!has_dw_bf16 || a->dw_bf16 == 0 || a->dw_bf16 == 1, "dw_bf16 must be 0 or 1 (got %d)", a->dw_bf16);
  const BwdTensorScale tsc = bwd_tensor_scale(a);
  const bool per_tensor = tsc.dy != nullptr;
  MGE_REQUIRE((tsc.dy == nullptr) == (tsc.dgu == nullptr), "dy_tensor_scale and dgu_tensor_scale go together");
  MGE_REQUIRE(!per_tensor || a->prec == MGE_PREC_MXFP8, "per-tensor scales need prec MXFP8");
  MGE_REQUIRE(!tsc.dgu_bf16 || (per_tensor && aligned16(tsc.dgu_bf16)),
              "dgu_bf16 only with per-tensor scales, 16-byte aligned");
  MGE_REQUIRE(!(dw_bf16 && a->accumulate), "accumulate needs fp32 dW outputs");
  mge_status st = check_mlp_dims(a->prec, a->E, a->H, a->F, a->T, a->k, a->align);
  if (st != MGE_OK) return st;
  const bool mx = a->prec == MGE_PREC_MXFP8;
  MGE_REQUIRE(a->align % 32 == 0, "the backward (column forms along tokens) needs align %% 32 == 0 (got %d)",
              a->align);
  MGE_REQUIRE(a->dy && aligned16(a->dy), "dy must be non-NULL and 16-byte aligned");
  MGE_REQUIRE(a->split_sizes && a->group_offsets && a->perm_src && a->perm_pos && a->prob_perm,
              "routing maps are NULL");
  MGE_REQUIRE(a->saved_gu, "saved_gu is NULL");
  MGE_REQUIRE(a->h_col && aligned16(a->h_col) && a->x_col && aligned16(a->x_col), "h_col / x_col NULL or misaligned");
  MGE_REQUIRE(!mx || (a->h_col_scale && a->x_col_scale), "h_col_scale / x_col_scale NULL");
  MGE_REQUIRE(a->w_gate_up && a->w_down, "weight pointer arrays are NULL");
  MGE_REQUIRE(!mx || (a->w_gate_up_scale && a->w_down_scale), "weight scale arrays are NULL");
  MGE_REQUIRE(a->dw_gate_up && a->dw_down, "dW pointer arrays are NULL");
  for (int e = 0; e < a->E; ++e) {
    MGE_REQUIRE(a->w_gate_up[e] && aligned16(a->w_gate_up[e]), "w_gate_up[%d] NULL or misaligned", e);
    MGE_REQUIRE(a->w_down[e] && aligned16(a->w_down[e]), "w_down[%d] NULL or misaligned", e);
    if (mx) MGE_REQUIRE(a->w_gate_up_scale[e] && a->w_down_scale[e], "weight scales of expert %d NULL", e);
    MGE_REQUIRE(a->dw_gate_up[e] && a->dw_down[e], "dW outputs of expert %d NULL", e);
  }
  MGE_REQUIRE(a->dx_perm && aligned16(a->dx_perm) && a->d_prob, "dx_perm / d_prob NULL or misaligned");
  auto opt_ok = [&](void* c, uint8_t* s) { return !c || (aligned16(c) && (!mx || s)); };
  MGE_REQUIRE(opt_ok(a->dy_row, a->dy_row_scale) && opt_ok(a->dy_col, a->dy_col_scale) &&
                  opt_ok(a->dgu_row, a->dgu_row_scale) && opt_ok(a->dgu_col, a->dgu_col_scale),
              "an optional intermediate is misaligned or lacks its scales");
  const int R = int(mge_perm_rows(a->T, a->k, a->E, a->align));
  const size_t need = bwd_ws(a, R);
  if (!a->workspace || a->workspace_bytes < need) {
    set_error("backward workspace needs %zu bytes (got %zu)", need, a->workspace_bytes);
    return MGE_ERR_WORKSPACE;
  }
  if (a->T == 0) return MGE_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int E = a->E, H = a->H, F = a->F, F2 = 2 * F;
  const int elem = mx ? 1 : 2;
  Carve ws(a->workspace);
  void** tab = static_cast<void**>(ws.take(6 * size_t(E) * sizeof(void*)));
  const int nparts = dh_swiglu_nparts(a->F);
  float* dprob_part = static_cast<float*>(ws.take(size_t(R) * nparts * sizeof(float)));
  auto mat = [&](void* given, uint8_t* given_s, size_t rows, size_t cols, void** c, uint8_t** sc) {
    if (given) { *c = given; *sc = given_s; return; }
    if (mx) { *c = ws.take(rows * cols); *sc = static_cast<uint8_t*>(ws.take(rows * (cols / 32))); }
    else { *c = ws.take(rows * cols * 2); *sc = nullptr; }
  };
  float* ts_part = nullptr;   // per-tensor mode: amax partials, and [dG dU] in bf16
  uint16_t* dgu_b = nullptr;
  if (per_tensor) {
    const int parts = std::max(tensor_scale_parts(int64_t(a->T) * H), tensor_scale_parts(int64_t(R) * F2));
    ts_part = static_cast<float*>(ws.take(size_t(parts) * sizeof(float)));
    dgu_b = tsc.dgu_bf16 ? tsc.dgu_bf16 : static_cast<uint16_t*>(ws.take(size_t(R) * F2 * 2));
  }
  void *dyr, *dyc, *dgr, *dgc;
  uint8_t *dyrs, *dycs, *dgrs, *dgcs;
  mat(a->dy_row, a->dy_row_scale, R, H, &dyr, &dyrs);
  mat(a->dy_col, a->dy_col_scale, H, R, &dyc, &dycs);
  mat(a->dgu_row, a->dgu_row_scale, R, F2, &dgr, &dgrs);
  mat(a->dgu_col, a->dgu_col_scale, F2, R, &dgc, &dgcs);

  // weights in the K-contiguous orientation each GEMM reads
  const void* const* wd_k;     // [F][H] per expert (dh GEMM)
  const void* const* wgu_k;    // [H][2F] per expert (dX GEMM)
  std::vector<const void*> wd_t, wgu_t;
  if (mx) {
    wd_k = a->w_down;
    wgu_k = a->w_gate_up;
  } else {
    wd_t.resize(E); wgu_t.resize(E);
    for (int e = 0; e < E; ++e) {
      uint16_t* t1 = static_cast<uint16_t*>(ws.take(size_t(F) * H * 2));
      uint16_t* t2 = static_cast<uint16_t*>(ws.take(size_t(H) * F2 * 2));
      QuantTileParams q{};
      q.in = static_cast<const uint16_t*>(a->w_down[e]); q.in_row_stride = F;
      q.batch = 1; q.R = H; q.C = F; q.Rp = H; q.col_bf16 = t1;
      st = launch_quant_tile(q, false, s);
      if (st != MGE_OK) return st;
      QuantTileParams q2{};
      q2.in = static_cast<const uint16_t*>(a->w_gate_up[e]); q2.in_row_stride = H;
      q2.batch = 1; q2.R = F2; q2.C = H; q2.Rp = F2; q2.col_bf16 = t2;
      st = launch_quant_tile(q2, false, s);
      if (st != MGE_OK) return st;
      wd_t[e] = t1; wgu_t[e] = t2;
    }
    wd_k = wd_t.data();
    wgu_k = wgu_t.data();
  }
  {
    const void* const* tabs[6] = {wd_k, wgu_k,
                                  mx ? reinterpret_cast<const void* const*>(a->w_down_scale) : nullptr,
                                  mx ? reinterpret_cast<const void* const*>(a->w_gate_up_scale) : nullptr,
                                  reinterpret_cast<const void* const*>(a->dw_down),
                                  reinterpret_cast<const void* const*>(a->dw_gate_up)};
    st = launch_upload_tables(tabs, 6, E, tab, s);
    if (st != MGE_OK) return st;
  }

  // b1: dy gathered by perm_src, row form (along H) and column form (along tokens)
  {
    QuantTileParams q{};
    q.in = a->dy; q.in_row_stride = H; q.gather = a->perm_src; q.src_rows = a->T;
    q.batch = 1; q.R = R; q.C = H; q.Rp = R;
    if (per_tensor) {   // dy's one scale (its amax over [T][H] is the permuted dY's)
      st = launch_tensor_scale(a->dy, 1, int64_t(a->T) * H, 0, ts_part, tsc.dy, s);
      if (st != MGE_OK) return st;
      q.tensor_scale = tsc.dy;
    }
    if (mx) { q.row_codes = static_cast<uint8_t*>(dyr); q.row_scales = dyrs; q.col_codes = static_cast<uint8_t*>(dyc); q.col_scales = dycs; }
    else { q.row_bf16 = static_cast<uint16_t*>(dyr); q.col_bf16 = static_cast<uint16_t*>(dyc); }
    st = launch_quant_tile(q, mx, s);
    if (st != MGE_OK) return st;
  }
  const int64_t rows_bound = int64_t(a->T) * a->k;
  st = check_offsets(R, H, F, elem);
  if (st != MGE_OK) return st;
  // packed scales of every MX operand (the GEMMs read one dword per row and K slice)
  uint32_t *dyr_p = nullptr, *wdc_p = nullptr, *dyc_p = nullptr, *hc_p = nullptr;
  uint32_t *dgr_p = nullptr, *wguc_p = nullptr, *dgc_p = nullptr, *xc_p = nullptr;
  // the scale packs available at one point of the call go out as one launch
  ScalePackParams packs[SP_MAXD];
  int npacks = 0;
  auto pack = [&](const uint8_t* src, const uint8_t* const* src_tab, int batch, int rows, int kb,
                  const int32_t* kb_valid, uint32_t* dst) {
    ScalePackParams q{};
    q.src = src; q.src_tab = src_tab; q.ld = kb; q.batch = batch; q.rows = rows; q.kb = kb;
    q.kb_valid = kb_valid; q.dst = dst;
    packs[npacks++] = q;
  };
  auto flush_packs = [&]() {
    const mge_status r = launch_scale_pack_batch(packs, npacks, s);
    npacks = 0;
    return r;
  };
  const int32_t* rows_written = a->group_offsets + E;   // column forms from epilogues end here
  if (mx) {
    dyr_p = static_cast<uint32_t*>(ws.take(packed_bytes(1, R, H / 32)));
    wdc_p = static_cast<uint32_t*>(ws.take(packed_bytes(E, F, H / 32)));
    dyc_p = static_cast<uint32_t*>(ws.take(packed_bytes(1, H, R / 32)));
    hc_p = static_cast<uint32_t*>(ws.take(packed_bytes(1, F, R / 32)));
    dgr_p = static_cast<uint32_t*>(ws.take(packed_bytes(1, R, F2 / 32)));
    wguc_p = static_cast<uint32_t*>(ws.take(packed_bytes(E, H, F2 / 32)));
    dgc_p = static_cast<uint32_t*>(ws.take(packed_bytes(1, F2, R / 32)));
    xc_p = static_cast<uint32_t*>(ws.take(packed_bytes(1, H, R / 32)));
    pack(dyrs, nullptr, 1, R, H / 32, nullptr, dyr_p);
    pack(nullptr, reinterpret_cast<const uint8_t* const*>(tab + 2 * E), E, F, H / 32, nullptr, wdc_p);
    pack(dycs, nullptr, 1, H, R / 32, nullptr, dyc_p);
    pack(a->h_col_scale, nullptr, 1, F, R / 32, rows_written, hc_p);
    pack(nullptr, reinterpret_cast<const uint8_t* const*>(tab + 3 * E), E, H, F2 / 32, nullptr, wguc_p);
    pack(a->x_col_scale, nullptr, 1, H, R / 32, nullptr, xc_p);
    st = flush_packs();
    if (st != MGE_OK) return st;
  }
  // b2: dh = dY W_down, with the SwiGLU backward as the GEMM's epilogue (the saved G, U
  // and p): dGU in row and column forms and the d_prob partial row sums
  {
    GemmParams g{};
    g.mode = RAGGED_M; g.E = E; g.sizes = a->split_sizes; g.offs = a->group_offsets; g.rows = R;
    g.A = static_cast<const uint8_t*>(dyr); g.lda = int64_t(H) * elem; g.Asp = dyr_p; g.asp_ld = R; g.asp_bytes = packed_exact(1, R, H / 32);
    g.Bt = reinterpret_cast<const uint8_t* const*>(tab);
    g.Bsp = wdc_p; g.bsp_ld = F; g.bsp_estride = scale_pack_dwords(F, H / 32);
    g.bsp_bytes = packed_exact(E, F, H / 32);
    g.ldb = int64_t(H) * elem;
    g.N = F; g.K = H; g.F = F; g.Rp = R;
    g.out_dtype = MGE_DTYPE_F32;
    g.prob = a->prob_perm;
    g.gu_in = a->saved_gu;
    if (per_tensor) {   // [dG dU] in bf16, row form only; quantized below with its one scale
      g.out_dtype = MGE_DTYPE_BF16;
      g.dgu_row_bf16 = dgu_b;
    } else if (mx) {
      g.dgu_row_codes = static_cast<uint8_t*>(dgr); g.dgu_row_scales = dgrs;
      g.dgu_col_codes = static_cast<uint8_t*>(dgc); g.dgu_col_scales = dgcs;
    } else {
      g.dgu_row_bf16 = static_cast<uint16_t*>(dgr); g.dgu_col_bf16 = static_cast<uint16_t*>(dgc);
    }
    g.dprob_part = dprob_part; g.dprob_nparts = nparts;
    g.tiles_upper = gemm_tiles_upper(g, rows_bound);
    g.role = GEMM_DH;
    st = launch_gemm(g, a->prec, s);
    if (st != MGE_OK) return st;
  }
  if (per_tensor) {
    // padding rows to zero, the one scale of [dG dU], then both forms with it
    st = launch_zero_pad_rows(R, F2, a->perm_src, dgu_b, s);
    if (st != MGE_OK) return st;
    st = launch_tensor_scale(dgu_b, 1, int64_t(R) * F2, 0, ts_part, tsc.dgu, s);
    if (st != MGE_OK) return st;
    QuantTileParams q{};
    q.in = dgu_b; q.in_row_stride = F2;
    q.batch = 1; q.R = R; q.C = F2; q.Rp = R;
    q.row_codes = static_cast<uint8_t*>(dgr); q.row_scales = dgrs;
    q.col_codes = static_cast<uint8_t*>(dgc); q.col_scales = dgcs;
    q.tensor_scale = tsc.dgu;
    st = launch_quant_tile(q, true, s, "quant_dgu_mx");
    if (st != MGE_OK) return st;
  }
  if (mx) {
    pack(dgrs, nullptr, 1, R, F2 / 32, nullptr, dgr_p);
    pack(dgcs, nullptr, 1, F2, R / 32, rows_written, dgc_p);
    st = flush_packs();
    if (st != MGE_OK) return st;
  }
  // b3: d_prob[t][i] = the row sum of the assignment's permuted row
  st = launch_dprob_reduce(a->T, a->k, nparts, dprob_part, int64_t(R), a->perm_pos, a->d_prob, s);
  if (st != MGE_OK) return st;
  // b4: dW_down[e] = dY_e^T h_e  (K = tokens of e)
  {
    GemmParams g{};
    g.mode = RAGGED_K; g.E = E; g.sizes = a->split_sizes; g.offs = a->group_offsets; g.rows = R;
    g.A = static_cast<const uint8_t*>(dyc); g.lda = int64_t(R) * elem; g.Asp = dyc_p; g.asp_ld = H; g.asp_bytes = packed_exact(1, H, R / 32);
    g.B = static_cast<const uint8_t*>(a->h_col); g.ldb = int64_t(R) * elem; g.Bsp = hc_p; g.bsp_ld = F; g.bsp_bytes = packed_exact(1, F, R / 32);
    g.M = H; g.N = F;
    g.out_dtype = dw_bf16 ? MGE_DTYPE_BF16 : MGE_DTYPE_F32; g.Ct = reinterpret_cast<void* const*>(tab + 4 * E); g.ldc = F;
    g.accumulate = a->accumulate;
    g.tiles_upper = gemm_tiles_upper(g, rows_bound);
    g.band_m = kBandDwDown;
    g.role = GEMM_DW_DOWN;
    st = launch_gemm(g, a->prec, s);
    if (st != MGE_OK) return st;
  }
  // b5: dX = dGU W_gate_up  (K = 2F)
  {
    GemmParams g{};
    g.mode = RAGGED_M; g.E = E; g.sizes = a->split_sizes; g.offs = a->group_offsets; g.rows = R;
    g.A = static_cast<const uint8_t*>(dgr); g.lda = int64_t(F2) * elem; g.Asp = dgr_p; g.asp_ld = R; g.asp_bytes = packed_exact(1, R, F2 / 32);
    g.Bt = reinterpret_cast<const uint8_t* const*>(tab + E);
    g.Bsp = wguc_p; g.bsp_ld = H; g.bsp_estride = scale_pack_dwords(H, F2 / 32);
    g.bsp_bytes = packed_exact(E, H, F2 / 32);
    g.ldb = int64_t(F2) * elem;
    g.N = H; g.K = F2;
    g.out_dtype = MGE_DTYPE_BF16; g.C = a->dx_perm; g.ldc = H;
    g.tiles_upper = gemm_tiles_upper(g, rows_bound);
    g.role = GEMM_DX;
    st = launch_gemm(g, a->prec, s);
    if (st != MGE_OK) return st;
  }
  // b6: dW_gate_up[e] = dGU_e^T X_e  (K = tokens of e)
  {
    GemmParams g{};
    g.mode = RAGGED_K; g.E = E; g.sizes = a->split_sizes; g.offs = a->group_offsets; g.rows = R;
    g.A = static_cast<const uint8_t*>(dgc); g.lda = int64_t(R) * elem; g.Asp = dgc_p; g.asp_ld = F2; g.asp_bytes = packed_exact(1, F2, R / 32);
    g.B = static_cast<const uint8_t*>(a->x_col); g.ldb = int64_t(R) * elem; g.Bsp = xc_p; g.bsp_ld = H; g.bsp_bytes = packed_exact(1, H, R / 32);
    g.M = F2; g.N = H;
    g.out_dtype = dw_bf16 ? MGE_DTYPE_BF16 : MGE_DTYPE_F32; g.Ct = reinterpret_cast<void* const*>(tab + 5 * E); g.ldc = H;
    g.accumulate = a->accumulate;
    g.tiles_upper = gemm_tiles_upper(g, rows_bound);
    g.band_m = kBandDwGateUp;
    g.role = GEMM_DW_GATEUP;
    st = launch_gemm(g, a->prec, s);
  }
  return st;
}

// ------------------------------------------------------------------ combine
mge_status unpermute_combine(const mge_combine_args* a, void* stream) {
  g_err[0] = 0;
  MGE_REQUIRE(a != nullptr, "args is NULL");
  MGE_REQUIRE(a->struct_size == sizeof(mge_combine_args), "struct_size mismatch");
  MGE_REQUIRE(a->T >= 0 && a->k >= 1 && a->k <= 8, "T must be >= 0 and k in [1, 8]");
  MGE_REQUIRE(a->H >= 32 && a->H % 32 == 0, "H must be a positive multiple of 32");
  MGE_REQUIRE((a->in_dtype == MGE_DTYPE_BF16 || a->in_dtype == MGE_DTYPE_F32) &&
                  (a->out_dtype == MGE_DTYPE_BF16 || a->out_dtype == MGE_DTYPE_F32),
              "dtypes must be BF16 or F32");
  MGE_REQUIRE(a->in && aligned16(a->in) && a->out && aligned16(a->out) && a->perm_pos,
              "in / out / perm_pos NULL or misaligned");
  MGE_REQUIRE(a->in_rows >= 0, "in_rows must be >= 0 (got %lld)", (long long)a->in_rows);
  return launch_combine(a->T, a->k, a->H, a->in_dtype, a->out_dtype, a->in, a->in_rows, a->perm_pos, a->weights,
                        a->out, static_cast<hipStream_t>(stream));
}

mge_status moe_router_bwd(const mge_router_bwd_args* a, void* stream) {
  g_err[0] = 0;
  MGE_REQUIRE(a != nullptr, "args is NULL");
  MGE_REQUIRE(a->struct_size == sizeof(mge_router_bwd_args), "struct_size mismatch");
  MGE_REQUIRE(a->T >= 0, "T must be >= 0 (got %d)", a->T);
  MGE_REQUIRE(a->E >= 1 && a->E <= 256, "E must be in [1, 256] (got %d)", a->E);
  MGE_REQUIRE(a->k >= 1 && a->k <= 8 && a->k <= a->E, "k must be in [1, min(E, 8)] (got k=%d, E=%d)", a->k, a->E);
  if (a->T == 0) return MGE_OK;
  MGE_REQUIRE(a->topk_idx && a->topk_prob && a->d_prob && a->d_logits, "topk_idx / topk_prob / d_prob / d_logits NULL");
  return launch_router_bwd(a->T, a->E, a->k, a->topk_idx, a->topk_prob, a->d_prob, a->d_logits,
                           static_cast<hipStream_t>(stream));
}

mge_status mge_check_device_errors(void* route_workspace, void* stream) {
  g_err[0] = 0;
  MGE_REQUIRE(route_workspace != nullptr, "workspace is NULL");
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t flag = 0;
  if (hipStreamSynchronize(s) != hipSuccess) return hip_check("hipStreamSynchronize");
  if (hipMemcpy(&flag, route_workspace, sizeof(flag), hipMemcpyDeviceToHost) != hipSuccess)
    return hip_check("hipMemcpy");
  if (flag != 0) {
    int32_t zero = 0;
    hipMemcpy(route_workspace, &zero, sizeof(zero), hipMemcpyHostToDevice);
    set_error("a kernel flagged invalid data (expert index outside [0, E))");
    return MGE_ERR_DEVICE_CHECK;
  }
  return MGE_OK;
}

}  // extern "C"
