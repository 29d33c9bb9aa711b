// MXFP8 block quantization (E4M3 + E8M0 per 32) of bf16 matrices, row and column
// orientation, with an optional row gather (the permuted x / dy of the grouped MLP).
//
// One workgroup (512 threads) owns a 128 x 128 tile.  Row form: each thread quantizes one
// 32-value block (read back from the LDS tile, or, gathered, loaded by itself); the 4 lanes
// of a row write its 128 codes as one 128-byte piece.  Column form: from the tile in LDS,
// each thread quantizes 32 consecutive rows of one column, writing the transposed,
// K-contiguous layout the weight-gradient GEMMs read; the 4 lanes of a column are
// neighbours, so its 128 rows also leave as one 128-byte piece (whole cache lines in both
// forms: half lines measured 10% slower on MI355X).  Where the layout allows it, the 4 scale bytes a quad of lanes
// produces go out as one dword (single-byte stores cost another 11%).  The bf16 variant
// of the same kernel writes a plain (gathered) copy and the bf16 transpose.
// With a per-tensor scale given (FP8 with one scale per tensor), every block takes that
// scale instead of its own and the scale arrays hold it replicated, so the block-scaled
// GEMMs consume such operands unchanged.
// HBM-bound: 2 B read + (1 + 1/32) B written per element and orientation.
#include "mge_common.hpp"
#include "mge_internal.hpp"

namespace mge {

constexpr int QT_ROWS = 128;
constexpr int QT_COLS = 128;
constexpr int QT_THREADS = 512;
constexpr int QT_LDS_STRIDE = QT_COLS + 8;   // bf16 elements per LDS row
// extra bf16 per 32-row group: the column reads of a wave (16 columns x 4 row groups)
// then fall on 32 distinct banks
constexpr int QT_GRP = 16;
__device__ __forceinline__ int qt_at(int row, int col) { return row * QT_LDS_STRIDE + (row >> 5) * QT_GRP + col; }

// One block of 32 bf16 values held as 16 packed pairs (low half first) -> 32 E4M3 codes
// (8 dwords, element order) and the block's E8M0 scale byte: from the block's amax, or
// `given` (a tensor's one scale) when it is not negative.
__device__ __forceinline__ uint32_t quant32(const uint32_t* w, uint32_t* out, int given) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    amax = fmaxf(amax, fabsf(__uint_as_float(w[i] << 16)));
    amax = fmaxf(amax, fabsf(__uint_as_float(w[i] & 0xffff0000u)));
  }
  const uint32_t s = given >= 0 ? uint32_t(given) : mx_scale_byte(amax);
  const float inv = mx_inv_scale(s);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t q0 = e4m3_rne(__uint_as_float(w[2 * i] << 16) * inv);
    const uint32_t q1 = e4m3_rne(__uint_as_float(w[2 * i] & 0xffff0000u) * inv);
    const uint32_t q2 = e4m3_rne(__uint_as_float(w[2 * i + 1] << 16) * inv);
    const uint32_t q3 = e4m3_rne(__uint_as_float(w[2 * i + 1] & 0xffff0000u) * inv);
    out[i] = q0 | (q1 << 8) | (q2 << 16) | (q3 << 24);
  }
  return s;
}

// A quad of lanes q = 0..3 holds bytes [32q, 32q + 32) of a 128-byte piece as out[0..7].
// Rearranged so that the quad's first store writes bytes [0, 64) and its second bytes
// [64, 128) (lane q: [16q, 16q + 16), then [64 + 16q, ...)): each store instruction then
// covers whole 64-byte runs instead of 16-byte pieces spread over the line.
__device__ __forceinline__ void quad_store128(uint8_t* base, const uint32_t* out) {
  const bool odd = (threadIdx.x & 1) != 0;
  uint32_t a[4], b[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t x0 = uint32_t(__builtin_amdgcn_mov_dpp(int(out[j]), 0x50, 0xf, 0xf, false));       // lane q>>1
    const uint32_t x1 = uint32_t(__builtin_amdgcn_mov_dpp(int(out[4 + j]), 0x50, 0xf, 0xf, false));
    const uint32_t y0 = uint32_t(__builtin_amdgcn_mov_dpp(int(out[j]), 0xFA, 0xf, 0xf, false));       // lane 2 + (q>>1)
    const uint32_t y1 = uint32_t(__builtin_amdgcn_mov_dpp(int(out[4 + j]), 0xFA, 0xf, 0xf, false));
    a[j] = odd ? x1 : x0;
    b[j] = odd ? y1 : y0;
  }
  const int q = threadIdx.x & 3;
  *reinterpret_cast<uint4*>(base + 16 * q) = make_uint4(a[0], a[1], a[2], a[3]);
  *reinterpret_cast<uint4*>(base + 64 + 16 * q) = make_uint4(b[0], b[1], b[2], b[3]);
}

template <bool MX>
__global__ __launch_bounds__(QT_THREADS) void quant_tile_kernel(QuantTileParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[QT_ROWS * QT_LDS_STRIDE + (QT_ROWS / 32) * QT_GRP];
  const int tid = threadIdx.x;
  const int c0 = blockIdx.x * QT_COLS;
  const int r0 = blockIdx.y * QT_ROWS;
  const int b = blockIdx.z;
  const uint16_t* in = p.in + int64_t(b) * p.in_batch_stride;
  const int given = p.tensor_scale ? int(p.tensor_scale[b]) : -1;   // uniform

  // ---- load.  Without a gather the tile goes to LDS first, in whole lines (16 lanes per
  // 256-byte tile row, a wave covering 4 rows per instruction, 4 rounds of 32 rows, all 4
  // loads in flight together), and each thread reads its block back: 4% faster on the
  // weight matrices than each thread loading its own 64 bytes, which spreads an
  // instruction over 32 lines.  With a gather (the permuted x and dy) each thread loads its
  // block itself: staging the gathered rows measured 7% slower.
  // Thread -> (row r0 + tid/4, columns c0 + (tid%4)*32 .. +32).
  const int rl = tid >> 2;
  const int cl = (tid & 3) * 32;
  const int r = r0 + rl;
  const int c = c0 + cl;
  uint4 v[4];
  if (!p.gather) {   // uniform
    const int lr = tid >> 4;
    const int ch = (tid & 15) * 8;
    const int cg = c0 + ch;
    // branch-free, so that the 4 loads are in flight together: a lane outside the matrix
    // reads its first element (the launch has R, C > 0) and stores zeros
    uint4 val[4];
    bool ok[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rg = r0 + 32 * i + lr;
      ok[i] = rg < p.R && cg < p.C;
      val[i] = *reinterpret_cast<const uint4*>(in + (ok[i] ? int64_t(rg) * p.in_row_stride + cg : 0));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<uint4*>(tile + qt_at(32 * i + lr, ch)) = ok[i] ? val[i] : make_uint4(0, 0, 0, 0);
    lds_barrier();
    const uint4* t4 = reinterpret_cast<const uint4*>(tile + qt_at(rl, cl));
    v[0] = t4[0]; v[1] = t4[1]; v[2] = t4[2]; v[3] = t4[3];
  } else {
    bool have = false;
    if (r < p.R && c < p.C) {
      const int64_t src = p.gather[r];
      // a gathered row outside the source rows (only bad data can give one) reads as zero
      if (src >= 0 && src < p.src_rows) {
        const uint4* g = reinterpret_cast<const uint4*>(in + src * p.in_row_stride + c);
        v[0] = g[0]; v[1] = g[1]; v[2] = g[2]; v[3] = g[3];
        have = true;
      }
    }
    if (!have) {
      for (int i = 0; i < 4; ++i) v[i] = make_uint4(0, 0, 0, 0);
    }
  }

  // ---- row form
  if (r < p.R && c < p.C && (p.row_codes || p.row_bf16)) {
    const int64_t ob = int64_t(b) * p.R + r;
    if (MX) {
      uint32_t out[8];
      const uint32_t s = quant32(reinterpret_cast<const uint32_t*>(v), out, given);
      if ((p.C & (QT_COLS - 1)) == 0) {   // uniform: the quad's 4 lanes are all here
        quad_store128(p.row_codes + ob * p.C + c0, out);
      } else {
        uint4* dst = reinterpret_cast<uint4*>(p.row_codes + ob * p.C + c);
        dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
        dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
      }
      uint8_t* rs = p.row_scales + ob * (p.C / 32) + c / 32;
      // uniform: the 4 lanes of the row are all active and the dword is aligned
      if ((p.C & (QT_COLS - 1)) == 0 && (reinterpret_cast<uintptr_t>(p.row_scales) & 3) == 0) {
        const uint32_t w = quad_bytes(s);
        if ((tid & 3) == 0) *reinterpret_cast<uint32_t*>(rs) = w;
      } else {
        *rs = uint8_t(s);
      }
    } else {
      uint4* dst = reinterpret_cast<uint4*>(p.row_bf16 + ob * p.C + c);
      dst[0] = v[0]; dst[1] = v[1]; dst[2] = v[2]; dst[3] = v[3];
    }
  }

  if (!(p.col_codes || p.col_bf16)) return;

  // ---- column form: the tile in LDS (a gathered tile is staged now, so that the row-form
  // stores leave first), then thread -> (column tid/4, rows (tid%4)*32..+32)
  if (p.gather) {   // uniform
    uint4* t4 = reinterpret_cast<uint4*>(tile + qt_at(rl, cl));
    t4[0] = v[0]; t4[1] = v[1]; t4[2] = v[2]; t4[3] = v[3];
    lds_barrier();   // (the row-form stores need not have landed)
  }
  const int cc = tid >> 2;
  const int rb = tid & 3;
  const int col = c0 + cc;
  const int rowb = r0 + rb * 32;
  if (col >= p.C || rowb >= p.Rp) return;
  // the column's 32 values as 16 packed bf16 pairs (rows 2i, 2i + 1)
  uint32_t hw[16];
#pragma unroll
  for (int i = 0; i < 16; ++i)
    hw[i] = uint32_t(tile[qt_at(rb * 32 + 2 * i, cc)]) | (uint32_t(tile[qt_at(rb * 32 + 2 * i + 1, cc)]) << 16);
  const int64_t ocol = int64_t(b) * p.C + col;
  if (MX) {
    uint32_t out[8];
    const uint32_t s = quant32(hw, out, given);
    if ((p.Rp & (QT_ROWS - 1)) == 0) {   // uniform: the quad's 4 row blocks are all here
      quad_store128(p.col_codes + ocol * p.Rp + r0, out);
    } else {
      uint4* dst = reinterpret_cast<uint4*>(p.col_codes + ocol * p.Rp + rowb);
      dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
      dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
    }
    uint8_t* cs = p.col_scales + ocol * (p.Rp / 32) + rowb / 32;
    // uniform: the 4 row blocks of every column exist and the dword is aligned
    if ((p.Rp & (QT_ROWS - 1)) == 0 && (reinterpret_cast<uintptr_t>(p.col_scales) & 3) == 0) {
      const uint32_t w = quad_bytes(s);
      if (rb == 0) *reinterpret_cast<uint32_t*>(cs) = w;
    } else {
      *cs = uint8_t(s);
    }
  } else {
    uint4* dst = reinterpret_cast<uint4*>(p.col_bf16 + ocol * p.Rp + rowb);
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = make_uint4(hw[4 * i], hw[4 * i + 1], hw[4 * i + 2], hw[4 * i + 3]);
  }
}

// ---------------------------------------------------------------- segmented row map
// Segments s = input rows [seg[s], seg[s+1]) placed at 32-row multiples: output row o of
// the padded order -> its input row, or -1 (the zero rows that pad a segment to 32).
// Every block builds the padded starts in LDS (4 segments per thread, a Hillis-Steele
// scan of the 256 thread sums), then maps its grid-stride share of the Rp output rows.
// Offsets are clamped to [0, R] and made non-decreasing, and rows past Rp are not
// mapped, so malformed offsets give undefined results but stay in bounds.
constexpr int SEG_THREADS = 256;
constexpr int SEG_PER_THREAD = SEG_MAX / SEG_THREADS;

__global__ __launch_bounds__(SEG_THREADS) void seg_map_kernel(const int32_t* __restrict__ seg, int S, int R, int Rp,
                                                              int32_t* __restrict__ map) {
  __shared__ int32_t pstart[SEG_MAX + 1];
  __shared__ int32_t istart[SEG_MAX];
  __shared__ int32_t slen[SEG_MAX];
  __shared__ int32_t tsum[SEG_THREADS];
  const int t = threadIdx.x;
  int padded[SEG_PER_THREAD];
  int mine = 0;
#pragma unroll
  for (int j = 0; j < SEG_PER_THREAD; ++j) {
    const int s = t * SEG_PER_THREAD + j;
    padded[j] = 0;
    if (s < S) {
      const int a = min(max(seg[s], 0), R);
      const int b = min(max(seg[s + 1], a), R);
      istart[s] = a;
      slen[s] = b - a;
      padded[j] = (b - a + 31) / 32 * 32;
      mine += padded[j];
    }
  }
  tsum[t] = mine;
  __syncthreads();
  for (int d = 1; d < SEG_THREADS; d <<= 1) {   // inclusive scan of the thread sums
    const int v = t >= d ? tsum[t - d] : 0;
    __syncthreads();
    tsum[t] += v;
    __syncthreads();
  }
  int acc = tsum[t] - mine;
#pragma unroll
  for (int j = 0; j < SEG_PER_THREAD; ++j) {
    const int s = t * SEG_PER_THREAD + j;
    if (s < S) pstart[s] = acc;
    acc += padded[j];
  }
  if (t == SEG_THREADS - 1) pstart[S] = tsum[t];
  __syncthreads();
  for (int o = blockIdx.x * SEG_THREADS + t; o < Rp; o += gridDim.x * SEG_THREADS) {
    int src = -1;
    if (o < pstart[S]) {
      int lo = 0, hi = S - 1;   // the last segment whose padded start is <= o
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (pstart[mid] <= o) lo = mid; else hi = mid - 1;
      }
      const int i = o - pstart[lo];
      if (i < slen[lo]) src = istart[lo] + i;
    }
    map[o] = src;
  }
}

mge_status launch_seg_map(const int32_t* seg, int S, int R, int Rp, int32_t* map, hipStream_t s) {
  if (Rp <= 0) return MGE_OK;
  int blocks = (Rp + SEG_THREADS - 1) / SEG_THREADS;
  if (blocks > 256) blocks = 256;
  ProfScope prof(s, "seg_map");
  hipLaunchKernelGGL(seg_map_kernel, dim3(blocks), dim3(SEG_THREADS), 0, s, seg, S, R, Rp, map);
  return hip_check("seg_map_kernel");
}

// ---------------------------------------------------------------- per-tensor scale
// FP8 with one scale per tensor: amax over each of `batch` tensors of n bf16 values, then
// the block rule's E8M0 byte of that amax (the whole tensor as one block).  Two launches,
// no atomics: each workgroup writes the max of its grid-stride share of a tensor, and one
// workgroup per tensor reduces those partials.  HBM-bound: 2 B read per element.
constexpr int TS_THREADS = 256;

__device__ __forceinline__ float ts_block_max(float m, float* red) {
  m = wave_max_xor(m, 64);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = m;
  __syncthreads();
  m = red[0];
#pragma unroll
  for (int w = 1; w < TS_THREADS / 64; ++w) m = fmaxf(m, red[w]);
  return m;
}

__global__ __launch_bounds__(TS_THREADS) void tensor_amax_kernel(const uint16_t* __restrict__ in, int64_t n,
                                                                 int64_t bstride, float* __restrict__ part) {
  __shared__ float red[TS_THREADS / 64];
  const uint16_t* x = in + int64_t(blockIdx.y) * bstride;
  const int64_t stride = int64_t(gridDim.x) * TS_THREADS;
  const int64_t t0 = int64_t(blockIdx.x) * TS_THREADS + threadIdx.x;
  float m = 0.f;
  // 16-byte loads where the tensor's base is 16-byte aligned, element loads for the rest
  const int64_t head = ((16 - (reinterpret_cast<uintptr_t>(x) & 15)) & 15) / 2;
  const int64_t h = head < n ? head : n;
  const int64_t nv = (n - h) / 8;
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4* xv = reinterpret_cast<const u32x4*>(x + h);
  for (int64_t i = t0; i < nv; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(xv + i);   // read once
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      m = fmaxf(m, fabsf(__uint_as_float(u[j] << 16)));
      m = fmaxf(m, fabsf(__uint_as_float(u[j] & 0xffff0000u)));
    }
  }
  for (int64_t i = t0; i < h; i += stride) m = fmaxf(m, fabsf(bf16_to_f32(x[i])));
  for (int64_t i = h + nv * 8 + t0; i < n; i += stride) m = fmaxf(m, fabsf(bf16_to_f32(x[i])));
  m = ts_block_max(m, red);
  if (threadIdx.x == 0) part[int64_t(blockIdx.y) * gridDim.x + blockIdx.x] = m;
}

__global__ __launch_bounds__(TS_THREADS) void tensor_scale_kernel(const float* __restrict__ part, int nparts,
                                                                  uint8_t* __restrict__ scale) {
  __shared__ float red[TS_THREADS / 64];
  const float* pb = part + int64_t(blockIdx.x) * nparts;
  float m = 0.f;
  for (int i = threadIdx.x; i < nparts; i += TS_THREADS) m = fmaxf(m, pb[i]);
  m = ts_block_max(m, red);
  if (threadIdx.x == 0) scale[blockIdx.x] = uint8_t(mx_scale_byte(m));
}

int tensor_scale_parts(int64_t n) {
  const int64_t v = (n / 8 + TS_THREADS - 1) / TS_THREADS;
  return int(v < 1 ? 1 : (v > 1024 ? 1024 : v));
}

mge_status launch_tensor_scale(const uint16_t* in, int batch, int64_t n, int64_t bstride, float* part,
                               uint8_t* scale, hipStream_t s) {
  if (batch <= 0) return MGE_OK;
  const int nparts = tensor_scale_parts(n);
  {
    ProfScope prof(s, "tensor_amax");
    hipLaunchKernelGGL(tensor_amax_kernel, dim3(nparts, batch), dim3(TS_THREADS), 0, s, in, n, bstride, part);
    const mge_status st = hip_check("tensor_amax_kernel");
    if (st != MGE_OK) return st;
  }
  ProfScope prof(s, "tensor_scale");
  hipLaunchKernelGGL(tensor_scale_kernel, dim3(batch), dim3(TS_THREADS), 0, s, part, nparts, scale);
  return hip_check("tensor_scale_kernel");
}

// ---------------------------------------------------------------- scale packing
// A 64-row x 128-byte tile of a scale matrix goes through LDS in two passes of 32 rows:
// thread t reads 16 bytes of row t/8 (one 16-byte load where the batch's base and row
// stride allow it, else byte loads), so the 8 threads of a row read one whole 128-byte
// line (64-byte pieces measured 7% slower); the packed dwords leave with consecutive
// threads on consecutive rows.  One
// launch packs up to SP_MAXD matrices: the flat grid walks the tiles of matrix 0 (all its
// batches), then of matrix 1, ...
constexpr int SP_ROWS = 64;
constexpr int SP_BYTES = 128;
constexpr int SP_LD = SP_BYTES + 4;   // LDS row stride in bytes: 33 dwords, so the dword reads of 64 rows hit 64 banks

struct ScalePackBatch {
  ScalePackParams d[SP_MAXD];
  int start[SP_MAXD + 1];   // first flat tile of matrix j
  int n;
};

__global__ __launch_bounds__(256) void scale_pack_kernel(ScalePackBatch B) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[SP_ROWS * SP_LD];
  const int blk = blockIdx.x;
  int jd = 0;
  while (jd + 1 < B.n && B.start[jd + 1] <= blk) ++jd;
  const ScalePackParams& p = B.d[jd];
  const int tx_n = (p.kb + SP_BYTES - 1) / SP_BYTES;
  const int ty_n = (p.rows + SP_ROWS - 1) / SP_ROWS;
  const int local = blk - B.start[jd];
  const int b = local / (tx_n * ty_n);
  const int rem = local - b * tx_n * ty_n;
  const int c0 = (rem % tx_n) * SP_BYTES;
  const int r0 = (rem / tx_n) * SP_ROWS;
  const int tid = threadIdx.x;
  const uint8_t* src = p.src_tab ? p.src_tab[b] : p.src + int64_t(b) * p.src_bstride;
  const int kb_lim = p.kb_valid ? min(p.kb, p.kb_valid[0] / 32) : p.kb;
  for (int pass = 0; pass < SP_ROWS * SP_BYTES / (256 * 16); ++pass) {
    const int rr = pass * (256 * 16 / SP_BYTES) + tid / (SP_BYTES / 16), cc = (tid % (SP_BYTES / 16)) * 16;
    const int r = r0 + rr, c = c0 + cc;
    uint32_t w[4];
    const bool vec = ((reinterpret_cast<uintptr_t>(src) | uintptr_t(p.ld)) & 15) == 0;   // uniform
    if (vec && r < p.rows && c + 16 <= kb_lim) {
      const uint4 v = *reinterpret_cast<const uint4*>(src + int64_t(r) * p.ld + c);
      w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t x = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int cb = c + 4 * q + k;
          const uint32_t byte = (r < p.rows && cb < kb_lim) ? src[int64_t(r) * p.ld + cb] : 127u;
          x |= byte << (8 * k);
        }
        w[q] = x;
      }
    }
    uint32_t* t32 = reinterpret_cast<uint32_t*>(tile + rr * SP_LD + cc);
#pragma unroll
    for (int q = 0; q < 4; ++q) t32[q] = w[q];
  }
  lds_barrier();
  const int kb4 = (p.kb + 3) / 4;
  uint32_t* dst = p.dst + int64_t(b) * kb4 * p.rows;
#pragma unroll
  for (int i = tid; i < SP_ROWS * (SP_BYTES / 4); i += 256) {
    const int jj = i / SP_ROWS, rr = i % SP_ROWS;
    const int j = c0 / 4 + jj, r = r0 + rr;
    if (r < p.rows && j < kb4) dst[int64_t(j) * p.rows + r] = *reinterpret_cast<const uint32_t*>(tile + rr * SP_LD + 4 * jj);
  }
}

mge_status launch_scale_pack_batch(const ScalePackParams* list, int n, hipStream_t s) {
  MGE_REQUIRE(n >= 0 && n <= SP_MAXD, "at most %d scale packs per launch (got %d)", SP_MAXD, n);
  ScalePackBatch B{};
  int total = 0;
  B.n = 0;
  for (int i = 0; i < n; ++i) {
    const ScalePackParams& p = list[i];
    if (p.rows <= 0 || p.kb <= 0 || p.batch <= 0) continue;
    const int64_t tiles = int64_t((p.kb + SP_BYTES - 1) / SP_BYTES) * ((p.rows + SP_ROWS - 1) / SP_ROWS) * p.batch;
    MGE_REQUIRE(total + tiles < (int64_t(1) << 31), "scale pack grid too large");
    B.d[B.n] = p;
    B.start[B.n] = total;
    total += int(tiles);
    ++B.n;
  }
  B.start[B.n] = total;
  if (total == 0) return MGE_OK;
  ProfScope prof(s, "scale_pack");
  hipLaunchKernelGGL(scale_pack_kernel, dim3(total), dim3(256), 0, s, B);
  return hip_check("scale_pack_kernel");
}

mge_status launch_scale_pack(const ScalePackParams& p, hipStream_t s) { return launch_scale_pack_batch(&p, 1, s); }

mge_status launch_quant_tile(const QuantTileParams& p, bool mx, hipStream_t s, const char* timing_name) {
  if (p.R <= 0 || p.C <= 0 || p.batch <= 0) return MGE_OK;
  int rows_cover = p.Rp > p.R ? p.Rp : p.R;
  dim3 grid((p.C + QT_COLS - 1) / QT_COLS, (rows_cover + QT_ROWS - 1) / QT_ROWS, p.batch);
  const char* name = timing_name ? timing_name
                     : mx ? (p.gather ? "permute_quant_mx" : "quant_mx") : (p.gather ? "permute_bf16" : "transpose_bf16");
  ProfScope prof(s, name);
  if (mx)
    hipLaunchKernelGGL(quant_tile_kernel<true>, grid, dim3(QT_THREADS), 0, s, p);
  else
    hipLaunchKernelGGL(quant_tile_kernel<false>, grid, dim3(QT_THREADS), 0, s, p);
  return hip_check("quant_tile_kernel");
}

}  // namespace mge
