// Persistent grouped GEMM for gfx950: C_e = A_e B_e^T for every expert in one launch.
//
// Both operands are K-contiguous ("NT"): row forms along K for the forward and dX
// GEMMs, column forms (transposed, blocks along tokens) for the weight gradients.
//   RAGGED_M: expert e owns rows [off[e], off[e] + sizes[e]) of a shared A and of the
//             output; B is the expert's own weight (pointer table).  (gate-up, down,
//             dh, dX)
//   RAGGED_K: the reduction runs over expert e's tokens, the column span
//             [off[e], off[e] + roundup32(sizes[e])) of shared A and B; the output is
//             the expert's own [M][N] gradient.  (dW_down, dW_gate_up)
// Tiles are 256 x 256, 4 waves in a 2 x 2 grid, each wave 128 x 128 built from 32 x 32
// MFMA blocks whose fp32 accumulators stay in AGPRs:
//   MXFP8: v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 x E4M3, one E8M0 scale per lane and
//          32-element K block, applied by the matrix core — no dequantize pass).
//          Operand layout (measured on gfx950): lane l = 32h + i feeds row/column i;
//          its register bytes 0..15 are K elements 16h..16h+15 and bytes 16..31 are
//          32+16h..32+16h+15 of the 64-element step, so K block h (elements
//          32h..32h+31) is scaled by the scale register of the lanes with that h, the
//          byte chosen by op_sel.
//   BF16:  v_mfma_f32_32x32x16_bf16
// Operands stream HBM -> LDS directly (buffer_load ... lds, no register staging) in
// 128-byte K slices (128 FP8 or 64 BF16 elements) through 2 LDS stages of 64 KB; a
// stage is refilled as soon as every wave has read its fragments, so a slice has one
// and a half iterations to arrive.  LDS rows are 128 bytes with the 16-byte chunks
// XOR-swizzled by row so the MFMA fragment reads spread over the 64 banks.  The MX
// scales of a slice ride along into LDS (packed: one dword = 4 blocks of a row).
// A persistent grid walks the tiles (expert-major, then bands of 8 M-tiles walked across
// N with M fastest, so that the 32 tiles an XCD runs at once are an 8 x 4 block sharing
// A and B tiles in its L2); virtual workgroup ids are remapped so
// that the workgroups of one XCD (hardware dispatches round-robin over the 8 XCDs)
// take consecutive tiles and share that XCD's L2.  Empty experts own no tiles (RAGGED_M)
// or produce zero gradients (RAGGED_K).  Before a plain-store or SwiGLU epilogue the next
// tile's first slice is issued, so its latency hides behind the epilogue.
// Epilogues (fp32 accumulators never reach HBM; no per-element branches: stores go
// through buffer resources whose record bound ends at the last valid row, so the
// hardware range check drops rows past the group, and columns past N get an offset
// beyond every bound):
//   EPI_STORE       bf16 / f32 store, or f32 added to the output (OutForm)
//   EPI_SWIGLU      h = p * silu(G) * U with G, U of the same rows/columns in the same
//                   lane; h quantized along F (MXFP8, amax over the 32 lanes that hold
//                   one 32-column block) or rounded to bf16; training also stores G, U
//                   (bf16) and the column form of h (blocks of 32 rows: 16 in a lane,
//                   16 in its partner lane 32 apart)
//   EPI_SWIGLU_BWD  dh = dY W_down stays in the accumulators; G, U of the same rows and
//                   columns come in by LDS DMA, and dG, dU (row and column forms, as
//                   above) and the d_prob partial row sums leave
#pragma once

#include "mge_common.hpp"
#include "mge_internal.hpp"

#include <type_traits>

namespace mge {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int G_WAVES_M = 2;
constexpr int G_WAVES_N = 2;
constexpr int G_WMB = 4;   // 32-row MFMA blocks per wave (M)
constexpr int G_WNB = 4;   // 32-col MFMA blocks per wave (N)
constexpr int G_BM = G_WAVES_M * G_WMB * 32;
constexpr int G_BN = G_WAVES_N * G_WNB * 32;
constexpr int G_BKB = 128;                    // K bytes per slice: one whole 128-byte line per operand row
#ifndef G_TAIL_SPLIT
#define G_TAIL_SPLIT 1   // plain-store ragged-M GEMMs: the grid's last round as quarter-width items
#endif
#ifndef G_EPI_GROUP
#define G_EPI_GROUP 1   // SwiGLU epilogues: 32 x 32 blocks the scheduler may interleave
#endif
#ifndef G_BAR_AT32
#define G_BAR_AT32 8   // a slice's stage is released after this many 32nds of its MFMAs
#endif
constexpr int G_STAGES = 2;                   // LDS stages, each refilled once its slice is in registers
constexpr int G_THREADS = 64 * G_WAVES_M * G_WAVES_N;
constexpr int G_STAGE_BYTES = (G_BM + G_BN) * G_BKB;   // 64 KB
constexpr int G_MAXE = 256;
constexpr int G_GROUP_M = 8;                  // M-tiles per band of the tile raster (GemmParams::group_m = 0)
// Buffer-resource word 3 of the gfx9 family (raw buffer, 32-bit dwords), the record
// bound, and the offset that lies beyond it (such a lane loads zeros).
constexpr int kRsrcFlags = 0x00020000;
constexpr int kRsrcRecords = 0x7fffffff;
constexpr uint32_t kInvalid = 0x80000000u;   // OR-ed into an offset: the lane reads zeros
// Cache-policy operand of the buffer builtins: non-temporal (gfx950's nt bit).  Used for
// output streams that no workgroup of the same kernel reads again, so that they do not
// evict the operand lines other workgroups of the XCD are about to share from its L2
// (weight-gradient GEMMs, 256 KB of fp32 per tile: 7% faster on MI355X).  Only for
// whole-line stores: partial lines with the hint measured slower.
constexpr int kNonTemporal = 2;

static_assert(G_THREADS == 256, "loader assumes 256 threads");

// Compile-time loop: the body sees its index as a constant expression, so register
// arrays (the accumulators) are never indexed dynamically.
template <int I, int N, typename Fn>
__device__ __forceinline__ void static_for(Fn&& fn) {
  if constexpr (I < N) {
    fn(std::integral_constant<int, I>{});
    static_for<I + 1, N>(fn);
  }
}

// Values that are the same in every lane, moved to scalar registers so that buffer
// resources and LDS-DMA destinations need no per-lane handling.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
// Element i (wave-uniform) of a table the kernel never writes (sizes, offsets, pointer
// tables), read through the constant address space: the compiler then emits a scalar
// load, counted by lgkmcnt.  A vector load would be counted by vmcnt, and waiting for
// it would also wait for every operand DMA and epilogue store issued before it.
template <typename T>
__device__ __forceinline__ T ld_uniform(const T* base, int i) {
  typedef const __attribute__((address_space(4))) T const_t;
  return reinterpret_cast<const_t*>(reinterpret_cast<uintptr_t>(base))[i];
}
template <typename T>
__device__ __forceinline__ const T* uniform_ptr(const T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(v >> 32));
  return reinterpret_cast<const T*>((uint64_t(hi) << 32) | lo);
}

// Byte offset of 16-byte chunk `chunk` (0..7) of tile row `row` in LDS.  The LDS of
// gfx950 has 64 four-byte banks and serves a ds_read_b128 16 lanes at a time; a fragment
// read has 16 consecutive rows read the same chunk.  A 128-byte row covers half of the
// banks (even rows one half, odd rows the other), so the chunk is XOR-ed with
// (row / 2) mod 8: the 8 rows of each parity land on 8 distinct 16-byte bank groups.
__device__ __forceinline__ int swz(int row, int chunk) { return row * G_BKB + ((chunk ^ ((row >> 1) & 7)) << 4); }

// Raw buffer resource over `base` (gfx9 word 3, full 31-bit range) ...
__device__ __forceinline__ i32x4 make_rsrc(const void* base) {
  const uint64_t v = reinterpret_cast<uint64_t>(base);
  return i32x4{int(uint32_t(v)), int(uint32_t(v >> 32) & 0xffff), kRsrcRecords, kRsrcFlags};
}
// ... and one bounded to `bytes` (reads past it return zeros).
// The words go through readfirstlane: the inline-asm users take the resource in SGPRs and
// the compiler keeps some uniform values (clamps) in VGPRs.
__device__ __forceinline__ i32x4 make_rsrc_n(const void* base, uint32_t bytes) {
  const uint64_t v = reinterpret_cast<uint64_t>(base);
  return i32x4{uniform(int(uint32_t(v))), uniform(int(uint32_t(v >> 32) & 0xffff)), uniform(int(bytes)), kRsrcFlags};
}

// One accumulator element into a VGPR.  The explicit read (an AGPR operand) keeps the
// accumulator tile in AGPRs until the epilogue reaches its block; left to itself the
// compiler copies all 256 accumulators into VGPRs at the end of the K loop and spills.
// The MFMA -> read hazard is covered by the wait states issued after the K loop
// (acc_settle), which the compiler cannot see through the asm.
__device__ __forceinline__ float acc_read(float x) {
  float y;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(y) : "a"(x));
  return y;
}
// 64 wait states: more than the longest MFMA result latency of gfx950 (a 16-pass XDL
// op needs 18 before a VALU may read its result)
__device__ __forceinline__ void acc_settle() {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
}

// s_waitcnt immediate (gfx9 encoding): wait until at most `vm` vector-memory and `lgkm`
// LDS/scalar operations are outstanding (export counter not waited on).
constexpr int waitcnt_imm(int vm, int lgkm) { return (vm & 0xf) | ((vm >> 4) << 14) | (7 << 4) | (lgkm << 8); }

// Workgroup barriers of the K loop.  __syncthreads() would also wait for every
// outstanding vector-memory operation (its fence), including the LDS DMAs that are meant
// to stay in flight across the barrier; these wait only for what they name (lds_barrier
// is in mge_common.hpp).
// vm_barrier<N>: at most N of this wave's vector-memory operations (the newest, as they
// complete in order) and no LDS read still outstanding, then all waves meet.
template <int N>
__device__ __forceinline__ void vm_barrier() {
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(N, 0));
  asm volatile("s_barrier" ::: "memory");
}

// 16 bytes per lane from buffer offset `voff` straight into LDS at lds_addr + 16*lane
// (buffer_load_dwordx4 ... lds; M0 holds the wave's LDS destination).  Written as asm
// so the compiler neither waits on it before unrelated LDS reads nor moves LDS accesses
// across it; every VMEM operation of the K loop is one of these, and the loop waits for
// them with explicit vmcnt values.  An s_nop separates the M0 write from the DMA that
// reads it.
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t lds_addr, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(lds_addr), "v"(voff),
               "s"(rsrc)
               : "memory", "m0");
}

// The same with the non-temporal hint, for data read once (the SwiGLU backward's G and
// U): it keeps that stream from evicting the K loop's shared operand lines from L2
// (dh GEMM 3% faster on MI355X).  Partial-line stores with the hint measured slower.
__device__ __forceinline__ void dma16_nt(i32x4 rsrc, uint32_t lds_addr, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds" ::"s"(lds_addr), "v"(voff),
               "s"(rsrc)
               : "memory", "m0");
}

// A decoded tile: which expert and block it is, its K range and operand bases.
struct Tile {
  int valid;
  int e, nt, off, m_valid, m0;
  int kbase, klo, khi, nkt;   // K range in bytes; slices of G_BKB from kbase
  // operand buffer resources: A starts at the tile's first row and B at its first weight
  // row (SwiGLU: the gate half; the up half is F rows further); the record bounds end at
  // the last valid row, so the hardware range check zeroes rows past the group / N / F
  int nb;                     // first output column (and B row) of the work item
  const uint8_t* A;
  const uint8_t* B;
  uint32_t arec, brec;
  int64_t sa_rows, sb_rows;   // MX: packed-scale dword of the tile's first A / B row at group 0
};

// LDS map (bytes from the start of the dynamic block):
//   [0, G_STAGES*G_STAGE_BYTES)   operand tiles, G_STAGES x (A 256 x 128 B, B 256 x 128 B)
//   then G_STAGES x 4 KB          E8M0 scales: four 1 KB slots per stage, slot w filled
//                                 by wave w (A rows 0-127, 128-255, B rows 0-127,
//                                 128-255; 512 B used per slot)
constexpr int G_SCALE_STAGE = 4096;
constexpr int G_SCALE_BASE = G_STAGES * G_STAGE_BYTES;
constexpr int G_DYN_LDS = G_SCALE_BASE + G_STAGES * G_SCALE_STAGE;

// QT = 1: the quarter-width tail kernel of a plain-store ragged-M GEMM.  The tiles past the
// last whole round of the main launch's grid would run alone on a fraction of the chip;
// this launch runs each of them as four 256 x 64 work items instead (the main launch leaves
// them out; both take the same decision from the same tile table).  Every output element is
// still accumulated by one wave over K in the same order: the results are bit-identical.
template <bool MX, int EPI, int MODE, int OUT, int QT = 0>
__device__ __forceinline__ void gemm_body(const GemmParams& p) {
  static_assert(QT == 0 || (EPI == EPI_STORE && MODE == RAGGED_M), "the quarter-width tail is for plain-store ragged-M GEMMs");
  constexpr int BW = QT ? G_BN / 4 : G_BN;        // output columns (B rows) of a work item
  constexpr int WNB = BW / (32 * G_WAVES_N);       // 32-column MFMA blocks per wave
  constexpr int NOPS = 8 + BW / 32;                // operand DMA instructions per wave and slice (A: 8)
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  // LDS byte address of the dynamic shared block (the low half of its generic address)
  const uint32_t lds_base = uniform(int(uint32_t(reinterpret_cast<uintptr_t>(smem))));
  __shared__ int32_t s_prefix[G_MAXE + 1];
  __shared__ int32_t s_mtiles[G_MAXE];
  __shared__ __attribute__((aligned(16))) float s_prob[G_BM];   // SwiGLU: routing probability of each tile row
  __shared__ __attribute__((aligned(16))) float s_inv[G_WAVES_M * G_WAVES_N * 32];   // SwiGLU: row-scale broadcast

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int wm = wave / G_WAVES_N;
  const int wn = wave % G_WAVES_N;
  // l32 / hi are re-derived from an opaque copy of the lane id at the top of every tile
  // and again after its K loop: the per-lane addresses of the K loop (LDS fragments) and
  // of the epilogue (stores) are then computed in their own phase instead of being
  // hoisted to kernel start, where together they would stay live and spill.
  int l32 = lane & 31;
  int hi = lane >> 5;
  auto rederive_lane = [&]() {
    int v = lane;
    asm volatile("" : "+v"(v));
    l32 = v & 31;
    hi = v >> 5;
  };
  constexpr int ELEM = MX ? 1 : 2;           // bytes per element

  // ---- tile table: tiles of expert e = mtiles(e) * ntiles
  const int ncols_per_tile = (EPI == EPI_SWIGLU) ? G_BN / 2 : G_BN;
  const int ncols = (EPI == EPI_SWIGLU) ? p.F : p.N;
  const int ntiles = (ncols + ncols_per_tile - 1) / ncols_per_tile;
  // A group's span, clamped into the R permuted rows, so that maps other than the routing
  // call's give wrong results but no access outside the buffers (the host cannot check
  // device-side maps).
  auto group_off = [&](int off) { return off < 0 ? 0 : (off > p.rows ? p.rows : off); };
  auto group_size = [&](int size, int off) { return size < 0 ? 0 : (size > p.rows - off ? p.rows - off : size); };
  if (tid == 0) {
    int acc = 0;
    for (int e = 0; e < p.E; ++e) {
      int mt = MODE == RAGGED_M ? (group_size(p.sizes[e], group_off(p.offs[e])) + G_BM - 1) / G_BM
                                : (p.M + G_BM - 1) / G_BM;
      s_prefix[e] = acc;
      s_mtiles[e] = mt;
      acc += mt * ntiles;
    }
    s_prefix[p.E] = acc;
  }
  __syncthreads();
  const int total = uniform(s_prefix[p.E]);
  const int nwg = gridDim.x;
  int vid = blockIdx.x;
  if ((nwg & 7) == 0) vid = (blockIdx.x & 7) * (nwg >> 3) + (blockIdx.x >> 3);
  // Work items of this launch.  With tail_split the tiles past the main launch's last whole
  // round go to the tail launch as quarter-width items, when there are at most two rounds of
  // those (each item streams the whole A slice, so it takes well over a quarter of a tile's
  // time).  Both launches decide from the same numbers: the tile count and the main grid.
  int items = total, t_full = total;
  {
    const int g = p.grid_main > 0 ? p.grid_main : nwg;
    const int full = (total / g) * g, tail = total - full;
    const bool split = p.tail_split != 0 && full > 0 && tail > 0 && tail * 4 <= 2 * g;
    if constexpr (QT) {
      t_full = full;
      items = split ? tail * 4 : 0;
    } else {
      items = split ? full : total;
    }
    items = uniform(items);
    t_full = uniform(t_full);
  }

  // every tile quantity is wave-uniform: kept in scalar registers
  auto decode = [&](int item) {
    Tile t{};
    t.valid = item < items;
    if (!t.valid) return t;
    int tile = item, quarter = 0;
    if constexpr (QT) {
      tile = t_full + item / 4;
      quarter = item % 4;
    }
    int lo = 0, hi_ = p.E - 1;
    while (lo < hi_) {
      int mid = (lo + hi_ + 1) >> 1;
      if (s_prefix[mid] <= tile) lo = mid; else hi_ = mid - 1;
    }
    t.e = uniform(lo);
    const int local = tile - uniform(s_prefix[t.e]);
    const int mtn = uniform(s_mtiles[t.e]);
    // grouped raster: bands of GM = 8 M-tiles, each band walked across all N-tiles with M
    // fastest, so that the 32 consecutive tiles an XCD runs (an 8 x 4 block) share a few A
    // and B tiles in that XCD's L2.  With group_m set (ragged M only), an expert's last band
    // takes a remainder under 4 M-tiles (9 M-tiles walked as one band, not as 8 + a lone 1)
    const int GM = uniform(p.band_m > 0 ? p.band_m : G_GROUP_M);
    int nband = (mtn + GM - 1) / GM;
    if (MODE == RAGGED_M && p.group_m > 0 && nband > 1 && mtn - (nband - 1) * GM < GM / 2) --nband;
    nband = uniform(nband);
    const int band = min(local / (GM * ntiles), nband - 1);
    const int within = local - band * GM * ntiles;
    const int gm = band == nband - 1 ? mtn - band * GM : GM;
    const int mt = band * GM + within % gm;
    t.nt = within / gm;
    t.off = uniform(group_off(ld_uniform(p.offs, t.e)));
    t.m_valid = MODE == RAGGED_M ? uniform(group_size(ld_uniform(p.sizes, t.e), t.off)) : p.M;
    t.m0 = mt * G_BM;
    // K range in bytes.  RAGGED_M: [0, K).  RAGGED_K: the expert's token span
    // [off, off + roundup32(size)) of the column forms; the loop starts at the slice
    // boundary below it and the chunks outside the span load as zeros.
    auto rows_left = [](int n, int cap) { return n < 0 ? 0 : (n > cap ? cap : n); };
    const uint8_t* bmat;
    if constexpr (MODE == RAGGED_M) {
      t.kbase = 0; t.klo = 0; t.khi = p.K * ELEM;
      t.A = p.A + (int64_t(t.off) + t.m0) * p.lda;
      bmat = ld_uniform(p.Bt, t.e);
    } else {
      const int span = uniform(group_size(((group_size(ld_uniform(p.sizes, t.e), t.off) + 31) / 32) * 32, t.off));
      t.klo = t.off * ELEM;
      t.khi = (t.off + span) * ELEM;
      t.kbase = span > 0 ? (t.klo / G_BKB) * G_BKB : t.klo;
      t.A = p.A + int64_t(t.m0) * p.lda;
      bmat = p.B;
    }
    t.arec = uint32_t(rows_left(t.m_valid - t.m0, G_BM)) * uint32_t(p.lda);
    if constexpr (EPI == EPI_SWIGLU) {
      t.nb = t.nt * (G_BN / 2);
      t.B = bmat + int64_t(t.nb) * p.ldb;
      t.brec = uint32_t(rows_left(p.F - t.nb, G_BN / 2)) * uint32_t(p.ldb);
    } else {
      t.nb = t.nt * G_BN + quarter * BW;
      t.B = bmat + int64_t(t.nb) * p.ldb;
      t.brec = uint32_t(rows_left(p.N - t.nb, BW)) * uint32_t(p.ldb);
    }
    t.nkt = (t.khi - t.kbase + G_BKB - 1) / G_BKB;
    if constexpr (MX) {
      // packed scales: dword (j, row) at row + j * ld holds the 4 blocks of K elements
      // [128j, 128j + 128); slice kt is group kbase/128 + kt
      if constexpr (MODE == RAGGED_M) {
        t.sa_rows = t.off + t.m0;
        t.sb_rows = int64_t(t.e) * p.bsp_estride;
      } else {
        t.sa_rows = t.m0;
        t.sb_rows = 0;
      }
    }
    return t;
  };


  // ---- loader geometry: wave instruction i (0..7) fills LDS rows [(wave*8+i)*8, +8) of
  // a 256-row operand tile, 1 KB contiguous (lane l -> row +l/8, LDS chunk l%8), so every
  // lane group of 8 reads one whole 128-byte line.  The lane loads the global chunk that
  // the swizzle maps to that LDS chunk: with row = 8q + l/8, (row/2) mod 8 =
  // 4*(q mod 2) + l/16, i.e. chunk (l%8) ^ (l/16) for even i and that ^ 4 for odd i.
  // Rows past the valid ones fall outside the resource's record bound and chunks
  // outside the K range get the top offset bit: both read zeros, so tails need no extra
  // path.  Lane offsets (row start + chunk) relative to the tile's first row, for even
  // and odd instructions; instruction i adds i*8 rows.
  const int lchunk0 = (lane & 7) ^ (lane >> 4);
  const int arow0 = wave * 64 + (lane >> 3);
  const int brow0 = (EPI == EPI_SWIGLU ? (wave & 1) * 64 : wave * (BW / 4)) + (lane >> 3);
  const uint32_t a_lane[2] = {uint32_t(arow0) * uint32_t(p.lda) + lchunk0 * 16,
                              uint32_t(arow0) * uint32_t(p.lda) + (lchunk0 ^ 4) * 16};
  const uint32_t b_lane[2] = {uint32_t(brow0) * uint32_t(p.ldb) + lchunk0 * 16,
                              uint32_t(brow0) * uint32_t(p.ldb) + (lchunk0 ^ 4) * 16};
  const uint32_t lda8 = uniform(int(8 * p.lda)), ldb8 = uniform(int(8 * p.ldb));

  // One K slice of tile t into LDS stage `stage` (operands and, MX, its scales); past
  // the last slice every lane is out of range and loads zeros.  prep_slice computes the
  // slice's resources and offsets; dma_operand(i) issues operand instruction i (0..7 A,
  // 8..15 B) so that the K loop can spread them between its MFMAs.
  constexpr int DMA_PER_SLICE = NOPS + (MX ? 1 : 0);   // VMEM operations of one slice
  struct SliceDma {
    i32x4 rA, rB, rS;
    uint32_t kadd, out0, out1, la, lb, ls, so;
  };
  auto prep_slice = [&](const Tile& t, int kt, int stage) {
    SliceDma c;
    c.rA = make_rsrc_n(t.A, t.arec);
    // SwiGLU: waves 0, 1 load the gate rows, waves 2, 3 the up rows (F rows further)
    const uint8_t* bb = t.B;
    if constexpr (EPI == EPI_SWIGLU) {
      if (wave >= 2) bb += int64_t(p.F) * p.ldb;
    }
    c.rB = make_rsrc_n(bb, t.brec);
    const int kslice = t.kbase + kt * G_BKB;         // first byte of the slice
    // this lane's chunk for even and odd instructions (the lane offsets hold the chunk
    // term); outside [klo, khi) the top offset bit is set
    const int kb0 = kslice + lchunk0 * 16;
    const int kb1 = kslice + (lchunk0 ^ 4) * 16;
    c.out0 = ((uint32_t(kb0 - t.klo) | uint32_t(t.khi - 1 - kb0)) >> 31) << 31;
    c.out1 = ((uint32_t(kb1 - t.klo) | uint32_t(t.khi - 1 - kb1)) >> 31) << 31;
    c.kadd = uint32_t(kslice);
    // A: 64 rows per wave (8 instructions of 8 rows); B: BW / 4 rows per wave, stored at
    // B row wave * BW / 4 of the stage (SwiGLU: waves 0, 1 the gate rows, 2, 3 the up rows)
    c.la = lds_base + stage * G_STAGE_BYTES + wave * 8 * 1024;
    c.lb = lds_base + stage * G_STAGE_BYTES + G_BM * G_BKB + wave * (BW / 4) * G_BKB;
    if constexpr (MX) {
      // wave w brings 128 rows of scale dwords (lanes 0..31, 16 B = 4 rows each):
      // A rows (w&1)*128.. for w < 2, B rows for w >= 2; the dwords of the slice's
      // 128-element group (a slice is exactly one group)
      const bool slice_ok = kt < t.nkt;
      const int half = wave & 1;
      const int64_t j = t.kbase / G_BKB + kt;
      int64_t dw;             // first dword of the 128 rows
      const uint32_t* base;
      uint32_t bytes;
      if (wave < 2) {
        dw = t.sa_rows + j * p.asp_ld + half * 128;
        base = p.Asp;
        bytes = p.asp_bytes;
      } else {
        int r0;
        if constexpr (EPI == EPI_SWIGLU) r0 = half == 0 ? t.nb : p.F + t.nb;
        else r0 = t.nb + half * 128;
        dw = t.sb_rows + j * p.bsp_ld + r0;
        base = p.Bsp;
        bytes = p.bsp_bytes;
      }
      c.rS = make_rsrc_n(base, bytes);
      // lanes of 4 rows each: 32 (128 rows), fewer for the B rows of a narrow work item
      constexpr int kBLanes0 = BW >= 128 ? 32 : BW / 4, kBLanes1 = BW >= 256 ? 32 : (BW > 128 ? (BW - 128) / 4 : 0);
      const int nlanes = wave < 2 ? 32 : (half == 0 ? kBLanes0 : kBLanes1);
      c.so = (slice_ok && lane < nlanes) ? uint32_t(dw * 4) + lane * 16 : kInvalid;
      c.ls = lds_base + G_SCALE_BASE + stage * G_SCALE_STAGE + wave * 1024;
    }
    return c;
  };
  auto dma_operand = [&](const SliceDma& c, int i) {
    const uint32_t out = (i & 1) ? c.out1 : c.out0;
    if (i < 8) dma16(c.rA, c.la + i * 1024, (a_lane[i & 1] + i * lda8 + c.kadd) | out);
    else dma16(c.rB, c.lb + (i - 8) * 1024, (b_lane[i & 1] + (i - 8) * ldb8 + c.kadd) | out);
  };
  auto dma_scale = [&](const SliceDma& c) {
    if constexpr (MX) dma16(c.rS, c.ls, c.so);
  };
  auto issue_slice = [&](const Tile& t, int kt, int stage) {
    const SliceDma c = prep_slice(t, kt, stage);
#pragma unroll
    for (int i = 0; i < NOPS; ++i) dma_operand(c, i);
    dma_scale(c);
  };

  int brow_tile[WNB];
#pragma unroll
  for (int ni = 0; ni < WNB; ++ni) {
    if constexpr (EPI == EPI_SWIGLU) {
      constexpr int hb = G_WNB / 2;
      brow_tile[ni] = ni < hb ? (wn * hb + ni) * 32 : G_BN / 2 + (wn * hb + ni - hb) * 32;
    } else {
      brow_tile[ni] = (wn * WNB + ni) * 32;
    }
  }

  // MFMA operand fragments of one K step, read from the swizzled LDS tile:
  //   MX  : 64-element step s (of 2); lane (hi, l32) takes 16-byte chunks 4s + hi and
  //         4s + hi + 2 of its row
  //   BF16: 16-element step s (of 4); lane takes chunk 2s + hi
  typedef typename std::conditional<MX, i32x8, bf16x8>::type frag_t;
  constexpr int NSTEP = MX ? 2 : 4;
  auto read_frags = [&](const uint8_t* sA, const uint8_t* sB, int s, frag_t* af, frag_t* bfr) {
#pragma unroll
    for (int mi = 0; mi < G_WMB; ++mi) {
      const int row = (wm * G_WMB + mi) * 32 + l32;
      if constexpr (MX) {
        const int c = 4 * s + hi;
        const uint4 x0 = *reinterpret_cast<const uint4*>(sA + swz(row, c));
        const uint4 x1 = *reinterpret_cast<const uint4*>(sA + swz(row, c + 2));
        af[mi] = i32x8{int(x0.x), int(x0.y), int(x0.z), int(x0.w), int(x1.x), int(x1.y), int(x1.z), int(x1.w)};
      } else {
        af[mi] = *reinterpret_cast<const bf16x8*>(sA + swz(row, s * 2 + hi));
      }
    }
#pragma unroll
    for (int ni = 0; ni < WNB; ++ni) {
      const int row = brow_tile[ni] + l32;
      if constexpr (MX) {
        const int c = 4 * s + hi;
        const uint4 x0 = *reinterpret_cast<const uint4*>(sB + swz(row, c));
        const uint4 x1 = *reinterpret_cast<const uint4*>(sB + swz(row, c + 2));
        bfr[ni] = i32x8{int(x0.x), int(x0.y), int(x0.z), int(x0.w), int(x1.x), int(x1.y), int(x1.z), int(x1.w)};
      } else {
        bfr[ni] = *reinterpret_cast<const bf16x8*>(sB + swz(row, s * 2 + hi));
      }
    }
  };

  Tile cur = decode(vid);
  // next-tile slices issued before the epilogue (see there)
  constexpr int G_PREFETCH = (OUT == OUT_F32_ACC || EPI == EPI_SWIGLU_BWD) ? 0 : 1;
  int cur_issued = 0;   // slices of `cur` (from 0) already on their way into their stages
  for (int item = vid; item < items; item += nwg) {
    rederive_lane();
    const Tile nxt = decode(item + nwg);
    const int e = cur.e, nt = cur.nt, nb = cur.nb, off = cur.off, m_valid = cur.m_valid, m0 = cur.m0, nkt = cur.nkt;
    // SwiGLU: the probability of tile row tid, loaded now so that its latency hides
    // behind the K loop (it is staged in LDS for the epilogue)
    float my_prob = 0.f;
    if constexpr (EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_BWD) {
      if (m0 + tid < m_valid) my_prob = p.prob[off + m0 + tid];
    }

    f32x16 acc[G_WMB][WNB];
#pragma unroll
    for (int mi = 0; mi < G_WMB; ++mi)
#pragma unroll
      for (int ni = 0; ni < WNB; ++ni)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;

    // The MFMAs of one slice, K step by K step (MX: in K step s, elements 64s..64s+63 of
    // the slice's 128-element group, lane hi scales K block 2s + hi: byte 2s + hi of the
    // group's dword, shifted down to byte 0, op_sel 0).  Before MFMA BAR_AT every wave
    // has its fragments (lds_barrier), so the stage is refilled from there on: the scale
    // DMA first, then the 16 operand DMAs spread evenly over the remaining MFMAs.  A
    // CU's texture-address path moves about 54 bytes per clock, so a slice's DMAs need
    // well over half of the slice's MFMA time; packed closer they fill its queue and
    // stall the issuing wave (measured on MI355X).
    constexpr int NMFMA = NSTEP * G_WMB * WNB;
    constexpr int BAR_AT = NMFMA * G_BAR_AT32 / 32;
    auto mfma_slice = [&](frag_t (*af)[G_WMB], frag_t (*bfr)[WNB], const uint32_t* sa, const uint32_t* sb,
                          const SliceDma& nx) {
      static_for<0, NMFMA>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        constexpr int s = i / (G_WMB * WNB);
        constexpr int mi = (i % (G_WMB * WNB)) / WNB;
        constexpr int ni = i % WNB;
        if constexpr (i == BAR_AT) {
          __builtin_amdgcn_sched_barrier(0);
          lds_barrier();   // every wave is done with this stage
          dma_scale(nx);
          __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (MX) {
          const int sh = 8 * (2 * s + hi);
          const int xa = int(sa[mi] >> sh);
          const int xb = int(sb[ni] >> sh);
          acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[s][mi], bfr[s][ni], acc[mi][ni], 0, 0, 0, xa, 0, xb);
        } else {
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[s][mi], bfr[s][ni], acc[mi][ni], 0, 0, 0);
        }
        if constexpr (i >= BAR_AT) {
          constexpr int n = NMFMA - BAR_AT;
          constexpr int d0 = NOPS * (i - BAR_AT) / n, d1 = NOPS * (i - BAR_AT + 1) / n;
          if constexpr (d1 > d0) {
            __builtin_amdgcn_sched_barrier(0);
            static_for<d0, d1>([&](auto dc) { dma_operand(nx, decltype(dc)::value); });
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      });
    };

    // ---- K loop over two LDS stages.  A wave reads every fragment and scale of slice kt
    // into registers at the top of iteration kt; those reads have landed by the end of the
    // first half of the K steps (the LDS needs about as long to serve them as the MFMAs of
    // that half take).  From there on the stage is dead, so once every wave has passed
    // that point it is refilled with slice kt+2.  A slice thus has one and a half
    // iterations to arrive instead of one, with the same LDS.  The two slices past the
    // tile's last are issued too, with every lane out of range (they land as zeros and
    // touch no memory), so that every iteration waits on the same count.
    if (cur_issued == 0 && nkt > 0) {
      lds_barrier();   // no wave still reads a stage
      issue_slice(cur, 0, 0);
      issue_slice(cur, 1, 1);
      vm_barrier<DMA_PER_SLICE>();   // slice 0 resident, slice 1 may be on its way
    } else if (cur_issued == 1) {
      issue_slice(cur, 1, 1);
      vm_barrier<DMA_PER_SLICE>();   // slice 0 and the epilogue's stores done
    } else {
      vm_barrier<0>();               // prefetched slices 0, 1 and the epilogue's stores
    }
    for (int kt = 0; kt < nkt; ++kt) {
      const int stage = kt & (G_STAGES - 1);
      const uint8_t* sA = smem + stage * G_STAGE_BYTES;
      const uint8_t* sB = sA + G_BM * G_BKB;
      uint32_t sa[G_WMB], sb[WNB];
      if constexpr (MX) {
        const uint8_t* sS = smem + G_SCALE_BASE + stage * G_SCALE_STAGE;
#pragma unroll
        for (int mi = 0; mi < G_WMB; ++mi) {
          const int r = (wm * G_WMB + mi) * 32 + l32;
          sa[mi] = *reinterpret_cast<const uint32_t*>(sS + (r >> 7) * 1024 + (r & 127) * 4);
        }
#pragma unroll
        for (int ni = 0; ni < WNB; ++ni) {
          const int r = brow_tile[ni] + l32;
          sb[ni] = *reinterpret_cast<const uint32_t*>(sS + 2048 + (r >> 7) * 1024 + (r & 127) * 4);
        }
      }
      frag_t af[NSTEP][G_WMB], bfr[NSTEP][WNB];
#pragma unroll
      for (int s = 0; s < NSTEP; ++s) read_frags(sA, sB, s, af[s], bfr[s]);
      const SliceDma nx = prep_slice(cur, kt + G_STAGES, stage);
      mfma_slice(af, bfr, sa, sb, nx);
      __builtin_amdgcn_sched_barrier(0);
      vm_barrier<DMA_PER_SLICE>();   // slice kt+1 resident (kt+2 still on its way)
    }
    __builtin_amdgcn_s_waitcnt(0);   // the past-the-end (all-zero) slices have landed
    acc_settle();                    // the last MFMA results are readable
    rederive_lane();
    // both stages are free (the loop ends on a barrier): start the next tile's first
    // slice now so that its latency hides behind the epilogue (which uses no stage
    // memory); slice 1 follows at the top of the next tile (one or two slices ahead
    // measure the same on MI355X, and one leaves more of the 63 vector-memory operations
    // a wave may have outstanding to the epilogue's stores).  None when the epilogue
    // reads the output back: those loads would queue behind the slice.
    cur_issued = 0;
    if (nxt.valid && nxt.nkt > 0 && G_PREFETCH > 0) {
      issue_slice(nxt, 0, 0);
      if constexpr (G_PREFETCH > 1) issue_slice(nxt, 1, 1);
      cur_issued = G_PREFETCH;
    }

    // ---------------------------------------------------------------- epilogues
    // Accumulator element r of block (mi, ni) is row 8*(r/4) + 4*hi + (r%4) and column
    // l32 of that 32 x 32 block.
    const int wrow0 = m0 + wm * G_WMB * 32;   // wave's first row (group-local)
    if constexpr (EPI == EPI_STORE) {
      // Lane (hi, l32) stores column l32 of each 32 x 32 block, rows 8*(r/4) + 4*hi +
      // r%4; the record bound of the resource ends at the last valid row of the wave's
      // 128-row span and lanes whose column is past N get an offset beyond every bound.
      constexpr int ESZ = OUT == OUT_BF16 ? 2 : 4;
      int vr = m_valid - wrow0;
      vr = uniform(vr < 0 ? 0 : (vr > G_WMB * 32 ? G_WMB * 32 : vr));
      uint8_t* cbase;
      if constexpr (MODE == RAGGED_M) {
        cbase = static_cast<uint8_t*>(p.C) + (int64_t(off) + wrow0) * p.ldc * ESZ;
      } else {
        cbase = static_cast<uint8_t*>(ld_uniform(p.Ct, e)) +
                int64_t(wrow0) * p.ldc * ESZ;
      }
      const uint32_t rowb = uint32_t(p.ldc) * ESZ;
      const __amdgpu_buffer_rsrc_t rC = __builtin_amdgcn_make_buffer_rsrc(cbase, 0, int(uint32_t(vr) * rowb), kRsrcFlags);
      static_for<0, G_WMB>([&](auto mic) {
        constexpr int mi = decltype(mic)::value;
        if (wrow0 + mi * 32 >= m_valid) return;
        static_for<0, WNB>([&](auto nic) {
          constexpr int ni = decltype(nic)::value;
          const int col = nb + brow_tile[ni] + l32;
          const uint32_t lo = col < p.N ? uint32_t(col) * ESZ + uint32_t(4 * hi) * rowb : kInvalid;
          constexpr int pol = MODE == RAGGED_K ? kNonTemporal : 0;   // gradients: written once
          if constexpr (OUT == OUT_F32_ACC) {
            uint32_t old[16];
#pragma unroll
            for (int r = 0; r < 16; ++r)
              old[r] = __builtin_amdgcn_raw_buffer_load_b32(rC, int(lo + uint32_t(mi * 32 + 8 * (r >> 2) + (r & 3)) * rowb), 0, pol);
#pragma unroll
            for (int r = 0; r < 16; ++r)
              __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc_read(acc[mi][ni][r]) + __uint_as_float(old[r])), rC,
                                                    int(lo + uint32_t(mi * 32 + 8 * (r >> 2) + (r & 3)) * rowb), 0, pol);
          } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int o = int(lo + uint32_t(mi * 32 + 8 * (r >> 2) + (r & 3)) * rowb);
              if constexpr (OUT == OUT_BF16)
                __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(acc_read(acc[mi][ni][r])), rC, o, 0, pol);
              else
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[mi][ni][r]), rC, o, 0, pol);
            }
          }
          __builtin_amdgcn_sched_barrier(0);   // one block at a time (register peak)
        });
      });
    } else if constexpr (EPI == EPI_SWIGLU) {
      // h = p * silu(G) * U over the wave's 128 rows x 64 ffn columns, written as the row
      // form (blocks of 32 along F) and, in training, the column form (blocks of 32 rows)
      // plus G and U in bf16.  Lanes 0..31 of a half-wave hold 32 consecutive columns of
      // one row, so a row block's amax is a half-wave all-reduce; a lane holds 16 rows of
      // one column and the two half-waves together a column's 32-row block.  Row-form
      // stores go through buffer resources whose record bound ends at the group's last
      // row, so rows past it are dropped by the hardware range check; 32-row blocks past
      // the group and 32-column blocks past F are skipped whole (wave-uniform).
      s_prob[tid] = my_prob;
      lds_barrier();   // (the next tile's first slice stays in flight)
      constexpr int hb = G_WNB / 2;
      const int F = p.F;
      const int F2 = 2 * F;
      const bool train = p.saved_gu != nullptr;
      int vr = m_valid - wrow0;                         // valid rows of the wave's span
      vr = uniform(vr < 0 ? 0 : (vr > G_WMB * 32 ? G_WMB * 32 : vr));
      const int64_t grow0 = int64_t(off) + wrow0;       // permuted row of span row 0
      auto rsrc = [](const void* base, uint32_t bytes) {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(bytes), kRsrcFlags);
      };
      __amdgpu_buffer_rsrc_t rH, rHs, rGU;
      if constexpr (MX) {
        rH = rsrc(p.h_codes + grow0 * F, uint32_t(vr) * F);
        rHs = rsrc(p.h_scales + grow0 * (F / 32), uint32_t(vr) * (F / 32));
      } else {
        rH = rsrc(p.h_bf16 + grow0 * F, uint32_t(vr) * F * 2);
        rHs = rH;
      }
      rGU = rsrc(train ? p.saved_gu + grow0 * F2 : p.saved_gu, train ? uint32_t(vr) * F2 * 2 : 0u);
      static_for<0, G_WMB>([&](auto mic) {
        constexpr int mi = decltype(mic)::value;
        const int rb = mi * 32;                          // block row within the span
        if (wrow0 + rb >= m_valid) return;               // past the group and its padding
        // rows of this lane's 16 values within the span: rb + 8*(r/4) + 4*hi + r%4
        float pr[16];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float4 q = *reinterpret_cast<const float4*>(&s_prob[wm * G_WMB * 32 + rb + 8 * g + 4 * hi]);
          pr[4 * g] = q.x; pr[4 * g + 1] = q.y; pr[4 * g + 2] = q.z; pr[4 * g + 3] = q.w;
        }
        static_for<0, hb>([&](auto jc) {
          constexpr int j = decltype(jc)::value;
          const int fb0 = nt * (G_BN / 2) + (wn * hb + j) * 32;   // first column of the block
          if (fb0 >= F) return;
          const int f = fb0 + l32;
          auto lrow = [&](int r) { return rb + 8 * (r >> 2) + 4 * hi + (r & 3); };
          // Neighbouring lanes (columns c, c+1) trade halves so that a lane holds one row x
          // two columns instead of two rows x one column: bf16 pairs then leave as dword
          // stores (even lane: row r, odd lane: row r + 1, columns c & ~1, +1).  A lane
          // packs its rows (r, r + 1) as one dword, reads its neighbour's by DPP and picks
          // the halves with one byte permute (even: own low, neighbour's low; odd:
          // neighbour's high, own high).
          const bool odd = (l32 & 1) != 0;
          const int fpair = f & ~1;
          // the lane's share of the MXFP8 offsets (as in the backward's epilogue)
          const int q2 = l32 >> 1;
          const int row_lane = (4 * hi + (l32 & 3)) * F + (l32 & ~3);
          const uint32_t sc_lane = (l32 & 1) == 0 ? uint32_t((8 * (q2 >> 2) + 4 * hi + (q2 & 3)) * (F / 32)) : kInvalid;
          const uint32_t psel = odd ? 0x03020706u : 0x05040100u;
          auto pair2 = [&](float v0, float v1) {
            const uint32_t own = bf16x2(v0, v1);
            const uint32_t nb = uint32_t(__builtin_amdgcn_mov_dpp(int(own), 0xB1, 0xf, 0xf, false));
            return __builtin_amdgcn_perm(nb, own, psel);
          };
          float h[16];
#pragma unroll
          for (int r = 0; r < 16; r += 2) {
            const float G0 = acc_read(acc[mi][j][r]), G1 = acc_read(acc[mi][j][r + 1]);
            const float U0 = acc_read(acc[mi][j + hb][r]), U1 = acc_read(acc[mi][j + hb][r + 1]);
            if (train) {
              const int o = ((lrow(r) + (odd ? 1 : 0)) * F2 + fpair) * 2;
              __builtin_amdgcn_raw_buffer_store_b32(pair2(G0, G1), rGU, o, 0, 0);
              __builtin_amdgcn_raw_buffer_store_b32(pair2(U0, U1), rGU, o + 2 * F, 0, 0);
            }
            h[r] = pr[r] * (G0 * __builtin_amdgcn_rcpf(1.f + __expf(-G0))) * U0;
            h[r + 1] = pr[r + 1] * (G1 * __builtin_amdgcn_rcpf(1.f + __expf(-G1))) * U1;
          }
          if constexpr (MX) {
            // row form: one scale per (row, 32-column block), shared by the half-wave
            float inv[16];
            const uint32_t sc = row_block_inv16(h, l32, inv, s_inv + wave * 32 + hi * 16);   // sc: row l32 / 2
            // codes of 4 consecutive rows: a lane holds its column's 4 codes (bytes =
            // rows); a 4 x 4 byte transpose inside each quad of lanes (16-bit halves with
            // the lane 2 apart, then bytes with the lane 1 apart) leaves row (l32 % 4) of
            // the quad's 4 columns in the lane: one dword store per lane and 4 rows
            // the 16-bit halves (one v_perm_b32, bytes 0-3 of v, 4-7 of x): lanes with
            // l32 & 2 == 0 keep their low half under the partner's low half, the others take
            // the partner's high half under their own high half
            const uint32_t sel16 = (l32 & 2) == 0 ? 0x05040100u : 0x03020706u;
            const uint32_t sel = odd ? 0x03070105u : 0x06020400u;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              uint32_t v = e4m3x4(h[4 * g] * inv[4 * g], h[4 * g + 1] * inv[4 * g + 1], h[4 * g + 2] * inv[4 * g + 2],
                                  h[4 * g + 3] * inv[4 * g + 3]);
              const uint32_t x = uint32_t(__builtin_amdgcn_mov_dpp(int(v), 0x4E, 0xf, 0xf, false));
              v = __builtin_amdgcn_perm(x, v, sel16);   // low half: own | partner's; high: partner's | own
              const uint32_t y = uint32_t(__builtin_amdgcn_mov_dpp(int(v), 0xB1, 0xf, 0xf, false));
              v = __builtin_amdgcn_perm(y, v, sel);
              __builtin_amdgcn_raw_buffer_store_b32(v, rH, (rb + 8 * g) * F + fb0 + row_lane, 0, 0);
            }
            // the even lanes write the scale of their row l32 / 2
            const uint32_t so = sc_lane == kInvalid ? kInvalid : sc_lane + uint32_t(rb * (F / 32) + fb0 / 32);
            __builtin_amdgcn_raw_buffer_store_b8(uint8_t(sc), rHs, so, 0, 0);
          } else {
#pragma unroll
            for (int r = 0; r < 16; r += 2)
              __builtin_amdgcn_raw_buffer_store_b32(pair2(h[r], h[r + 1]), rH, ((lrow(r) + (odd ? 1 : 0)) * F + fpair) * 2,
                                                    0, 0);
          }
          if (train) {
            // column form of column f, rows [rb, rb + 32): after the half-wave swaps,
            // lane hi holds rows 16*hi .. 16*hi + 15 in order
            const int64_t cbase = int64_t(fb0) * p.Rp + grow0 + rb + (int64_t(l32) * p.Rp + 16 * hi);   // element index
            if constexpr (MX) {
              float cmax = 0.f;
#pragma unroll
              for (int r = 0; r < 16; ++r) cmax = fmaxf(cmax, fabsf(h[r]));
              cmax = max_xor32(cmax);
              const uint32_t s = mx_scale_byte(cmax);
              const float inv = mx_inv_scale(s);
              uint32_t c[4];
#pragma unroll
              for (int g = 0; g < 4; ++g) c[g] = e4m3x4(h[4 * g] * inv, h[4 * g + 1] * inv, h[4 * g + 2] * inv, h[4 * g + 3] * inv);
              const U32Pair x02 = permlane32_swap(c[0], c[2]);
              const U32Pair x13 = permlane32_swap(c[1], c[3]);
              *reinterpret_cast<uint4*>(p.hc_codes + cbase) = make_uint4(x02.a, x02.b, x13.a, x13.b);
              if (hi == 0) p.hc_scales[int64_t(f) * (p.Rp / 32) + (grow0 + rb) / 32] = uint8_t(s);
            } else {
              uint32_t c[8];
#pragma unroll
              for (int g = 0; g < 4; ++g) {
                c[2 * g] = bf16x2(h[4 * g], h[4 * g + 1]);
                c[2 * g + 1] = bf16x2(h[4 * g + 2], h[4 * g + 3]);
              }
              const U32Pair a0 = permlane32_swap(c[0], c[4]), a1 = permlane32_swap(c[1], c[5]);
              const U32Pair b0 = permlane32_swap(c[2], c[6]), b1 = permlane32_swap(c[3], c[7]);
              uint4* dst = reinterpret_cast<uint4*>(p.hc_bf16 + cbase);
              dst[0] = make_uint4(a0.a, a1.a, a0.b, a1.b);
              dst[1] = make_uint4(b0.a, b1.a, b0.b, b1.b);
            }
          }
          if constexpr (G_EPI_GROUP == 1 || (j % G_EPI_GROUP) == G_EPI_GROUP - 1) __builtin_amdgcn_sched_barrier(0);   // blocks in groups (register peak)
        });
      });
    } else if constexpr (EPI == EPI_SWIGLU_BWD) {
      // dh = dY W_down sits in the accumulators: lane (hi, l32) of block (mi, ni) holds ffn
      // column fw0 + 32 ni + l32 of span rows 32 mi + 8 (r/4) + 4 hi + r%4.  Per 32-row
      // block, G and U of the wave's 32 rows x 128 columns come into this wave's share of
      // the (now idle) stage memory by LDS DMA, two buffers so that block mi + 1 streams in
      // while mi is processed.  Then dU = dh p silu(G), dG = dh p U silu'(G) and the row
      // sums of dh silu(G) U (d_prob), with dG (columns f) and dU (columns F + f) written in
      // row form (32-column blocks: the half-wave reduce-scatter of the forward) and column
      // form (32-row blocks: 16 rows in a lane, 16 in the lane 32 apart), MXFP8 or bf16.
      s_prob[tid] = my_prob;
      lds_barrier();
      const int F = p.F, F2 = 2 * F;
      int vr = m_valid - wrow0;                         // valid rows of the wave's span
      vr = uniform(vr < 0 ? 0 : (vr > G_WMB * 32 ? G_WMB * 32 : vr));
      const int64_t grow0 = int64_t(off) + wrow0;       // permuted row of span row 0
      const int fw0 = nt * G_BN + wn * (G_WNB * 32);    // the wave's first ffn column
      // staging: per buffer G then U, each 8 DMA blocks of 4 rows x 256 bytes, 1088 bytes
      // apart (rows 4 apart, read by the two half-waves, then fall 16 banks apart)
      constexpr int GS = 1088, GA = 8 * GS, GB = 2 * GA;
      static_assert(G_WAVES_M * G_WAVES_N * 2 * GB <= G_DYN_LDS, "G/U staging exceeds the stage memory");
      const uint32_t wl = lds_base + uint32_t(wave * 2 * GB);
      const uint8_t* wsm = smem + wave * 2 * GB;
      const i32x4 rIn = make_rsrc_n(reinterpret_cast<const uint8_t*>(p.gu_in + grow0 * F2), uint32_t(vr) * uint32_t(F2) * 2u);
      // DMA instruction j of a block: lane L brings row 4j + L/16, columns fw0 + 8 (L%16) ..+7
      const uint32_t dl = uint32_t(lane >> 4) * uint32_t(F2) * 2u + uint32_t(fw0 + (lane & 15) * 8) * 2u;
      auto issue_gu = [&](int mi, int buf) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t o = uint32_t(mi * 32 + 4 * j) * uint32_t(F2) * 2u + dl;
          dma16_nt(rIn, wl + uint32_t(buf * GB + j * GS), o);                      // G
          dma16_nt(rIn, wl + uint32_t(buf * GB + GA + j * GS), o + uint32_t(F) * 2u);   // U
        }
      };
      auto rsrc = [](const void* base, uint32_t bytes) {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(bytes), kRsrcFlags);
      };
      // outputs in MXFP8 (codes + block scales) or in bf16: the bf16 path of BF16 operands,
      // and of MX operands with OUT_BF16 (FP8 with one scale per tensor, whose scale needs
      // all of [dG dU] first); the bf16 column form only when asked for
      constexpr bool MXO = MX && OUT != OUT_BF16;
      const bool col_out = MXO || p.dgu_col_bf16 != nullptr;
      __amdgpu_buffer_rsrc_t rR, rRs;
      if constexpr (MXO) {
        rR = rsrc(p.dgu_row_codes + grow0 * F2, uint32_t(vr) * F2);
        rRs = rsrc(p.dgu_row_scales + grow0 * (F2 / 32), uint32_t(vr) * (F2 / 32));
      } else {
        rR = rsrc(p.dgu_row_bf16 + grow0 * F2, uint32_t(vr) * F2 * 2);
        rRs = rR;
      }
      const bool odd = (l32 & 1) != 0;
      const uint32_t psel = odd ? 0x03020706u : 0x05040100u;
      auto pair2 = [&](float v0, float v1) {
        const uint32_t own = bf16x2(v0, v1);
        const uint32_t nb = uint32_t(__builtin_amdgcn_mov_dpp(int(own), 0xB1, 0xf, 0xf, false));
        return __builtin_amdgcn_perm(nb, own, psel);
      };
      // the lane's share of the MXFP8 output offsets, once per tile (the block's share is
      // wave-uniform): the row-form dword of rows 4g + (l32 % 4) and columns l32 & ~3, the
      // scale byte of row l32 / 2 (even lanes), the column form's 16 rows from 16 hi
      const int q2 = l32 >> 1;
      const int row_lane = (4 * hi + (l32 & 3)) * F2 + (l32 & ~3);
      const uint32_t sc_lane = (l32 & 1) == 0 ? uint32_t((8 * (q2 >> 2) + 4 * hi + (q2 & 3)) * (F2 / 32)) : kInvalid;
      const int64_t col_lane = int64_t(l32) * p.Rp + 16 * hi;
      const int lds_lane = hi * GS + 2 * l32;            // the lane's G, U element in a staged block
      if (vr > 0) {                                      // wave-uniform
      issue_gu(0, 0);
      issue_gu(1, 1);
      // One 32-row block.  With MXFP8 outputs the blocks run as a loop, not unrolled:
      // unrolled four times that epilogue was larger than the instruction cache two CUs
      // share (89 KB of code against 37 KB).  AGPR indexes are compile-time, so block mi's
      // accumulators are read in a uniform branch per value of mi (folded away when the
      // blocks are unrolled, as they stay for bf16 outputs, whose loop form spills).
      auto row_block = [&](const int mi) __attribute__((always_inline)) {
        const int buf = mi & 1;
        // block mi's G, U have landed (block mi + 1's, the newest 16 operations, may still
        // be on their way); asm with a memory clobber, so that no LDS read moves above it
        if (mi + 1 < G_WMB) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
        else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        const int rb = mi * 32;                          // block row within the span
        if (wrow0 + rb < m_valid) {                      // wave-uniform
          auto lrow = [&](int r) { return rb + 8 * (r >> 2) + 4 * hi + (r & 3); };
          float pr[16];
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const float4 q = *reinterpret_cast<const float4*>(&s_prob[wm * G_WMB * 32 + rb + 8 * g + 4 * hi]);
            pr[4 * g] = q.x; pr[4 * g + 1] = q.y; pr[4 * g + 2] = q.z; pr[4 * g + 3] = q.w;
          }
          float dps[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) dps[r] = 0.f;
          const uint8_t* gs = wsm + buf * GB;
          static_for<0, G_WNB>([&](auto nic) {
            constexpr int ni = decltype(nic)::value;
            const int fb0 = fw0 + ni * 32;                 // first column of the block
            if (fb0 >= F) return;                          // wave-uniform
            float dg[16], du[16], dhv[4];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              if ((r & 3) == 0) {                          // four accumulators at a time (register peak)
                static_for<0, G_WMB>([&](auto mc) {
                  constexpr int m = decltype(mc)::value;
                  if (mi == m) {                           // wave-uniform
#pragma unroll
                    for (int k = 0; k < 4; ++k) dhv[k] = acc_read(acc[m][ni][r + k]);
                  }
                });
              }
              // row 8 (r / 4) + 4 hi + r % 4 of the block: 4-row group 2 (r / 4) + hi, row r % 4 in it
              const int lo = 2 * (r >> 2) * GS + (r & 3) * 256 + ni * 64 + lds_lane;
              const float G = __uint_as_float(uint32_t(*reinterpret_cast<const uint16_t*>(gs + lo)) << 16);
              const float U = __uint_as_float(uint32_t(*reinterpret_cast<const uint16_t*>(gs + GA + lo)) << 16);
              const float dh = dhv[r & 3];
              const float sg = __builtin_amdgcn_rcpf(1.f + __expf(-G));
              const float sl = G * sg;                       // silu(G)
              const float t = dh * sl;
              dps[r] = fmaf(t, U, dps[r]);
              du[r] = t * pr[r];
              const float ds = fmaf(sl, 1.f - sg, sg);       // silu'(G) = sg (1 + G (1 - sg))
              dg[r] = (dh * pr[r]) * (U * ds);
            }
            // both arrays: h = 0 -> dG at column fb0 + l32, h = 1 -> dU at F + fb0 + l32
            static_for<0, 2>([&](auto hc) {
              constexpr int h = decltype(hc)::value;
              const float* v = h == 0 ? dg : du;
              const int cb = h * F + fb0;                    // first [dG dU] column of the block
              if constexpr (MXO) {
                float inv[16];
                const uint32_t sc = row_block_inv16(v, l32, inv, s_inv + wave * 32 + hi * 16);   // sc: row l32 / 2
                const uint32_t sel16 = (l32 & 2) == 0 ? 0x05040100u : 0x03020706u;   // halves, as in the forward
                const uint32_t sel = odd ? 0x03070105u : 0x06020400u;
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                  uint32_t w = e4m3x4(v[4 * g] * inv[4 * g], v[4 * g + 1] * inv[4 * g + 1], v[4 * g + 2] * inv[4 * g + 2],
                                      v[4 * g + 3] * inv[4 * g + 3]);
                  const uint32_t x = uint32_t(__builtin_amdgcn_mov_dpp(int(w), 0x4E, 0xf, 0xf, false));
                  w = __builtin_amdgcn_perm(x, w, sel16);
                  const uint32_t y = uint32_t(__builtin_amdgcn_mov_dpp(int(w), 0xB1, 0xf, 0xf, false));
                  w = __builtin_amdgcn_perm(y, w, sel);
                  __builtin_amdgcn_raw_buffer_store_b32(w, rR, (rb + 8 * g) * F2 + cb + row_lane, 0, 0);
                }
                const uint32_t so = sc_lane == kInvalid ? kInvalid : sc_lane + uint32_t(rb * (F2 / 32) + cb / 32);
                __builtin_amdgcn_raw_buffer_store_b8(uint8_t(sc), rRs, so, 0, 0);
                // column form of column cb + l32, rows [rb, rb + 32)
                const int64_t cbase = int64_t(cb) * p.Rp + grow0 + rb + col_lane;
                float cmax = 0.f;
#pragma unroll
                for (int r = 0; r < 16; ++r) cmax = fmaxf(cmax, fabsf(v[r]));
                cmax = max_xor32(cmax);
                const uint32_t s = mx_scale_byte(cmax);
                const float ic = mx_inv_scale(s);
                uint32_t c[4];
#pragma unroll
                for (int g = 0; g < 4; ++g) c[g] = e4m3x4(v[4 * g] * ic, v[4 * g + 1] * ic, v[4 * g + 2] * ic, v[4 * g + 3] * ic);
                const U32Pair x02 = permlane32_swap(c[0], c[2]);
                const U32Pair x13 = permlane32_swap(c[1], c[3]);
                *reinterpret_cast<uint4*>(p.dgu_col_codes + cbase) = make_uint4(x02.a, x02.b, x13.a, x13.b);
                if (hi == 0) p.dgu_col_scales[int64_t(cb + l32) * (p.Rp / 32) + (grow0 + rb) / 32] = uint8_t(s);
              } else {
                const int cpair = (cb + l32) & ~1;
#pragma unroll
                for (int r = 0; r < 16; r += 2)
                  __builtin_amdgcn_raw_buffer_store_b32(pair2(v[r], v[r + 1]), rR,
                                                        ((lrow(r) + (odd ? 1 : 0)) * F2 + cpair) * 2, 0, 0);
                if (!col_out) return;                       // wave-uniform
                const int64_t cbase = int64_t(cb + l32) * p.Rp + grow0 + rb + 16 * hi;
                uint32_t c[8];
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                  c[2 * g] = bf16x2(v[4 * g], v[4 * g + 1]);
                  c[2 * g + 1] = bf16x2(v[4 * g + 2], v[4 * g + 3]);
                }
                const U32Pair a0 = permlane32_swap(c[0], c[4]), a1 = permlane32_swap(c[1], c[5]);
                const U32Pair b0 = permlane32_swap(c[2], c[6]), b1 = permlane32_swap(c[3], c[7]);
                uint4* dst = reinterpret_cast<uint4*>(p.dgu_col_bf16 + cbase);
                dst[0] = make_uint4(a0.a, a1.a, a0.b, a1.b);
                dst[1] = make_uint4(b0.a, b1.a, b0.b, b1.b);
              }
            });
            if constexpr (G_EPI_GROUP == 1 || (ni % G_EPI_GROUP) == G_EPI_GROUP - 1) __builtin_amdgcn_sched_barrier(0);   // blocks in groups (register peak)
          });
          // d_prob partial of each row over the wave's 128 columns: lanes 2k, 2k + 1 hold row k
          const float ps = row_block_sum16(dps, l32);
          if ((l32 & 1) == 0 && wrow0 + lrow(l32 >> 1) < m_valid)
            p.dprob_part[(grow0 + lrow(l32 >> 1)) * p.dprob_nparts + nt * 2 + wn] = ps;
        }
        // the buffer takes block mi + 2 once this wave's reads of it have completed
        if (mi + 2 < G_WMB) {
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
          issue_gu(mi + 2, buf);
        }
      };
      if constexpr (MXO) {
#pragma clang loop unroll(disable)
        for (int mi = 0; mi < G_WMB; ++mi) row_block(mi);
      } else {
        static_for<0, G_WMB>([&](auto mic) { row_block(decltype(mic)::value); });
      }
      }
    }
    cur = nxt;
  }
  __builtin_amdgcn_s_waitcnt(0);   // no LDS DMA outlives the workgroup
}

// ---------------------------------------------------------------- host-side launch
static inline int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  hipGetDevice(&dev);
  if (dev < 0 || dev >= 64) dev = 0;
  if (cus[dev] == 0) {
    int v = 0;
    hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
    cus[dev] = v > 0 ? v : 256;
  }
  return cus[dev];
}

// Persistent launch: one workgroup per CU (the kernel holds one workgroup per CU by its
// LDS use), fewer when the tile count is smaller.
template <typename Kern>
static mge_status launch_gemm_kernel(Kern kern, const char* name, const GemmParams& p, hipStream_t s) {
  hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, G_DYN_LDS);
  int grid = device_cus();
  if (p.tiles_upper < grid) grid = p.tiles_upper;
  if (grid <= 0) return MGE_OK;
  ProfScope prof(s, name);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(G_THREADS), G_DYN_LDS, s, p);
  return hip_check(name);
}

// A plain-store ragged-M GEMM as two launches: the main kernel over the whole rounds of
// its grid, then the tail kernel over the rest as quarter-width work items (each kernel
// finds its share on the device: the tile count depends on the group sizes there).
template <typename KernMain, typename KernTail>
static mge_status launch_gemm_split(KernMain kmain, KernTail ktail, const char* name, const GemmParams& p0,
                                    hipStream_t s) {
  hipFuncSetAttribute(reinterpret_cast<const void*>(kmain), hipFuncAttributeMaxDynamicSharedMemorySize, G_DYN_LDS);
  hipFuncSetAttribute(reinterpret_cast<const void*>(ktail), hipFuncAttributeMaxDynamicSharedMemorySize, G_DYN_LDS);
  const int cus = device_cus();
  int grid = cus;
  if (p0.tiles_upper < grid) grid = p0.tiles_upper;
  if (grid <= 0) return MGE_OK;
  GemmParams p = p0;
  p.tail_split = G_TAIL_SPLIT;
  p.grid_main = grid;
  {
    ProfScope prof(s, name);
    hipLaunchKernelGGL(kmain, dim3(grid), dim3(G_THREADS), G_DYN_LDS, s, p);
  }
  mge_status st = hip_check(name);
  if (st != MGE_OK) return st;
  // at most two rounds of quarter-width items (the kernel exits at once when there is no tail)
  const int tail_grid = (p0.tiles_upper < grid ? p0.tiles_upper : grid);
  {
    ProfScope prof(s, name);
    hipLaunchKernelGGL(ktail, dim3(tail_grid), dim3(G_THREADS), G_DYN_LDS, s, p);
  }
  return hip_check(name);
}

}  // namespace mge
