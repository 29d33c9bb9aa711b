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
// Tiles are 256 x 256 with 128-byte K slices (128 FP8 or 64 BF16 elements), 4 waves in
// a 2 x 2 grid, each wave 128 x 128 built from 32 x 32 MFMA blocks:
//   MXFP8: v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 x E4M3, one E8M0 scale per lane and
//          32-element K block, applied by the matrix core — no dequantize pass).
//          Operand layout (measured on gfx950): lane l = 32h + i feeds row/column i;
//          its register bytes 0..15 are K elements 16h..16h+15 and bytes 16..31 are
//          32+16h..32+16h+15 of the 64-element step, so K block h (elements
//          32h..32h+31) is scaled by the scale register of the lanes with that h, the
//          byte chosen by op_sel.
//   BF16:  v_mfma_f32_32x32x16_bf16
// Operand tiles go HBM -> registers -> LDS (double-buffered, XOR-swizzled 16-byte
// chunks so both the row-wise stores and the MFMA fragment reads are bank-conflict
// free); the next K slice is fetched while the current one is multiplied.
// A persistent grid walks the tiles (expert-major, then N, M fastest so that
// consecutive tiles share the weight tile); virtual workgroup ids are remapped so
// that the workgroups of one XCD (hardware dispatches round-robin over the 8 XCDs)
// take consecutive tiles and share that XCD's L2.  Empty experts own no tiles (RAGGED_M)
// or produce zero gradients (RAGGED_K).
// Epilogues (fp32 accumulators never reach HBM):
//   EPI_STORE       bf16 / f32 store (optionally accumulate), row masking
//   EPI_SWIGLU      h = p * silu(G) * U with G, U of the same rows/columns in the same
//                   lane; h quantized along F (MXFP8, amax over the 32 lanes that hold
//                   one 32-column block) or rounded to bf16; training also stores G, U
//                   (bf16) and the column form of h (blocks of 32 rows: 16 in a lane,
//                   16 in its partner lane 32 apart)
//   EPI_SWIGLU_BWD  dh -> dG, dU (with saved G, U, p) quantized row- and column-wise,
//                   plus per-row partial sums of dh * silu(G) * U for d_prob
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
constexpr int G_BKB = 128;                    // K bytes per slice
constexpr int G_THREADS = 64 * G_WAVES_M * G_WAVES_N;
constexpr int G_STAGE_BYTES = (G_BM + G_BN) * G_BKB;
constexpr int G_LDS_BYTES = 2 * G_STAGE_BYTES;
constexpr int G_MAXE = 256;
// Buffer-resource word 3 of the gfx9 family (raw buffer, 32-bit dwords), the record
// bound, and the offset that lies beyond it (such a lane loads zeros).
constexpr int kRsrcFlags = 0x00020000;
constexpr int kRsrcRecords = 0x7fffffff;
constexpr uint32_t kInvalid = 0x80000000u;   // OR-ed into an offset: the lane reads zeros

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
template <typename T>
__device__ __forceinline__ const T* uniform_ptr(const T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(v >> 32));
  return reinterpret_cast<const T*>((uint64_t(hi) << 32) | lo);
}

__device__ __forceinline__ int swz(int row, int chunk) { return row * G_BKB + ((chunk ^ (row & 7)) << 4); }

struct TileInfo {
  int e, mt, nt;
  int m_valid;          // rows of the tile's group (RAGGED_M) or M (RAGGED_K)
  int row_off;          // first permuted row of the group (RAGGED_M) / K offset (RAGGED_K)
  int k_len;            // reduction length in elements
};

// Raw buffer resource over `base` (gfx9 word 3, full 31-bit range).
__device__ __forceinline__ i32x4 make_rsrc(const void* base) {
  const uint64_t v = reinterpret_cast<uint64_t>(base);
  return i32x4{int(uint32_t(v)), int(uint32_t(v >> 32) & 0xffff), kRsrcRecords, kRsrcFlags};
}

// 16 bytes per lane from buffer offset `voff` straight into LDS at lds_addr + 16*lane
// (buffer_load_dwordx4 ... lds; M0 holds the wave's LDS destination).  Written as asm
// so the compiler neither waits on it before unrelated LDS reads nor reorders LDS
// accesses across it; the caller waits (vmcnt) and synchronizes before reading.
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t lds_addr, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(lds_addr), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}

template <bool MX, int EPI, int MODE>
__device__ __forceinline__ void gemm_body(const GemmParams& p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  // LDS byte address of the dynamic shared block (the low half of its generic address)
  const uint32_t lds_base = uniform(int(uint32_t(reinterpret_cast<uintptr_t>(smem))));
  __shared__ int32_t s_prefix[G_MAXE + 1];
  __shared__ int32_t s_mtiles[G_MAXE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int wm = wave / G_WAVES_N;
  const int wn = wave % G_WAVES_N;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  constexpr int ELEM = MX ? 1 : 2;           // bytes per element

  // ---- tile table: tiles of expert e = mtiles(e) * ntiles
  const int ncols_per_tile = (EPI == EPI_SWIGLU) ? G_BN / 2 : G_BN;
  const int ncols = (EPI == EPI_SWIGLU) ? p.F : p.N;
  const int ntiles = (ncols + ncols_per_tile - 1) / ncols_per_tile;
  if (tid == 0) {
    int acc = 0;
    for (int e = 0; e < p.E; ++e) {
      int mt = MODE == RAGGED_M ? (p.sizes[e] + G_BM - 1) / G_BM : (p.M + G_BM - 1) / G_BM;
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

  for (int tile = vid; tile < total; tile += nwg) {
    // ---- decode the tile
    int lo = 0, hi_ = p.E - 1;
    while (lo < hi_) {
      int mid = (lo + hi_ + 1) >> 1;
      if (s_prefix[mid] <= tile) lo = mid; else hi_ = mid - 1;
    }
    // every tile quantity is wave-uniform: keep it in scalar registers
    const int e = uniform(lo);
    const int local = tile - uniform(s_prefix[e]);
    const int mtn = uniform(s_mtiles[e]);
    const int mt = local % mtn;
    const int nt = local / mtn;
    const int off = uniform(p.offs[e]);
    const int m_valid = MODE == RAGGED_M ? uniform(p.sizes[e]) : p.M;
    const int m0 = mt * G_BM;
    // K range in bytes.  RAGGED_M: [0, K).  RAGGED_K: the expert's token span
    // [off, off + roundup32(size)) of the column forms; the loop starts at the slice
    // boundary below it and the chunks outside the span load as zeros.
    int kbase, klo, khi;
    if constexpr (MODE == RAGGED_M) {
      kbase = 0; klo = 0; khi = p.K * ELEM;
    } else {
      const int span = ((uniform(p.sizes[e]) + 31) / 32) * 32;
      klo = off * ELEM;
      khi = (off + span) * ELEM;
      kbase = span > 0 ? (klo / G_BKB) * G_BKB : klo;
    }
    const int nkt = (khi - kbase + G_BKB - 1) / G_BKB;

    // ---- operands as buffer resources: a lane whose offset is kInvalid reads zeros
    // (rows past the group, chunks outside the K range), so tails need no extra path.
    const uint8_t* Abase;
    const uint8_t* Bbase;
    if constexpr (MODE == RAGGED_M) {
      Abase = p.A + int64_t(off) * p.lda;
      Bbase = uniform_ptr(p.Bt[e]);
    } else {
      Abase = p.A;
      Bbase = p.B;
    }
    const i32x4 rsrcA = make_rsrc(Abase);
    const i32x4 rsrcB = make_rsrc(Bbase);

    // ---- loader geometry: wave instruction i fills LDS rows [(wave*8+i)*8, +8) of a
    // 256-row operand tile, 1 KB contiguous (lane l -> row +l/8, LDS chunk l%8).  The
    // lane loads the global chunk that the XOR swizzle maps to that LDS chunk.
    const int lchunk = (lane & 7) ^ (lane >> 3);
    uint32_t a_off[8], b_off[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = wave * 64 + i * 8 + (lane >> 3);   // row within the tile
      const int ra = m0 + r;
      a_off[i] = ra < m_valid ? uint32_t(ra) * uint32_t(p.lda) + lchunk * 16 : kInvalid;
      int grow;
      if constexpr (EPI == EPI_SWIGLU) {
        constexpr int half = G_BN / 2;
        const int f = nt * half + (r % half);
        grow = f < p.F ? (r < half ? f : p.F + f) : -1;
      } else {
        grow = nt * G_BN + r;
        grow = grow < p.N ? grow : -1;
      }
      b_off[i] = grow >= 0 ? uint32_t(grow) * uint32_t(p.ldb) + lchunk * 16 : kInvalid;
    }
    auto issue_loads = [&](int kt, int buf) {
      // chunks outside [klo, khi) get the top offset bit set (-> zeros); arithmetic
      // rather than a select so the loads stay straight-line code
      const int kslice = kbase + kt * G_BKB;          // first byte of the slice
      const int kb = kslice + lchunk * 16;             // this lane's chunk (a_off/b_off hold the chunk term)
      const uint32_t out = ((uint32_t(kb - klo) | uint32_t(khi - 1 - kb)) >> 31) << 31;
      const uint32_t kadd = uint32_t(kslice);
      const uint32_t la = lds_base + buf * G_STAGE_BYTES + wave * 8 * 1024;
      const uint32_t lb = la + G_BM * G_BKB;
#pragma unroll
      for (int i = 0; i < 8; ++i) dma16(rsrcA, la + i * 1024, (a_off[i] + kadd) | out);
#pragma unroll
      for (int i = 0; i < 8; ++i) dma16(rsrcB, lb + i * 1024, (b_off[i] + kadd) | out);
    };

    // ---- MX scales: packed as one dword per (row, 128-element slice) holding the 4
    // E8M0 bytes of that slice, rows contiguous, so the 32 lanes of a block read 128
    // consecutive bytes.
    int brow_tile[G_WNB];
#pragma unroll
    for (int ni = 0; ni < G_WNB; ++ni) {
      if constexpr (EPI == EPI_SWIGLU) {
        constexpr int hb = G_WNB / 2;
        brow_tile[ni] = ni < hb ? (wn * hb + ni) * 32 : G_BN / 2 + (wn * hb + ni - hb) * 32;
      } else {
        brow_tile[ni] = (wn * G_WNB + ni) * 32;
      }
    }
    const uint32_t* sa_ptr[G_WMB];
    const uint32_t* sb_ptr[G_WNB];
    int64_t sa_step = 0, sb_step = 0;
    if constexpr (MX) {
      int64_t j0 = MODE == RAGGED_M ? 0 : kbase / 128;   // first packed slice
      const uint32_t* Ap;
      const uint32_t* Bp;
      if constexpr (MODE == RAGGED_M) {
        Ap = p.Asp + off;
        Bp = p.Bsp + int64_t(e) * p.bsp_estride;
      } else {
        Ap = p.Asp;
        Bp = p.Bsp;
      }
      sa_step = p.asp_ld;
      sb_step = p.bsp_ld;
#pragma unroll
      for (int mi = 0; mi < G_WMB; ++mi) {
        int r = m0 + (wm * G_WMB + mi) * 32 + l32;
        r = r >= m_valid ? m_valid - 1 : r;
        r = r < 0 ? 0 : r;
        sa_ptr[mi] = Ap + j0 * sa_step + r;
      }
#pragma unroll
      for (int ni = 0; ni < G_WNB; ++ni) {
        const int r = brow_tile[ni] + l32;
        int grow;
        if constexpr (EPI == EPI_SWIGLU) {
          constexpr int half = G_BN / 2;
          int f = nt * half + (r % half);
          f = f >= p.F ? p.F - 1 : f;
          grow = r < half ? f : p.F + f;
        } else {
          grow = nt * G_BN + r;
          grow = grow >= p.N ? p.N - 1 : grow;
        }
        sb_ptr[ni] = Bp + j0 * sb_step + grow;
      }
    }
    // raw packed dwords; the lane's byte (block 4kt + hi, and + 2 for the second
    // 64-element step) is selected at the MFMA by shift + op_sel, so a load is only
    // waited for where it is used
    uint32_t sa[G_WMB], sb[G_WNB];
    uint32_t nsa[G_WMB], nsb[G_WNB];
    auto sload = [&](int kt, uint32_t* da, uint32_t* db) {
#pragma unroll
      for (int mi = 0; mi < G_WMB; ++mi) da[mi] = sa_ptr[mi][kt * sa_step];
#pragma unroll
      for (int ni = 0; ni < G_WNB; ++ni) db[ni] = sb_ptr[ni][kt * sb_step];
    };

    f32x16 acc[G_WMB][G_WNB];
#pragma unroll
    for (int mi = 0; mi < G_WMB; ++mi)
#pragma unroll
      for (int ni = 0; ni < G_WNB; ++ni)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;

    // MFMA operand fragments of one K step, read from the swizzled LDS tile:
    //   MX  : 64-element step s of the slice; lane (hi, l32) takes 16-byte chunks
    //         4s + hi and 4s + hi + 2 of its row
    //   BF16: 16-element step s; lane takes chunk 2s + hi
    typedef typename std::conditional<MX, i32x8, bf16x8>::type frag_t;
    constexpr int NSTEP = MX ? 2 : 4;
    auto read_frags = [&](const uint8_t* sA, const uint8_t* sB, int s, frag_t* af, frag_t* bfr) {
#pragma unroll
      for (int mi = 0; mi < G_WMB; ++mi) {
        const int row = (wm * G_WMB + mi) * 32 + l32;
        if constexpr (MX) {
          const int c = s * 4 + hi;
          const uint4 x0 = *reinterpret_cast<const uint4*>(sA + swz(row, c));
          const uint4 x1 = *reinterpret_cast<const uint4*>(sA + swz(row, c + 2));
          af[mi] = i32x8{int(x0.x), int(x0.y), int(x0.z), int(x0.w), int(x1.x), int(x1.y), int(x1.z), int(x1.w)};
        } else {
          af[mi] = *reinterpret_cast<const bf16x8*>(sA + swz(row, s * 2 + hi));
        }
      }
#pragma unroll
      for (int ni = 0; ni < G_WNB; ++ni) {
        const int row = brow_tile[ni] + l32;
        if constexpr (MX) {
          const int c = s * 4 + hi;
          const uint4 x0 = *reinterpret_cast<const uint4*>(sB + swz(row, c));
          const uint4 x1 = *reinterpret_cast<const uint4*>(sB + swz(row, c + 2));
          bfr[ni] = i32x8{int(x0.x), int(x0.y), int(x0.z), int(x0.w), int(x1.x), int(x1.y), int(x1.z), int(x1.w)};
        } else {
          bfr[ni] = *reinterpret_cast<const bf16x8*>(sB + swz(row, s * 2 + hi));
        }
      }
    };
    auto mfma_step = [&](int s, const frag_t* af, const frag_t* bfr) {
#pragma unroll
      for (int mi = 0; mi < G_WMB; ++mi)
#pragma unroll
        for (int ni = 0; ni < G_WNB; ++ni) {
          if constexpr (MX) {
            const int xa = int(sa[mi] >> (8 * hi));
            const int xb = int(sb[ni] >> (8 * hi));
            if (s == 0)
              acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[mi], bfr[ni], acc[mi][ni], 0, 0, 0, xa, 0,
                                                                            xb);
            else
              acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[mi], bfr[ni], acc[mi][ni], 0, 0, 2, xa, 2,
                                                                            xb);
          } else {
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfr[ni], acc[mi][ni], 0, 0, 0);
          }
        }
    };

    __syncthreads();   // previous tile's LDS readers are done
    if (nkt > 0) {
      issue_loads(0, 0);
      if constexpr (MX) sload(0, sa, sb);
    }
    __builtin_amdgcn_s_waitcnt(0);   // vmcnt(0) lgkmcnt(0): the LDS copies have landed
    __syncthreads();
    for (int kt = 0; kt < nkt; ++kt) {
      const int buf = kt & 1;
      // 1. the next slice streams into the other LDS buffer while this one is used
      //    (past the last slice every chunk is out of range and loads zeros: no branch)
      issue_loads(kt + 1, buf ^ 1);
      if constexpr (MX) sload(kt + 1 < nkt ? kt + 1 : kt, nsa, nsb);
      __builtin_amdgcn_sched_barrier(0);
      // 2. MFMAs on this slice; the fragments of step s+1 are read while step s runs
      const uint8_t* sA = smem + buf * G_STAGE_BYTES;
      const uint8_t* sB = sA + G_BM * G_BKB;
      frag_t af[2][G_WMB], bfr[2][G_WNB];
      read_frags(sA, sB, 0, af[0], bfr[0]);
#pragma unroll
      for (int s = 0; s < NSTEP; ++s) {
        if (s + 1 < NSTEP) read_frags(sA, sB, s + 1, af[(s + 1) & 1], bfr[(s + 1) & 1]);
        mfma_step(s, af[s & 1], bfr[s & 1]);
      }
      __builtin_amdgcn_sched_barrier(0);
      // 3. the next slice is resident and every wave is done with this one
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if constexpr (MX) {
#pragma unroll
        for (int mi = 0; mi < G_WMB; ++mi) sa[mi] = nsa[mi];
#pragma unroll
        for (int ni = 0; ni < G_WNB; ++ni) sb[ni] = nsb[ni];
      }
    }

    // ---------------------------------------------------------------- epilogues
    // Accumulator element r of block (mi, ni) is row 8*(r/4) + 4*hi + (r%4) and column
    // l32 of that 32 x 32 block.
    const int wrow0 = m0 + wm * G_WMB * 32;   // wave's first row (group-local)
    if constexpr (EPI == EPI_STORE) {
      static_for<0, G_WMB>([&](auto mic) {
        constexpr int mi = decltype(mic)::value;
        static_for<0, G_WNB>([&](auto nic) {
          constexpr int ni = decltype(nic)::value;
          const int col = nt * G_BN + brow_tile[ni] + l32;
          const bool cok = col < p.N;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = wrow0 + mi * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
            float v = acc[mi][ni][r];
            if (cok && row < m_valid) {
              if constexpr (MODE == RAGGED_M) {
                int64_t idx = int64_t(off + row) * p.ldc + col;
                if (p.out_dtype == MGE_DTYPE_BF16) reinterpret_cast<uint16_t*>(p.C)[idx] = f32_to_bf16(v);
                else reinterpret_cast<float*>(p.C)[idx] = v;
              } else {
                int64_t idx = int64_t(row) * p.ldc + col;
                if (p.out_dtype == MGE_DTYPE_BF16) {
                  uint16_t* o = reinterpret_cast<uint16_t*>(p.Ct[e]);
                  if (p.accumulate) v += bf16_to_f32(o[idx]);
                  o[idx] = f32_to_bf16(v);
                } else {
                  float* o = reinterpret_cast<float*>(p.Ct[e]);
                  if (p.accumulate) v += o[idx];
                  o[idx] = v;
                }
              }
            }
          }
        });
      });
    } else if constexpr (EPI == EPI_SWIGLU) {
      constexpr int hb = G_WNB / 2;
      const int F = p.F;
      const int F2 = 2 * F;
      const int m_pad = (m_valid + 31) / 32 * 32;
      static_for<0, G_WMB>([&](auto mic) {
        constexpr int mi = decltype(mic)::value;
        float pr[16];
        const int rbase = wrow0 + mi * 32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = rbase + 8 * (r >> 2) + 4 * hi + (r & 3);
          pr[r] = row < m_valid ? p.prob[off + row] : 0.f;
        }
        static_for<0, hb>([&](auto jc) {
          constexpr int j = decltype(jc)::value;
          const int f = nt * (G_BN / 2) + (wn * hb + j) * 32 + l32;
          const bool fok = f < F;
          float h[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = rbase + 8 * (r >> 2) + 4 * hi + (r & 3);
            const bool ok = fok && row < m_valid;
            const float G = acc[mi][j][r];
            const float U = acc[mi][j + hb][r];
            h[r] = ok ? pr[r] * silu_f(G) * U : 0.f;
            if (p.saved_gu && ok) {
              int64_t o = int64_t(off + row) * F2 + f;
              p.saved_gu[o] = f32_to_bf16(G);
              p.saved_gu[o + F] = f32_to_bf16(U);
            }
          }
          // row form of h (blocks of 32 along F = the 32 lanes of this half-wave)
          if (MX) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int row = rbase + 8 * (r >> 2) + 4 * hi + (r & 3);
              float amax = wave_max_xor(fabsf(h[r]), 32);
              uint32_t s = mx_scale_byte(amax);
              uint32_t code = e4m3_rne(h[r] * mx_inv_scale(s));
              if (row < m_valid && fok) {
                int64_t o = int64_t(off + row) * F + f;
                p.h_codes[o] = uint8_t(code);
                if (l32 == 0) p.h_scales[int64_t(off + row) * (F / 32) + f / 32] = uint8_t(s);
              }
            }
          } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int row = rbase + 8 * (r >> 2) + 4 * hi + (r & 3);
              if (row < m_valid && fok) p.h_bf16[int64_t(off + row) * F + f] = f32_to_bf16(h[r]);
            }
          }
          // column form of h (training): this 32-row block of column f
          if ((p.hc_codes || p.hc_bf16) && fok && rbase < m_pad) {
            if (MX) {
              float amax = 0.f;
#pragma unroll
              for (int r = 0; r < 16; ++r) amax = fmaxf(amax, fabsf(h[r]));
              amax = fmaxf(amax, __shfl_xor(amax, 32));
              uint32_t s = mx_scale_byte(amax);
              float inv = mx_inv_scale(s);
              uint8_t* dst = p.hc_codes + int64_t(f) * p.Rp + off + rbase + 4 * hi;
#pragma unroll
              for (int g = 0; g < 4; ++g) {
                uint32_t w = e4m3_rne(h[4 * g] * inv) | (e4m3_rne(h[4 * g + 1] * inv) << 8) |
                             (e4m3_rne(h[4 * g + 2] * inv) << 16) | (e4m3_rne(h[4 * g + 3] * inv) << 24);
                *reinterpret_cast<uint32_t*>(dst + 8 * g) = w;
              }
              if (hi == 0) p.hc_scales[int64_t(f) * (p.Rp / 32) + (off + rbase) / 32] = uint8_t(s);
            } else {
              uint16_t* dst = p.hc_bf16 + int64_t(f) * p.Rp + off + rbase + 4 * hi;
#pragma unroll
              for (int g = 0; g < 4; ++g) {
                uint2 w;
                w.x = uint32_t(f32_to_bf16(h[4 * g])) | (uint32_t(f32_to_bf16(h[4 * g + 1])) << 16);
                w.y = uint32_t(f32_to_bf16(h[4 * g + 2])) | (uint32_t(f32_to_bf16(h[4 * g + 3])) << 16);
                *reinterpret_cast<uint2*>(dst + 8 * g) = w;
              }
            }
          }
        });
      });
    } else {  // EPI_SWIGLU_BWD: columns are f, the accumulator is dh
      const int F = p.F;
      const int F2 = 2 * F;
      const int m_pad = (m_valid + 31) / 32 * 32;
      const int part = nt * G_WAVES_N + wn;
      static_for<0, G_WMB>([&](auto mic) {
        constexpr int mi = decltype(mic)::value;
        float pr[16], dps[16];
        const int rbase = wrow0 + mi * 32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = rbase + 8 * (r >> 2) + 4 * hi + (r & 3);
          pr[r] = row < m_valid ? p.prob[off + row] : 0.f;
          dps[r] = 0.f;
        }
        static_for<0, G_WNB>([&](auto nic) {
          constexpr int ni = decltype(nic)::value;
          const int f = nt * G_BN + (wn * G_WNB + ni) * 32 + l32;
          const bool fok = f < F;
          float dG[16], dU[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = rbase + 8 * (r >> 2) + 4 * hi + (r & 3);
            const bool ok = fok && row < m_valid;
            float G = 0.f, U = 0.f;
            if (ok) {
              int64_t o = int64_t(off + row) * F2 + f;
              G = bf16_to_f32(p.gu[o]);
              U = bf16_to_f32(p.gu[o + F]);
            }
            const float dh = acc[mi][ni][r];
            const float sg = sigmoid_f(G);
            const float sl = G * sg;
            dps[r] += ok ? dh * sl * U : 0.f;
            dU[r] = ok ? dh * pr[r] * sl : 0.f;
            dG[r] = ok ? dh * pr[r] * U * sg * (1.f + G * (1.f - sg)) : 0.f;
          }
          // row form [R][2F]: dG at column f, dU at column F + f
          static_for<0, 2>([&](auto halfc) {
            constexpr int half = decltype(halfc)::value;
            float* v = half == 0 ? dG : dU;
            const int col = half * F + f;
            if (MX) {
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int row = rbase + 8 * (r >> 2) + 4 * hi + (r & 3);
                float amax = wave_max_xor(fabsf(v[r]), 32);
                uint32_t s = mx_scale_byte(amax);
                uint32_t code = e4m3_rne(v[r] * mx_inv_scale(s));
                if (row < m_valid && fok) {
                  p.dgu_codes[int64_t(off + row) * F2 + col] = uint8_t(code);
                  if (l32 == 0) p.dgu_scales[int64_t(off + row) * (F2 / 32) + col / 32] = uint8_t(s);
                }
              }
            } else {
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int row = rbase + 8 * (r >> 2) + 4 * hi + (r & 3);
                if (row < m_valid && fok) p.dgu_bf16[int64_t(off + row) * F2 + col] = f32_to_bf16(v[r]);
              }
            }
            // column form [2F][Rp]
            if ((p.dguc_codes || p.dguc_bf16) && fok && rbase < m_pad) {
              if (MX) {
                float amax = 0.f;
#pragma unroll
                for (int r = 0; r < 16; ++r) amax = fmaxf(amax, fabsf(v[r]));
                amax = fmaxf(amax, __shfl_xor(amax, 32));
                uint32_t s = mx_scale_byte(amax);
                float inv = mx_inv_scale(s);
                uint8_t* dst = p.dguc_codes + int64_t(col) * p.Rp + off + rbase + 4 * hi;
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                  uint32_t w = e4m3_rne(v[4 * g] * inv) | (e4m3_rne(v[4 * g + 1] * inv) << 8) |
                               (e4m3_rne(v[4 * g + 2] * inv) << 16) | (e4m3_rne(v[4 * g + 3] * inv) << 24);
                  *reinterpret_cast<uint32_t*>(dst + 8 * g) = w;
                }
                if (hi == 0) p.dguc_scales[int64_t(col) * (p.Rp / 32) + (off + rbase) / 32] = uint8_t(s);
              } else {
                uint16_t* dst = p.dguc_bf16 + int64_t(col) * p.Rp + off + rbase + 4 * hi;
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                  uint2 w;
                  w.x = uint32_t(f32_to_bf16(v[4 * g])) | (uint32_t(f32_to_bf16(v[4 * g + 1])) << 16);
                  w.y = uint32_t(f32_to_bf16(v[4 * g + 2])) | (uint32_t(f32_to_bf16(v[4 * g + 3])) << 16);
                  *reinterpret_cast<uint2*>(dst + 8 * g) = w;
                }
              }
            }
          });
        });
        // d_prob partial of each row over this wave's columns (fixed xor-tree order)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float v = wave_sum_xor(dps[r], 32);
          const int row = rbase + 8 * (r >> 2) + 4 * hi + (r & 3);
          if (l32 == 0 && row < m_valid) p.dprob_part[int64_t(off + row) * p.nparts + part] = v;
        }
      });
    }
  }
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
  hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, G_LDS_BYTES);
  int grid = device_cus();
  if (p.tiles_upper < grid) grid = p.tiles_upper;
  if (grid <= 0) return MGE_OK;
  ProfScope prof(s, name);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(G_THREADS), G_LDS_BYTES, s, p);
  return hip_check(name);
}

}  // namespace mge
