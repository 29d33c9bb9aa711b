// Top-k routing, per-expert histogram, prefix sum and the stable scatter that builds
// the permuted (grouped-by-expert) layout.
//
// Kernels (all one pass over the tokens, no host synchronization):
//   route_clear_kernel     clears the device error flag of this call
//   route_topk_kernel      one thread per token: top-k of the fp32 logits (ties to the
//                          lower index), softmax over the selected k, and a per-block
//                          per-expert count (LDS histogram built with LDS atomic adds:
//                          integer counts, so the result does not depend on their order)
//   route_scan_kernel      per expert, exclusive scan of the block counts -> block
//                          bases; split_sizes; group_offsets (sizes rounded to align)
//   route_scatter_kernel   stable rank of every assignment inside its block: within a
//                          wave by ballot match masks + popcount (plus the token's own
//                          earlier slots with the same expert), across the block's
//                          waves by per-wave counts in LDS; row = offset + block base +
//                          rank.  Writes perm_src / perm_pos / prob_perm and marks the
//                          padding rows.
// Being a counting sort over (t, i) order, the result is unique: bit-exact indices.
//   router_bwd_kernel      the backward of the top-k softmax: d_logits from d_prob
#include <math.h>

#include <mutex>

#include "mge_common.hpp"
#include "mge_internal.hpp"

namespace mge {

// ------------------------------------------------------------ fixed scratch
// The workspace of moe_route_permute_noalloc (the device error flag and the per-block
// expert counts), for callers that cannot allocate: a file-scope device array, one copy
// per GPU the library runs on, held until the process ends.  In host code `scratch` only
// names the symbol; its device address (different on every GPU) comes from
// hipGetSymbolAddress, taken once per device with that device current, and only that
// address is ever handed to a kernel.
static __device__ __align__(256) uint8_t scratch[kRouteScratchBytes];

mge_status route_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* dev_ptr[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return hip_check("hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) {
    set_error("device index %d outside the %d the fixed scratch is kept for", dev, kMaxDevices);
    return MGE_ERR_UNSUPPORTED;
  }
  std::lock_guard<std::mutex> lk(mu);
  if (!dev_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      set_error("hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
      return MGE_ERR_HIP;
    }
    dev_ptr[dev] = p;
  }
  *ptr = dev_ptr[dev];
  return MGE_OK;
}

constexpr int RT_THREADS = 256;
constexpr int RT_WAVES = RT_THREADS / kWave;
constexpr int RT_MAXK = 8;
constexpr int RT_MAXE = 256;

__global__ void route_clear_kernel(int32_t* err) {
  if (threadIdx.x == 0) err[0] = 0;
}

__global__ __launch_bounds__(RT_THREADS) void route_topk_kernel(RouteParams p) {
  __shared__ int32_t cnt[RT_MAXE];
  const int tid = threadIdx.x;
  for (int e = tid; e < p.E; e += RT_THREADS) cnt[e] = 0;
  __syncthreads();
  const int t = blockIdx.x * RT_THREADS + tid;
  if (t < p.T) {
    int bi[RT_MAXK];
    if (p.flags & MGE_ROUTE_PROB_GIVEN) {
#pragma unroll
      for (int j = 0; j < RT_MAXK; ++j) {
        if (j < p.k) {
          int e = p.topk_idx[int64_t(t) * p.k + j];
          if (e < 0 || e >= p.E) {
            p.err_flag[0] = 1;
            e = e < 0 ? 0 : p.E - 1;
          }
          bi[j] = e;
        }
      }
    } else {
      float bv[RT_MAXK];
#pragma unroll
      for (int j = 0; j < RT_MAXK; ++j) { bv[j] = -INFINITY; bi[j] = 0; }
      const float* l = p.logits + int64_t(t) * p.E;
      int filled = 0;
      for (int e = 0; e < p.E; ++e) {
        float cv = l[e];
        int ci = e;
        bool shifting = false;
#pragma unroll
        for (int j = 0; j < RT_MAXK; ++j) {
          if (j < p.k) {
            // strict '>' keeps an earlier (lower) index ahead of an equal later one
            bool take = shifting || j >= filled || cv > bv[j];
            if (take) {
              float tv = bv[j]; bv[j] = cv; cv = tv;
              int ti = bi[j]; bi[j] = ci; ci = ti;
              shifting = true;
            }
          }
        }
        filled = filled < p.k ? filled + 1 : p.k;
      }
      float m = bv[0];
      float ex[RT_MAXK];
      float sum = 0.f;
#pragma unroll
      for (int j = 0; j < RT_MAXK; ++j) {
        if (j < p.k) { ex[j] = expf(bv[j] - m); sum += ex[j]; }
      }
      float inv = 1.0f / sum;
#pragma unroll
      for (int j = 0; j < RT_MAXK; ++j) {
        if (j < p.k) {
          p.topk_idx[int64_t(t) * p.k + j] = bi[j];
          p.topk_prob[int64_t(t) * p.k + j] = ex[j] * inv;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < RT_MAXK; ++j)
      if (j < p.k) atomicAdd(&cnt[bi[j]], 1);
  }
  __syncthreads();
  for (int e = tid; e < p.E; e += RT_THREADS) p.block_counts[int64_t(blockIdx.x) * p.E + e] = cnt[e];
}

__global__ __launch_bounds__(RT_THREADS) void route_scan_kernel(RouteParams p) {
  __shared__ int32_t tot[RT_MAXE];
  const int e = threadIdx.x;
  if (e < p.E) {
    int run = 0;
    for (int b = 0; b < p.nblk; ++b) {
      int c = p.block_counts[int64_t(b) * p.E + e];
      p.block_counts[int64_t(b) * p.E + e] = run;   // becomes the exclusive block base
      run += c;
    }
    p.split_sizes[e] = run;
    tot[e] = run;
  }
  __syncthreads();
  if (e == 0) {
    int off = 0;
    for (int g = 0; g < p.E; ++g) {
      p.group_offsets[g] = off;
      off += (tot[g] + p.align - 1) / p.align * p.align;
    }
    p.group_offsets[p.E] = off;
  }
}

__global__ __launch_bounds__(RT_THREADS) void route_scatter_kernel(RouteParams p) {
  __shared__ int32_t wcnt[RT_WAVES][RT_MAXE];
  __shared__ int32_t offs[RT_MAXE + 1];
  __shared__ int32_t sizes[RT_MAXE];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int w = tid / kWave;
  for (int i = tid; i < RT_WAVES * RT_MAXE; i += RT_THREADS) (&wcnt[0][0])[i] = 0;
  for (int i = tid; i <= p.E; i += RT_THREADS) offs[i] = p.group_offsets[i];
  for (int i = tid; i < p.E; i += RT_THREADS) sizes[i] = p.split_sizes[i];
  __syncthreads();

  const int t = blockIdx.x * RT_THREADS + tid;
  const bool valid = t < p.T;
  int ex[RT_MAXK];
#pragma unroll
  for (int j = 0; j < RT_MAXK; ++j) {
    int e = p.E;   // sentinel for lanes without a token: matches no expert
    if (valid && j < p.k) {
      e = p.topk_idx[int64_t(t) * p.k + j];
      e = e < 0 ? 0 : (e >= p.E ? p.E - 1 : e);
    }
    ex[j] = e;
  }
  const uint64_t lt = (uint64_t(1) << lane) - 1;
  const uint64_t gt = ~lt & ~(uint64_t(1) << lane);
  const uint64_t vmask = __ballot(valid);
  int rank[RT_MAXK], after[RT_MAXK];
#pragma unroll
  for (int i = 0; i < RT_MAXK; ++i) { rank[i] = 0; after[i] = 0; }
  // A token may name one expert in several slots (caller-given indices, or an index
  // clamped into range): its earlier slots with the same expert come first, so the
  // order stays the stable (t, i) order and every row of the group is written once.
#pragma unroll
  for (int i = 0; i < RT_MAXK; ++i) {
#pragma unroll
    for (int j = 0; j < RT_MAXK; ++j) {
      if (i < p.k && j < p.k && ex[j] == ex[i]) {
        if (j < i) ++rank[i];
        if (j > i) ++after[i];
      }
    }
  }
  // For each slot j of the other lanes: mask of lanes whose slot-j expert equals my
  // slot-i expert, assembled bit by bit from ballots; the rank of (t, i) adds the
  // matching slots of the earlier tokens of the wave.  The last occurrence of an
  // expert in the wave (no later lane and no later slot of its own token with it)
  // holds the wave's count of that expert.
  for (int j = 0; j < p.k; ++j) {
    uint64_t m[RT_MAXK];
#pragma unroll
    for (int i = 0; i < RT_MAXK; ++i) m[i] = vmask;
    int ej = 0;
#pragma unroll
    for (int jj = 0; jj < RT_MAXK; ++jj) if (jj == j) ej = ex[jj];
    for (int b = 0; b < p.nbits; ++b) {
      uint64_t bal = __ballot((ej >> b) & 1);
#pragma unroll
      for (int i = 0; i < RT_MAXK; ++i) m[i] &= ((ex[i] >> b) & 1) ? bal : ~bal;
    }
#pragma unroll
    for (int i = 0; i < RT_MAXK; ++i) {
      rank[i] += __popcll(m[i] & lt);
      after[i] += __popcll(m[i] & gt);
    }
  }
#pragma unroll
  for (int i = 0; i < RT_MAXK; ++i)
    if (valid && i < p.k && after[i] == 0) wcnt[w][ex[i]] = rank[i] + 1;
  __syncthreads();
  if (valid) {
#pragma unroll
    for (int i = 0; i < RT_MAXK; ++i) {
      if (i < p.k) {
        int e = ex[i];
        int base = offs[e] + p.block_counts[int64_t(blockIdx.x) * p.E + e];
        for (int ww = 0; ww < w; ++ww) base += wcnt[ww][e];
        int row = base + rank[i];
        p.perm_src[row] = t;
        p.perm_pos[int64_t(t) * p.k + i] = row;
        p.prob_perm[row] = p.topk_prob[int64_t(t) * p.k + i];
      }
    }
  }
  // padding rows: not inside [offs[e], offs[e] + sizes[e]) of any group
  for (int r = t; r < p.R; r += p.nblk * RT_THREADS) {
    int lo = 0, hi = p.E;   // largest g with offs[g] <= r
    while (lo < hi) {
      int mid = (lo + hi + 1) >> 1;
      if (offs[mid] <= r) lo = mid; else hi = mid - 1;
    }
    bool pad = (lo >= p.E) || (r - offs[lo] >= sizes[lo]);
    if (pad) {
      p.perm_src[r] = -1;
      p.prob_perm[r] = 0.f;
    }
  }
}

// Router backward.  The k slot probabilities of token t are the softmax of its selected
// logits z_i = l[t][idx_i], so with s_t = sum_j p_j d_p_j the gradient of slot i is
// p_i (d_p_i - s_t), added into d_logits[t][idx_i]; logits no slot selected get 0.  One
// thread per output element (t, e), so the [T][E] rows leave as whole lines; the
// threads of a token re-read its k slots from cache.  s_t is summed in slot order with
// fused multiply-adds; slots with an index outside [0, E) match no e.
__global__ void router_bwd_kernel(int T, int E, int k, const int32_t* __restrict__ idx, const float* __restrict__ prob,
                                  const float* __restrict__ dprob, float* __restrict__ dlogits) {
  const int64_t g = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (g >= int64_t(T) * E) return;
  const int t = int(g / E);
  const int e = int(g - int64_t(t) * E);
  const int32_t* it = idx + int64_t(t) * k;
  const float* pt = prob + int64_t(t) * k;
  const float* dt = dprob + int64_t(t) * k;
  float s = 0.f;
  for (int j = 0; j < k; ++j) s = fmaf(pt[j], dt[j], s);
  float d = 0.f;
  for (int i = 0; i < k; ++i)
    if (it[i] == e) d += pt[i] * (dt[i] - s);
  dlogits[g] = d;
}

mge_status launch_router_bwd(int T, int E, int k, const int32_t* idx, const float* prob, const float* dprob,
                             float* dlogits, hipStream_t s) {
  const int64_t n = int64_t(T) * E;
  if (n == 0) return MGE_OK;
  ProfScope prof(s, "router_bwd");
  hipLaunchKernelGGL(router_bwd_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, s, T, E, k, idx, prob, dprob,
                     dlogits);
  return hip_check("router_bwd_kernel");
}

mge_status launch_route(const RouteParams& p, hipStream_t s) {
  {
    ProfScope prof(s, "route_clear");
    hipLaunchKernelGGL(route_clear_kernel, dim3(1), dim3(64), 0, s, p.err_flag);
  }
  {
    ProfScope prof(s, "route_topk");
    hipLaunchKernelGGL(route_topk_kernel, dim3(p.nblk), dim3(RT_THREADS), 0, s, p);
  }
  {
    ProfScope prof(s, "route_scan");
    hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(RT_THREADS), 0, s, p);
  }
  {
    ProfScope prof(s, "route_scatter");
    hipLaunchKernelGGL(route_scatter_kernel, dim3(p.nblk), dim3(RT_THREADS), 0, s, p);
  }
  return hip_check("route kernels");
}

}  // namespace mge
