// Atomic-free unpermute / combine, the d_prob reduction, and the upload of per-expert
// pointer tables into the workspace.
//
// combine: out[t][:] = sum_{i<k} w[t][i] * in[perm_pos[t][i]][:] — one workgroup per
// token, 16-byte vector loads of the k source rows, fp32 sum in slot order, one
// store.  HBM-bound: (k * in_bytes + out_bytes) per output element.
#include "mge_common.hpp"
#include "mge_internal.hpp"

namespace mge {

constexpr int CB_THREADS = 256;

template <typename TIn, typename TOut>
__global__ __launch_bounds__(CB_THREADS) void combine_kernel(int k, int H, const TIn* __restrict__ in,
                                                             int64_t in_rows,
                                                             const int32_t* __restrict__ perm_pos,
                                                             const float* __restrict__ weights,
                                                             TOut* __restrict__ out) {
  const int t = blockIdx.x;
  // a slot whose entry names no row of in (outside [0, in_rows), e.g. -1) adds nothing;
  // the test is uniform over the workgroup (one token)
  int rows[8];
  float w[8];
  bool use[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    use[i] = false;
    if (i < k) {
      rows[i] = perm_pos[int64_t(t) * k + i];
      use[i] = rows[i] >= 0 && rows[i] < in_rows;
      w[i] = weights ? weights[int64_t(t) * k + i] : 1.0f;
    }
  }
  const int nchunk = H / 8;
  for (int c = threadIdx.x; c < nchunk; c += CB_THREADS) {
    float acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (use[i]) {
        const TIn* src = in + int64_t(rows[i]) * H + c * 8;
        if constexpr (sizeof(TIn) == 2) {
          uint4 v = *reinterpret_cast<const uint4*>(src);
          const uint32_t* u = reinterpret_cast<const uint32_t*>(&v);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            acc[2 * j] += w[i] * __uint_as_float(u[j] << 16);
            acc[2 * j + 1] += w[i] * __uint_as_float(u[j] & 0xffff0000u);
          }
        } else {
          float4 a = *reinterpret_cast<const float4*>(src);
          float4 b = *reinterpret_cast<const float4*>(src + 4);
          acc[0] += w[i] * a.x; acc[1] += w[i] * a.y; acc[2] += w[i] * a.z; acc[3] += w[i] * a.w;
          acc[4] += w[i] * b.x; acc[5] += w[i] * b.y; acc[6] += w[i] * b.z; acc[7] += w[i] * b.w;
        }
      }
    }
    TOut* dst = out + int64_t(t) * H + c * 8;
    if constexpr (sizeof(TOut) == 2) {
      uint4 v;
      v.x = uint32_t(f32_to_bf16(acc[0])) | (uint32_t(f32_to_bf16(acc[1])) << 16);
      v.y = uint32_t(f32_to_bf16(acc[2])) | (uint32_t(f32_to_bf16(acc[3])) << 16);
      v.z = uint32_t(f32_to_bf16(acc[4])) | (uint32_t(f32_to_bf16(acc[5])) << 16);
      v.w = uint32_t(f32_to_bf16(acc[6])) | (uint32_t(f32_to_bf16(acc[7])) << 16);
      *reinterpret_cast<uint4*>(dst) = v;
    } else {
      *reinterpret_cast<float4*>(dst) = make_float4(acc[0], acc[1], acc[2], acc[3]);
      *reinterpret_cast<float4*>(dst + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
  }
}

mge_status launch_combine(int T, int k, int H, int in_dtype, int out_dtype, const void* in, int64_t in_rows,
                          const int32_t* perm_pos, const float* weights, void* out, hipStream_t s) {
  if (T <= 0) return MGE_OK;
  dim3 g(T), b(CB_THREADS);
  ProfScope prof(s, "combine");
  if (in_dtype == MGE_DTYPE_BF16 && out_dtype == MGE_DTYPE_BF16)
    hipLaunchKernelGGL((combine_kernel<uint16_t, uint16_t>), g, b, 0, s, k, H, (const uint16_t*)in, in_rows, perm_pos,
                       weights, (uint16_t*)out);
  else if (in_dtype == MGE_DTYPE_BF16)
    hipLaunchKernelGGL((combine_kernel<uint16_t, float>), g, b, 0, s, k, H, (const uint16_t*)in, in_rows, perm_pos,
                       weights, (float*)out);
  else if (out_dtype == MGE_DTYPE_BF16)
    hipLaunchKernelGGL((combine_kernel<float, uint16_t>), g, b, 0, s, k, H, (const float*)in, in_rows, perm_pos,
                       weights, (uint16_t*)out);
  else
    hipLaunchKernelGGL((combine_kernel<float, float>), g, b, 0, s, k, H, (const float*)in, in_rows, perm_pos, weights,
                       (float*)out);
  return hip_check("combine_kernel");
}

// d_prob[t][i] = sum_j partial[perm_pos[t][i]][j], j ascending (fixed order); 0 for an
// entry outside the R permuted rows.
__global__ void dprob_reduce_kernel(int n, int nparts, const float* __restrict__ partial, int64_t rows,
                                    const int32_t* __restrict__ perm_pos, float* __restrict__ d_prob) {
  int a = blockIdx.x * blockDim.x + threadIdx.x;
  if (a >= n) return;
  const int32_t pos = perm_pos[a];
  float s = 0.f;
  if (pos >= 0 && pos < rows) {
    const float* src = partial + int64_t(pos) * nparts;
    for (int j = 0; j < nparts; ++j) s += src[j];
  }
  d_prob[a] = s;
}

mge_status launch_dprob_reduce(int T, int k, int nparts, const float* partial, int64_t rows, const int32_t* perm_pos,
                               float* d_prob, hipStream_t s) {
  int n = T * k;
  if (n <= 0) return MGE_OK;
  ProfScope prof(s, "dprob_reduce");
  hipLaunchKernelGGL(dprob_reduce_kernel, dim3((n + 255) / 256), dim3(256), 0, s, n, nparts, partial, rows,
                     perm_pos, d_prob);
  return hip_check("dprob_reduce_kernel");
}

// Per-expert pointer tables travel in the kernel arguments (captured at launch) and
// land in the workspace, so host arrays may be reused as soon as the call returns.  One
// launch carries up to UP_CHUNK entries of several tables.
constexpr int UP_CHUNK = 128;
struct UploadChunk {
  void** dst;
  int n;
  int idx[UP_CHUNK];          // slot in dst
  const void* p[UP_CHUNK];
};

__global__ void upload_ptrs_kernel(UploadChunk c) {
  int i = threadIdx.x;
  if (i < c.n) c.dst[c.idx[i]] = const_cast<void*>(c.p[i]);
}

mge_status launch_upload_tables(const void* const* const* tables, int ntab, int n, void** dev_table, hipStream_t s) {
  UploadChunk c;
  c.dst = dev_table;
  c.n = 0;
  auto flush = [&]() {
    if (c.n == 0) return;
    ProfScope prof(s, "upload_ptrs");
    hipLaunchKernelGGL(upload_ptrs_kernel, dim3(1), dim3(UP_CHUNK), 0, s, c);
    c.n = 0;
  };
  for (int t = 0; t < ntab; ++t) {
    if (!tables[t]) continue;
    for (int i = 0; i < n; ++i) {
      c.idx[c.n] = t * n + i;
      c.p[c.n] = tables[t][i];
      if (++c.n == UP_CHUNK) flush();
    }
  }
  flush();
  return hip_check("upload_ptrs_kernel");
}

}  // namespace mge
