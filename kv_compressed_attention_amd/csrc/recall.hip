// Attention recall and density (paperlayer.ai section 4 "Motivation",
// attention sparsity): the dense-attention mass a sparse attention's retained
// keys keep, from the two attentions' log-sum-exp normalisers, and the share
// of keys retained.

#include "common.h"
#include "kernels.h"

namespace fastar {

namespace {

// One workgroup of 256 threads per head: per query recall = exp(lse_sparse -
// lse_dense) (0 for an empty retained set) and density = retained keys /
// n_keys; the head's means are summed in float64 in a fixed order (each
// thread's strided share, then a tree over the workgroup).
__global__ __launch_bounds__(256) void recall_kernel(const float* __restrict__ lse_s,
                                                     const float* __restrict__ lse_d, int64_t nq,
                                                     const int32_t* __restrict__ q_bucket, int P,
                                                     const int32_t* __restrict__ k_offsets, int nbits,
                                                     const int32_t* __restrict__ n_retained,
                                                     const int32_t* __restrict__ n_per_query,
                                                     const int32_t* __restrict__ n_keys,
                                                     float* __restrict__ recall, float* __restrict__ stats) {
  __shared__ double red[2][256];
  const int h = blockIdx.x;
  const double nk = (double)n_keys[h];
  const int32_t* off = k_offsets ? k_offsets + (int64_t)h * ((1 << nbits) + 1) : nullptr;
  double rs = 0.0, ds = 0.0;
  for (int64_t i = threadIdx.x; i < nq; i += blockDim.x) {
    const int64_t r = (int64_t)h * nq + i;
    const float a = lse_s[r], b = lse_d[r];
    const float rc = (a == -INFINITY || b == -INFINITY) ? 0.f : expf(a - b);
    if (recall) recall[r] = rc;
    int cnt = 0;
    if (n_per_query) {
      cnt = n_per_query[r];
    } else if (off) {
      // the keys of the query's distinct probe buckets
      const int32_t* qb = q_bucket + r * P;
      for (int p = 0; p < P; ++p) {
        bool dup = false;
        for (int p2 = 0; p2 < p; ++p2) dup = dup || qb[p2] == qb[p];
        if (!dup) cnt += off[qb[p] + 1] - off[qb[p]];
      }
    } else {
      cnt = n_retained[h];
    }
    rs += (double)rc;
    ds += nk > 0.0 ? (double)cnt / nk : 0.0;
  }
  red[0][threadIdx.x] = rs;
  red[1][threadIdx.x] = ds;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) {
      red[0][threadIdx.x] += red[0][threadIdx.x + w];
      red[1][threadIdx.x] += red[1][threadIdx.x + w];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    stats[2 * h] = nq > 0 ? (float)(red[0][0] / (double)nq) : 0.f;
    stats[2 * h + 1] = nq > 0 ? (float)(red[1][0] / (double)nq) : 0.f;
  }
}

}  // namespace

hipError_t launch_recall(const float* lse_s, const float* lse_d, int heads, int64_t nq,
                         const int32_t* q_bucket, int P, const int32_t* k_offsets, int nbits,
                         const int32_t* n_retained, const int32_t* n_keys, float* recall, float* stats,
                         hipStream_t s, const int32_t* n_per_query) {
  hipLaunchKernelGGL(recall_kernel, dim3(heads), dim3(256), 0, s, lse_s, lse_d, nq, q_bucket, P, k_offsets,
                     nbits, n_retained, n_per_query, n_keys, recall, stats);
  return hipGetLastError();
}

}  // namespace fastar
