// AnnCA prompt pruning: keep a prompt token iff some query of the current
// chunk occupies its bucket (gist.science technical summary, AnnCA: prompt
// tokens that share no bucket with any current-frame query are dropped for
// that frame; the Chinese summary's method steps say the same).
//
// One workgroup per head: the occupied set is a 2^b-bit bitmap in LDS built
// with LDS atomic OR from every probe of every query, then the prompt is
// tested and compacted in order with a ballot/popcount block scan.  With
// several LSH tables each table has its bitmap and a prompt token is kept if
// any table keeps it (q ids [ntab][H][n_q * P], prompt ids [ntab][H][n_p]).

#include "common.h"
#include "kernels.h"

namespace fastar {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / FASTAR_WAVE;

__global__ __launch_bounds__(kThreads) void prune_kernel(
    const int32_t* __restrict__ q_bucket, int64_t nqp, const int32_t* __restrict__ p_bucket,
    int64_t np, int nbits, uint8_t* __restrict__ keep, int32_t* __restrict__ kept_idx,
    int32_t* __restrict__ n_kept, int ntab) {
  __shared__ uint32_t bitmap[FASTAR_MAX_TABLES * 1024];  // up to 2^15 buckets per table
  __shared__ int wsum[kWaves];
  __shared__ int running;
  const int h = blockIdx.x;
  const int H = gridDim.x;
  const uint32_t mask = (1u << nbits) - 1u;
  const int words = ((1 << nbits) + 31) >> 5;
  for (int i = threadIdx.x; i < ntab * words; i += kThreads) bitmap[i] = 0u;
  if (threadIdx.x == 0) running = 0;
  __syncthreads();
  for (int tb = 0; tb < ntab; ++tb) {
    const int32_t* qb = q_bucket + ((int64_t)tb * H + h) * nqp;
    uint32_t* bm = bitmap + tb * words;
    for (int64_t i = threadIdx.x; i < nqp; i += kThreads) {
      const uint32_t id = (uint32_t)qb[i] & mask;
      atomicOr(&bm[id >> 5], 1u << (id & 31));
    }
  }
  __syncthreads();
  const int32_t* pb = p_bucket + (int64_t)h * np;
  uint8_t* kh = keep + (int64_t)h * np;
  int32_t* ih = kept_idx + (int64_t)h * np;
  const int wave = threadIdx.x >> 6;
  const int lane = lane_id();
  for (int64_t base = 0; base < np; base += kThreads) {
    const int64_t t = base + threadIdx.x;
    bool k = false;
    if (t < np) {
      for (int tb = 0; tb < ntab; ++tb) {
        const uint32_t id = (uint32_t)pb[(int64_t)tb * H * np + t] & mask;
        k = k || ((bitmap[tb * words + (id >> 5)] >> (id & 31)) & 1u);
      }
      kh[t] = k ? 1 : 0;
    }
    const uint64_t bal = ballot64(k);
    if (lane == 0) wsum[wave] = __popcll(bal);
    __syncthreads();
    int before = running;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    if (k) ih[before + __popcll(bal & lanemask_lt())] = (int32_t)t;
    __syncthreads();
    if (threadIdx.x == 0) {
      int s = 0;
      for (int w = 0; w < kWaves; ++w) s += wsum[w];
      running += s;
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) n_kept[h] = running;
}

}  // namespace

hipError_t launch_prune(const int32_t* q_bucket, int heads, int64_t n_q, int n_probes,
                        const int32_t* p_bucket, int64_t n_prompt, int n_bits, uint8_t* keep,
                        int32_t* kept_idx, int32_t* n_kept, hipStream_t s, int n_tables) {
  if (heads == 0) return hipSuccess;
  hipLaunchKernelGGL(prune_kernel, dim3(heads), dim3(kThreads), 0, s, q_bucket,
                     n_q * (int64_t)n_probes, p_bucket, n_prompt, n_bits, keep, kept_idx, n_kept, n_tables);
  return hipGetLastError();
}

}  // namespace fastar
