// Bucket-contiguous index: a stable sort of tokens by bucket, per head.
//
// Block-sparse bucket attention needs each bucket's members contiguous
// (gist.science technical summary, AnnSA: attention is restricted to the keys
// of the query's bucket(s) and run block-sparse).  With one probe the sort key
// is the bucket id; with two probes it is (first bucket, flipped bit), so that
// queries sharing their second bucket sit together.
//
// One workgroup (16 waves) per head runs an LSD radix sort with 8-bit digits.
// Each wave owns a contiguous slice of the input and walks it 64 items at a
// time in order; items with equal digits in a 64-item group are matched with
// 8 ballots, so ranks come from popcounts and the sort is stable without
// atomics.  Per-wave digit counters live in LDS (16 x 256 ints).  offsets[B]
// is the lower bound of B in the sorted first-bucket column.

#include "common.h"
#include "kernels.h"

namespace fastar {

namespace {

constexpr int kWaves = 16;
constexpr int kThreads = kWaves * FASTAR_WAVE;

__device__ __forceinline__ int32_t flip_bit(int32_t a, int32_t b) {
  const uint32_t x = (uint32_t)(a ^ b);
  return x ? (int32_t)__builtin_ctz(x) : 0;
}

// peers: lanes of this wave holding the same 8-bit digit (valid lanes only)
__device__ __forceinline__ uint64_t match_digit(uint32_t digit, bool valid) {
  uint64_t peers = ballot64(valid);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const bool bit = (digit >> k) & 1u;
    const uint64_t bk = ballot64(valid && bit);
    peers &= bit ? bk : ~bk;
  }
  return peers;
}

template <int P>
__global__ __launch_bounds__(kThreads) void bucket_index_kernel(
    const int32_t* __restrict__ bucket, int64_t n, int nbits, const int32_t* __restrict__ n_valid,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ ws) {
  __shared__ int cnt[kWaves][256];
  __shared__ int dbase[256];
  const int h = blockIdx.x;
  int64_t nh = n;
  if (n_valid) {
    const int64_t v = n_valid[h];
    nh = v < 0 ? 0 : (v < n ? v : n);
  }
  const int32_t* ids = bucket + (int64_t)h * n * P;
  int32_t* ph = perm + (int64_t)h * n;
  int32_t* k0 = ws + (int64_t)h * n * 4;
  int32_t* v0 = k0 + n;
  int32_t* k1 = v0 + n;
  int32_t* v1 = k1 + n;
  const int shift0 = (P == 2) ? 4 : 0;
  const int keybits = nbits + shift0;
  const int passes = (keybits + 7) / 8;
  const int wave = threadIdx.x >> 6;
  const int lane = lane_id();
  const int64_t chunk = (nh + kWaves - 1) / kWaves;
  const int64_t wbeg = (int64_t)wave * chunk < nh ? (int64_t)wave * chunk : nh;
  const int64_t wend = wbeg + chunk < nh ? wbeg + chunk : nh;
  const int32_t* kfinal = nullptr;

  if (passes == 0) {
    for (int64_t i = threadIdx.x; i < nh; i += kThreads) ph[i] = (int32_t)i;
  }
  for (int pass = 0; pass < passes; ++pass) {
    const int shift = pass * 8;
    const int32_t* ink = (pass & 1) ? k0 : k1;  // valid for pass >= 1
    const int32_t* inv = (pass & 1) ? v0 : v1;
    int32_t* outk = (pass & 1) ? k1 : k0;
    int32_t* outv = (pass == passes - 1) ? ph : ((pass & 1) ? v1 : v0);
    for (int i = threadIdx.x; i < kWaves * 256; i += kThreads) (&cnt[0][0])[i] = 0;
    __syncthreads();
    // count digits of this wave's slice
    for (int64_t base = wbeg; base < wend; base += FASTAR_WAVE) {
      const int64_t i = base + lane;
      const bool valid = i < wend;
      int32_t key = 0;
      if (valid) {
        if (pass == 0) key = P == 2 ? ((ids[2 * i] << 4) | flip_bit(ids[2 * i], ids[2 * i + 1])) : ids[i];
        else key = ink[i];
      }
      const uint32_t digit = ((uint32_t)key >> shift) & 255u;
      const uint64_t peers = match_digit(digit, valid);
      if (valid && lane == __builtin_ctzll(peers)) cnt[wave][digit] += __popcll(peers);
    }
    __syncthreads();
    // exclusive scan in (digit, wave) order
    if (threadIdx.x < 256) {
      int run = 0;
      for (int w = 0; w < kWaves; ++w) {
        const int c = cnt[w][threadIdx.x];
        cnt[w][threadIdx.x] = run;
        run += c;
      }
      dbase[threadIdx.x] = run;
    }
    __syncthreads();
    if (threadIdx.x < FASTAR_WAVE) {
      int t[4];
      int s = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        t[j] = dbase[4 * lane + j];
        s += t[j];
      }
      int incl = s;
#pragma unroll
      for (int off = 1; off < FASTAR_WAVE; off <<= 1) {
        const int y = __shfl_up(incl, off, FASTAR_WAVE);
        if (lane >= off) incl += y;
      }
      int ex = incl - s;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        dbase[4 * lane + j] = ex;
        ex += t[j];
      }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < kWaves * 256; i += kThreads) (&cnt[0][0])[i] += dbase[i & 255];
    __syncthreads();
    // stable scatter
    for (int64_t base = wbeg; base < wend; base += FASTAR_WAVE) {
      const int64_t i = base + lane;
      const bool valid = i < wend;
      int32_t key = 0, val = 0;
      if (valid) {
        if (pass == 0) {
          key = P == 2 ? ((ids[2 * i] << 4) | flip_bit(ids[2 * i], ids[2 * i + 1])) : ids[i];
          val = (int32_t)i;
        } else {
          key = ink[i];
          val = inv[i];
        }
      }
      const uint32_t digit = ((uint32_t)key >> shift) & 255u;
      const uint64_t peers = match_digit(digit, valid);
      const int pos = valid ? cnt[wave][digit] + __popcll(peers & lanemask_lt()) : 0;
      if (valid) {
        outk[pos] = key;
        outv[pos] = val;
        // the leader is the lowest peer: its rank is 0, so pos is the old count
        if (lane == __builtin_ctzll(peers)) cnt[wave][digit] = pos + __popcll(peers);
      }
    }
    __threadfence_block();
    __syncthreads();
    kfinal = outk;
  }
  // offsets[B] = #items whose first bucket < B: each run of equal buckets
  // writes its start, then a suffix minimum fills the empty buckets
  const int nbk = 1 << nbits;
  int32_t* off = offsets + (int64_t)h * (nbk + 1);
  if (passes == 0) {
    for (int B = threadIdx.x; B <= nbk; B += kThreads) off[B] = B == 0 ? 0 : (int32_t)nh;
    return;
  }
  for (int B = threadIdx.x; B <= nbk; B += kThreads) off[B] = B == nbk ? (int32_t)nh : INT_MAX;
  __threadfence_block();
  __syncthreads();
  for (int64_t p = threadIdx.x; p < nh; p += kThreads) {
    const int k = kfinal[p] >> shift0;
    if (p == 0 || (kfinal[p - 1] >> shift0) != k) off[k] = (int32_t)p;
  }
  __threadfence_block();
  __syncthreads();
  int* cmin = &cnt[0][0];  // [kThreads] chunk minima
  const int per = (nbk + 1 + kThreads - 1) / kThreads;
  const int c0 = threadIdx.x * per;
  const int c1 = c0 + per < nbk + 1 ? c0 + per : nbk + 1;
  int m = INT_MAX;
  for (int B = c0; B < c1; ++B) m = min(m, off[B]);
  cmin[threadIdx.x] = m;
  __syncthreads();
  // suffix minimum of the chunk minima (Hillis-Steele, reading to the right)
  for (int d = 1; d < kThreads; d <<= 1) {
    const int y = threadIdx.x + d < kThreads ? cmin[threadIdx.x + d] : INT_MAX;
    __syncthreads();
    cmin[threadIdx.x] = min(cmin[threadIdx.x], y);
    __syncthreads();
  }
  m = threadIdx.x + 1 < kThreads ? cmin[threadIdx.x + 1] : INT_MAX;
  for (int B = c1 - 1; B >= c0; --B) {
    m = min(m, off[B]);
    off[B] = m;
  }
}

}  // namespace

hipError_t launch_bucket_index(const int32_t* bucket, int heads, int64_t n, int n_probes,
                               int n_bits, const int32_t* n_valid, int32_t* offsets,
                               int32_t* perm, int32_t* ws, hipStream_t s) {
  if (heads == 0) return hipSuccess;
  if (n_probes == 2)
    hipLaunchKernelGGL(bucket_index_kernel<2>, dim3(heads), dim3(kThreads), 0, s, bucket, n,
                       n_bits, n_valid, offsets, perm, ws);
  else
    hipLaunchKernelGGL(bucket_index_kernel<1>, dim3(heads), dim3(kThreads), 0, s, bucket, n,
                       n_bits, n_valid, offsets, perm, ws);
  return hipGetLastError();
}

}  // namespace fastar
