// Bucket-contiguous index: a stable sort of tokens by bucket, per head.
//
// Block-sparse bucket attention needs each bucket's members contiguous
// (gist.science technical summary, AnnSA: attention is restricted to the keys
// of the query's bucket(s) and run block-sparse).  The sort key is the bucket
// id (with several probes, the smallest of the item's probe buckets), ties in
// token order.
//
// 3..15 bits take a single stable counting pass (index_direct.h): up to 12
// bits a head split by items over up to 8 workgroups, from 13 bits by bucket
// ranges.  0..2 bits fall back to one workgroup (16 waves) per head running
// an LSD radix sort with 8-bit digits.
// Each wave owns a contiguous slice of the input and walks it 64 items at a
// time in order; items with equal digits in a 64-item group are matched with
// 8 ballots, so ranks come from popcounts and the sort is stable without
// atomics.  Per-wave digit counters live in LDS (16 x 256 ints).  A head of at
// most kLdsItems items is sorted entirely in LDS (keys and 16-bit token
// indices, double-buffered); larger heads go through the workspace.
// offsets[B] is the number of items whose key is < B: every run of
// equal buckets writes its start and a suffix minimum fills the gaps.

#include "common.h"
#include <algorithm>

#include "index_direct.h"
#include "kernels.h"

namespace fastar {

namespace {

constexpr int kWaves = 16;
constexpr int kThreads = kWaves * FASTAR_WAVE;
constexpr int U = 4;               // groups of 64 keys loaded before they are ranked
constexpr int kLdsItems = 11264;   // 2 x (4 + 2) bytes per item in LDS

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

// One stable LSD pass on the 8-bit digit at `shift`.  load(i, key, val) reads
// item i of the input, store(pos, key, val) writes the output.  Whole
// workgroup; ends with a barrier.
template <typename Load, typename Store>
__device__ __forceinline__ void radix_pass(int64_t wbeg, int64_t wend, int shift,
                                           int (*cnt)[256], int* dbase, Load load, Store store) {
  const int wave = threadIdx.x >> 6;
  const int lane = lane_id();
  for (int i = threadIdx.x; i < kWaves * 256; i += kThreads) (&cnt[0][0])[i] = 0;
  __syncthreads();
  // count the digits of this wave's slice
  for (int64_t base = wbeg; base < wend; base += U * FASTAR_WAVE) {
    int32_t key[U], val[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + u * FASTAR_WAVE + lane;
      key[u] = 0;
      if (i < wend) load(i, key[u], val[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + u * FASTAR_WAVE + lane;
      const bool valid = i < wend;
      const uint32_t digit = ((uint32_t)key[u] >> shift) & 255u;
      const uint64_t peers = match_digit(digit, valid);
      if (valid && lane == __builtin_ctzll(peers)) cnt[wave][digit] += __popcll(peers);
    }
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
  // stable scatter, same order
  for (int64_t base = wbeg; base < wend; base += U * FASTAR_WAVE) {
    int32_t key[U], val[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + u * FASTAR_WAVE + lane;
      key[u] = 0;
      val[u] = 0;
      if (i < wend) load(i, key[u], val[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + u * FASTAR_WAVE + lane;
      const bool valid = i < wend;
      const uint32_t digit = ((uint32_t)key[u] >> shift) & 255u;
      const uint64_t peers = match_digit(digit, valid);
      const int pos = valid ? cnt[wave][digit] + __popcll(peers & lanemask_lt()) : 0;
      if (valid) {
        store(pos, key[u], val[u]);
        // the leader is the lowest peer: its rank is 0, so pos is the old count
        if (lane == __builtin_ctzll(peers)) cnt[wave][digit] = pos + __popcll(peers);
      }
    }
  }
  __threadfence_block();
  __syncthreads();
}

// offsets[B] = number of sorted items whose key (>> shift0) is < B.
template <typename KeyAt>
__device__ __forceinline__ void write_offsets(int32_t* off, int nbk, int64_t nh, int shift0,
                                              KeyAt key_at, int* cmin) {
  const int lane = lane_id();
  for (int B = threadIdx.x; B <= nbk; B += kThreads) off[B] = B == nbk ? (int32_t)nh : INT_MAX;
  __threadfence_block();
  __syncthreads();
  for (int64_t p = threadIdx.x; p < nh; p += kThreads) {
    const int k = key_at(p) >> shift0;
    if (p == 0 || (key_at(p - 1) >> shift0) != k) off[k] = (int32_t)p;
  }
  __threadfence_block();
  __syncthreads();
  const int per = (nbk + 1 + kThreads - 1) / kThreads;
  const int c0 = threadIdx.x * per;
  const int c1 = c0 + per < nbk + 1 ? c0 + per : nbk + 1;
  int m = INT_MAX;
  for (int B = c0; B < c1; ++B) m = min(m, off[B]);
  cmin[threadIdx.x] = m;
  __syncthreads();
  // suffix minimum of the chunk minima: wave 0, 16 chunks per lane
  if (threadIdx.x < FASTAR_WAVE) {
    constexpr int PL = kThreads / FASTAR_WAVE;
    int v[PL];
    int run = INT_MAX;
#pragma unroll
    for (int q = PL - 1; q >= 0; --q) {
      run = min(run, cmin[lane * PL + q]);
      v[q] = run;
    }
    int incl = run;
#pragma unroll
    for (int o = 1; o < FASTAR_WAVE; o <<= 1) {
      const int y = __shfl_down(incl, o, FASTAR_WAVE);
      if (lane + o < FASTAR_WAVE) incl = min(incl, y);
    }
    int right = __shfl_down(incl, 1, FASTAR_WAVE);
    if (lane == FASTAR_WAVE - 1) right = INT_MAX;
#pragma unroll
    for (int q = 0; q < PL; ++q) cmin[lane * PL + q] = min(v[q], right);
  }
  __syncthreads();
  m = threadIdx.x + 1 < kThreads ? cmin[threadIdx.x + 1] : INT_MAX;
  for (int B = c1 - 1; B >= c0; --B) {
    m = min(m, off[B]);
    off[B] = m;
  }
}

// P: the ids' row stride (probes per item); the smallest probe is the key
__global__ __launch_bounds__(kThreads) void bucket_index_kernel(
    const int32_t* __restrict__ bucket, int P, int64_t n, int nbits, const int32_t* __restrict__ n_valid,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ ws,
    int use_lds) {
  extern __shared__ int32_t lds[];  // kLdsItems x (key, key, u16 val, u16 val)
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
  const int shift0 = 0;
  const int passes = (nbits + 7) / 8;
  const int nbk = 1 << nbits;
  int32_t* off = offsets + (int64_t)h * (nbk + 1);
  if (passes == 0) {  // one bucket: identity
    for (int64_t i = threadIdx.x; i < nh; i += kThreads) ph[i] = (int32_t)i;
    for (int B = threadIdx.x; B <= nbk; B += kThreads) off[B] = B == 0 ? 0 : (int32_t)nh;
    return;
  }
  const int wave = threadIdx.x >> 6;
  const int64_t chunk = (nh + kWaves - 1) / kWaves;
  const int64_t wbeg = (int64_t)wave * chunk < nh ? (int64_t)wave * chunk : nh;
  const int64_t wend = wbeg + chunk < nh ? wbeg + chunk : nh;
  // the sort key: the smallest probe bucket
  auto key_of = [&](int64_t i) -> int32_t { return (int32_t)index_key(ids, i, P); };
  if (use_lds && nh <= kLdsItems) {
    int32_t* ka = lds;
    int32_t* kb = ka + kLdsItems;
    uint16_t* va = reinterpret_cast<uint16_t*>(kb + kLdsItems);
    uint16_t* vb = va + kLdsItems;
    for (int64_t i = threadIdx.x; i < nh; i += kThreads) {
      ka[i] = key_of(i);
      va[i] = (uint16_t)i;
    }
    __syncthreads();
    for (int pass = 0; pass < passes; ++pass) {
      int32_t* sk = (pass & 1) ? kb : ka;
      uint16_t* sv = (pass & 1) ? vb : va;
      int32_t* dk = (pass & 1) ? ka : kb;
      uint16_t* dv = (pass & 1) ? va : vb;
      radix_pass(
          wbeg, wend, pass * 8, cnt, dbase,
          [&](int64_t i, int32_t& k, int32_t& v) {
            k = sk[i];
            v = sv[i];
          },
          [&](int pos, int32_t k, int32_t v) {
            dk[pos] = k;
            dv[pos] = (uint16_t)v;
          });
    }
    const int32_t* fk = (passes & 1) ? kb : ka;
    const uint16_t* fv = (passes & 1) ? vb : va;
    for (int64_t i = threadIdx.x; i < nh; i += kThreads) ph[i] = fv[i];
    write_offsets(off, nbk, nh, shift0, [&](int64_t p) { return fk[p]; }, &cnt[0][0]);
    return;
  }
  // workspace path: [k0 | v0 | k1 | v1] per head
  int32_t* k0 = ws + (int64_t)h * n * 4;
  int32_t* v0 = k0 + n;
  int32_t* k1 = v0 + n;
  int32_t* v1 = k1 + n;
  const int32_t* kfinal = nullptr;
  for (int pass = 0; pass < passes; ++pass) {
    const int32_t* ink = (pass & 1) ? k0 : k1;  // valid for pass >= 1
    const int32_t* inv = (pass & 1) ? v0 : v1;
    int32_t* outk = (pass & 1) ? k1 : k0;
    int32_t* outv = (pass == passes - 1) ? ph : ((pass & 1) ? v1 : v0);
    radix_pass(
        wbeg, wend, pass * 8, cnt, dbase,
        [&](int64_t i, int32_t& k, int32_t& v) {
          if (pass == 0) {
            k = key_of(i);
            v = (int32_t)i;
          } else {
            k = ink[i];
            v = inv[i];
          }
        },
        [&](int pos, int32_t k, int32_t v) {
          outk[pos] = k;
          outv[pos] = v;
        });
    kfinal = outk;
  }
  write_offsets(off, nbk, nh, shift0, [&](int64_t p) { return kfinal[p]; }, &cnt[0][0]);
}

// One workgroup per part and head; the last xparts columns build the extra
// job's index (same heads and bits).
template <int NBITS, bool WIDE>
__global__ __launch_bounds__(kDirectThreads) void bucket_index_direct_kernel(
    const int32_t* __restrict__ bucket, int P, int64_t n, const int32_t* __restrict__ n_valid,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int stage, IndexJob xj, int xparts,
    int xstage) {
  extern __shared__ int4 lds4[];
  const int nparts = (int)gridDim.x - xparts;
  if constexpr (NBITS >= kRangeMinBits) {
    if ((int)blockIdx.x >= nparts) {
      range_index_body<NBITS, WIDE>(blockIdx.y, blockIdx.x - nparts, xparts, xj.bucket, xj.P, xj.n, nullptr,
                                    xj.offsets, xj.perm, lds4);
      return;
    }
    range_index_body<NBITS, WIDE>(blockIdx.y, blockIdx.x, nparts, bucket, P, n, n_valid, offsets, perm, lds4);
  } else {
    if ((int)blockIdx.x >= nparts) {
      direct_index_body<NBITS, WIDE>(blockIdx.y, blockIdx.x - nparts, xparts, xj.bucket, xj.P, xj.n,
                                     nullptr, xj.offsets, xj.perm, xstage, lds4);
      return;
    }
    direct_index_body<NBITS, WIDE>(blockIdx.y, blockIdx.x, nparts, bucket, P, n, n_valid, offsets, perm,
                                   stage, lds4);
  }
}

// counter width of a direct launch of n items (and an extra job's n_extra)
bool direct_wide(int64_t n, int64_t n_extra) { return direct_index_wide(n) || direct_index_wide(n_extra); }

}  // namespace

bool direct_index_supported(int64_t n, int n_probes, int n_bits, int64_t n_extra, int extra_probes) {
  const bool wide = direct_wide(n, n_extra);
  return direct_index_fits_wide(n, n_probes, n_bits, wide) &&
         (n_extra <= 0 || direct_index_fits_wide(n_extra, extra_probes, n_bits, wide));
}

hipError_t launch_bucket_index(const int32_t* bucket, int heads, int64_t n, int n_probes,
                               int n_bits, const int32_t* n_valid, int32_t* offsets,
                               int32_t* perm, int32_t* ws, hipStream_t s, const IndexJob* extra) {
  if (heads == 0) return hipSuccess;
  const bool with_x = extra && extra->n > 0;
  if (with_x && (extra->n_bits != n_bits ||
                 !direct_index_supported(n, n_probes, n_bits, extra->n, extra->P)))
    return hipErrorInvalidValue;
  if (direct_index_supported(n, n_probes, n_bits, with_x ? extra->n : 0, with_x ? extra->P : 1)) {
    const bool wide = direct_wide(n, with_x ? extra->n : 0);
    int stage, xstage = 0;
    const int parts = direct_index_parts(n, n_bits, wide);
    size_t lds = direct_index_lds(n, n_bits, wide, parts, &stage);
    const int xparts = with_x ? direct_index_parts(extra->n, n_bits, wide) : 0;
    if (with_x) lds = std::max(lds, direct_index_lds(extra->n, n_bits, wide, xparts, &xstage));
    const IndexJob xj = with_x ? *extra : IndexJob{nullptr, 0, n_bits, 1, nullptr, nullptr};
    const dim3 grid(parts + xparts, heads), block(kDirectThreads);
#define FASTAR_DIRECT_W(B, W)                                                                       \
  hipLaunchKernelGGL((bucket_index_direct_kernel<B, W>), grid, block, lds, s, bucket, n_probes, n,  \
                     n_valid, offsets, perm, stage, xj, xparts, xstage)
#define FASTAR_DIRECT(B)                      \
  case B:                                     \
    if (wide) FASTAR_DIRECT_W(B, true);       \
    else FASTAR_DIRECT_W(B, false);           \
    break;
    switch (n_bits) {
      FASTAR_DIRECT(3) FASTAR_DIRECT(4) FASTAR_DIRECT(5) FASTAR_DIRECT(6) FASTAR_DIRECT(7)
      FASTAR_DIRECT(8) FASTAR_DIRECT(9) FASTAR_DIRECT(10) FASTAR_DIRECT(11) FASTAR_DIRECT(12)
      FASTAR_DIRECT(13) FASTAR_DIRECT(14) FASTAR_DIRECT(15)
    }
#undef FASTAR_DIRECT
#undef FASTAR_DIRECT_W
    return hipGetLastError();
  }
  // LDS staging whenever a head can fit (n, or a device count, at most kLdsItems)
  const int use_lds = (n <= kLdsItems || n_valid) ? 1 : 0;
  const size_t lds = use_lds ? (size_t)kLdsItems * 12 : 0;
  hipLaunchKernelGGL(bucket_index_kernel, dim3(heads), dim3(kThreads), lds, s, bucket, n_probes, n, n_bits,
                     n_valid, offsets, perm, ws, use_lds);
  return hipGetLastError();
}

}  // namespace fastar
