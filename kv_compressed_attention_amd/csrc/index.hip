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
// atomics.  Per-wave digit counters live in LDS (16 x 256 ints).  A head of at
// most kLdsItems items is sorted entirely in LDS (keys and 16-bit token
// indices, double-buffered); larger heads go through the workspace.
// offsets[B] is the number of items whose first bucket is < B: every run of
// equal buckets writes its start and a suffix minimum fills the gaps.  One
// probe with at most 12 bits takes a single counting pass instead (below).

#include "common.h"
#include "kernels.h"

namespace fastar {

namespace {

constexpr int kWaves = 16;
constexpr int kThreads = kWaves * FASTAR_WAVE;
constexpr int U = 4;               // groups of 64 keys loaded before they are ranked
constexpr int kLdsItems = 11264;   // 2 x (4 + 2) bytes per item in LDS

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

// offsets[B] = number of sorted items whose first bucket (key >> shift0) < B.
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

template <int P>
__global__ __launch_bounds__(kThreads) void bucket_index_kernel(
    const int32_t* __restrict__ bucket, int64_t n, int nbits, const int32_t* __restrict__ n_valid,
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
  const int shift0 = (P == 2) ? 4 : 0;
  const int passes = (nbits + shift0 + 7) / 8;
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
  auto key_of = [&](int64_t i) -> int32_t {
    return P == 2 ? ((ids[2 * i] << 4) | flip_bit(ids[2 * i], ids[2 * i + 1])) : ids[i];
  };
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

// One probe, 3..12 bits, at most 65535 items: a single stable counting pass.
// Per-wave 16-bit bucket counters (kDirectWaves x 2^b) fit in LDS; one scan
// over (bucket, wave) gives each wave's scatter bases and the offsets.  With
// `stage`, the permutation is assembled in LDS and written out coalesced.
constexpr int kDirectWaves = 8;
constexpr int kDirectMinBits = 3;
constexpr int kDirectMaxBits = 12;
constexpr int64_t kDirectMaxItems = 65535;
constexpr int64_t kDirectStageItems = 24000;

__device__ __forceinline__ uint32_t half16(const int4& v, int e) {
  const uint32_t w = (uint32_t)(e < 2 ? v.x : e < 4 ? v.y : e < 6 ? v.z : v.w);
  return (e & 1) ? (w >> 16) : (w & 0xFFFFu);
}

template <int NBITS>
__global__ __launch_bounds__(kDirectWaves * FASTAR_WAVE) void bucket_index_direct_kernel(
    const int32_t* __restrict__ bucket, int64_t n, const int32_t* __restrict__ n_valid,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int stage) {
  constexpr int nbits = NBITS;
  // [kDirectWaves][2^nbits] uint16 counters (8 per 128-bit word), then the
  // staged permutation (int32, n entries) when stage is set
  extern __shared__ int4 lds4[];
  __shared__ int wtot[kDirectWaves];
  constexpr int NT = kDirectWaves * FASTAR_WAVE;
  static_assert((1 << kDirectMaxBits) / 8 == NT, "one 8-bucket group per thread");
  const int h = blockIdx.x;
  int64_t nh = n;
  if (n_valid) {
    const int64_t v = n_valid[h];
    nh = v < 0 ? 0 : (v < n ? v : n);
  }
  const int nbk = 1 << nbits;
  const int nb8 = nbk >> 3;
  uint16_t* cnt = reinterpret_cast<uint16_t*>(lds4);
  uint32_t* cnt32 = reinterpret_cast<uint32_t*>(lds4);
  int32_t* pst = reinterpret_cast<int32_t*>(lds4 + kDirectWaves * nb8);
  const uint32_t bmask = (uint32_t)nbk - 1u;
  const int32_t* ids = bucket + (int64_t)h * n;
  int32_t* ph = perm + (int64_t)h * n;
  int32_t* off = offsets + (int64_t)h * (nbk + 1);
  const int wave = threadIdx.x >> 6;
  const int lane = lane_id();
  for (int i = threadIdx.x; i < kDirectWaves * nb8; i += NT) lds4[i] = make_int4(0, 0, 0, 0);
  __syncthreads();
  const int64_t chunk = (nh + kDirectWaves - 1) / kDirectWaves;
  const int64_t wbeg = (int64_t)wave * chunk < nh ? (int64_t)wave * chunk : nh;
  const int64_t wend = wbeg + chunk < nh ? wbeg + chunk : nh;
  const int wrow = wave * nbk;
  // the wave's slice is handled in tiles of kTile ids per lane, loaded together
  constexpr int kTile = 16;
  // a slice of one tile keeps its ids in registers for the scatter
  const bool one_tile = wend - wbeg <= kTile * FASTAR_WAVE;
  uint32_t b[kTile];
  for (int64_t t0 = wbeg; t0 < wend; t0 += kTile * FASTAR_WAVE) {
#pragma unroll
    for (int r = 0; r < kTile; ++r) {
      const int64_t i = t0 + r * FASTAR_WAVE + lane;
      b[r] = i < wend ? ((uint32_t)ids[i] & bmask) : 0xFFFFFFFFu;
    }
    // counts (order does not matter): the 16-bit counter in its 32-bit word
#pragma unroll
    for (int r = 0; r < kTile; ++r)
      if (b[r] != 0xFFFFFFFFu)
        atomicAdd(&cnt32[(wrow + (int)b[r]) >> 1], 1u << (16 * (b[r] & 1u)));
  }
  __syncthreads();
  // exclusive scan over (bucket, wave): thread t owns buckets 8t .. 8t + 7,
  // one 128-bit word per wave
  const int t = threadIdx.x;
  int4 cw[kDirectWaves];
  uint32_t tot[8];
  uint32_t local = 0;
#pragma unroll
  for (int w = 0; w < kDirectWaves; ++w) cw[w] = t < nb8 ? lds4[w * nb8 + t] : make_int4(0, 0, 0, 0);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    tot[e] = 0;
#pragma unroll
    for (int w = 0; w < kDirectWaves; ++w) tot[e] += half16(cw[w], e);
    local += tot[e];
  }
  uint32_t incl = local;
#pragma unroll
  for (int o = 1; o < FASTAR_WAVE; o <<= 1) {
    const uint32_t y = (uint32_t)__shfl_up((int)incl, o, FASTAR_WAVE);
    if (lane >= o) incl += y;
  }
  if (lane == FASTAR_WAVE - 1) wtot[wave] = (int)incl;
  __syncthreads();
  uint32_t run = incl - local;
  for (int w = 0; w < wave; ++w) run += (uint32_t)wtot[w];
  if (t < nb8) {
    uint32_t base[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      base[e] = run;
      run += tot[e];
    }
    // each wave's base within each bucket
#pragma unroll
    for (int w = 0; w < kDirectWaves; ++w) {
      lds4[w * nb8 + t] = make_int4((int)(base[0] | (base[1] << 16)), (int)(base[2] | (base[3] << 16)),
                                    (int)(base[4] | (base[5] << 16)), (int)(base[6] | (base[7] << 16)));
#pragma unroll
      for (int e = 0; e < 8; ++e) base[e] += half16(cw[w], e);
    }
  }
  __syncthreads();
  // stable scatter: each wave walks its slice in order, 64 tokens at a time
  for (int64_t t0 = wbeg; t0 < wend; t0 += kTile * FASTAR_WAVE) {
    uint32_t bt[kTile];
#pragma unroll
    for (int r = 0; r < kTile; ++r) {
      const int64_t i = t0 + r * FASTAR_WAVE + lane;
      bt[r] = one_tile ? (b[r] & bmask) : (i < wend ? ((uint32_t)ids[i] & bmask) : 0u);
    }
#pragma unroll
    for (int r = 0; r < kTile; ++r) {
      const int64_t i = t0 + r * FASTAR_WAVE + lane;
      if (t0 + r * FASTAR_WAVE >= wend) break;  // uniform
      const bool valid = i < wend;
      const uint32_t bb = bt[r];
      // lanes of this row with the same bucket: those agreeing on every bit
      // (lanes past the end are out of the first ballot)
      uint64_t peers = ballot64(valid);
#pragma unroll
      for (int k = 0; k < NBITS; ++k) {
        const uint32_t bit = (bb >> k) & 1u;
        const uint64_t bk = ballot64(bit != 0u);
        peers &= ~(bk ^ (0ull - (uint64_t)bit));
      }
      if (valid) {
        const int rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(peers >> 32),
                                                   __builtin_amdgcn_mbcnt_lo((uint32_t)peers, 0u));
        const int pos = (int)cnt[wrow + (int)bb] + rank;
        // two stores, not one through a generic pointer: an LDS store must
        // not take the flat path that the next counter read would wait on
        if (stage) pst[pos] = (int32_t)i;
        else ph[pos] = (int32_t)i;
        // the lowest peer (rank 0) advances the counter
        if (rank == 0) cnt[wrow + (int)bb] = (uint16_t)(pos + __popcll(peers));
      }
    }
  }
  // after the scatter the last wave's counter of bucket B has reached the
  // start of bucket B + 1: the offsets are written from it, coalesced, and so
  // is a staged permutation
  __syncthreads();
  const uint16_t* last = cnt + (kDirectWaves - 1) * nbk;
  for (int B = threadIdx.x; B <= nbk; B += NT) off[B] = B == 0 ? 0 : (int32_t)last[B - 1];
  if (stage)
    for (int64_t p = threadIdx.x; p < nh; p += NT) ph[p] = pst[p];
}

}  // namespace

hipError_t launch_bucket_index(const int32_t* bucket, int heads, int64_t n, int n_probes,
                               int n_bits, const int32_t* n_valid, int32_t* offsets,
                               int32_t* perm, int32_t* ws, hipStream_t s) {
  if (heads == 0) return hipSuccess;
  if (n_probes == 1 && n_bits >= kDirectMinBits && n_bits <= kDirectMaxBits && n <= kDirectMaxItems) {
    const int stage = n <= kDirectStageItems ? 1 : 0;
    const size_t lds = (size_t)kDirectWaves * ((size_t)1 << n_bits) * sizeof(uint16_t) +
                       (stage ? (size_t)n * sizeof(int32_t) : 0);
    const dim3 grid(heads), block(kDirectWaves * FASTAR_WAVE);
    switch (n_bits) {
#define FASTAR_DIRECT(B)                                                                         \
  case B:                                                                                         \
    hipLaunchKernelGGL(bucket_index_direct_kernel<B>, grid, block, lds, s, bucket, n, n_valid,    \
                       offsets, perm, stage);                                                     \
    break;
      FASTAR_DIRECT(3) FASTAR_DIRECT(4) FASTAR_DIRECT(5) FASTAR_DIRECT(6) FASTAR_DIRECT(7)
      FASTAR_DIRECT(8) FASTAR_DIRECT(9) FASTAR_DIRECT(10) FASTAR_DIRECT(11) FASTAR_DIRECT(12)
#undef FASTAR_DIRECT
    }
    return hipGetLastError();
  }
  // LDS staging whenever a head can fit (n, or a device count, at most kLdsItems)
  const int use_lds = (n <= kLdsItems || n_valid) ? 1 : 0;
  const size_t lds = use_lds ? (size_t)kLdsItems * 12 : 0;
  if (n_probes == 2)
    hipLaunchKernelGGL(bucket_index_kernel<2>, dim3(heads), dim3(kThreads), lds, s, bucket, n,
                       n_bits, n_valid, offsets, perm, ws, use_lds);
  else
    hipLaunchKernelGGL(bucket_index_kernel<1>, dim3(heads), dim3(kThreads), lds, s, bucket, n,
                       n_bits, n_valid, offsets, perm, ws, use_lds);
  return hipGetLastError();
}

}  // namespace fastar
