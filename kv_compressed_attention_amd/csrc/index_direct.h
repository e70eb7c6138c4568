// Stable counting-sort bucket index (see index.hip) as a workgroup-level
// body, so that other launches can run it in workgroups of their own.
#pragma once

#include <type_traits>

#include "common.h"

namespace fastar {

// A single stable counting pass for 3..12 bits, any probe count (the sort
// key is the smallest of an item's probe buckets), any item count below 2^31 that the
// counters allow.  Per-wave bucket counters (one row of 2^b per scattering
// wave) sit in LDS: 16-bit while a head has at most 65535 items, 32-bit
// above.  One scan over (bucket, row) gives each wave its scatter bases and
// the offsets.  A head may be split into parts, one workgroup each: a part
// scatters its own slice of the items and counts the others (those before
// the slice and those after it, per bucket, in two more rows) to place it,
// so the parts need no exchange.  With `stage` (one part, room left in LDS)
// the permutation is assembled in LDS and written out coalesced.
// the sort key of item i of ids [n][P]: the smallest of its P probe buckets
// (queries probing the same bucket pair then sit together)
__device__ __forceinline__ uint32_t index_key(const int32_t* ids, int64_t i, int P) {
  const int32_t* r = ids + i * P;
  int m = r[0];
  if (P == 2) {
    m = min(m, r[1]);
  } else {
    for (int p = 1; p < P; ++p) m = min(m, r[p]);
  }
  return (uint32_t)m;
}

constexpr int kDirectWaves = 16;
constexpr int kDirectThreads = kDirectWaves * FASTAR_WAVE;
// waves that scatter a part's slice when a head has several parts, at most
constexpr int kDirectPartWaves = 8;
constexpr int kDirectMinBits = 3;
constexpr int kDirectMaxBits = 15;
// 13 bits and more: the parts of a head split its buckets, not its items
// (range_index_body); the counter rows of a part then take 64 KB of LDS, so
// that an index workgroup fits on a CU beside other launches' workgroups
constexpr int kRangeMinBits = 13;
constexpr int kRangeRowBytes = 64 * 1024 / 16;  // per scattering wave
// 16-bit counters up to this many items per head
constexpr int64_t kDirectNarrowItems = 65535;
// parts per head: about this many items each, at most kDirectMaxParts
constexpr int64_t kDirectPartItems = 1536;
constexpr int kDirectMaxParts = 8;
// LDS for the counter rows, and for counters plus a staged permutation
constexpr size_t kDirectCounterLds = 128 * 1024;
constexpr size_t kDirectLds = 152 * 1024;

// scattering waves and counter rows of a part
struct DirectShape {
  int sw, rows;
};
__host__ __device__ inline DirectShape direct_shape(int n_bits, bool wide, int nparts) {
  const size_t row = ((size_t)1 << n_bits) * (wide ? 4u : 2u);
  const int fit = (int)(kDirectCounterLds / row);
  DirectShape s;
  if (nparts == 1) {
    s.sw = fit < kDirectWaves ? fit : kDirectWaves;
    s.rows = s.sw;
  } else {
    s.sw = fit - 2 < kDirectPartWaves ? fit - 2 : kDirectPartWaves;
    s.rows = s.sw + 2;
  }
  return s;
}
// 32-bit counters for n items
inline bool direct_index_wide(int64_t n) { return n > kDirectNarrowItems; }
constexpr int ilog2_c(int v) { return v > 1 ? 1 + ilog2_c(v >> 1) : 0; }
// buckets of one part of a head in range mode
__host__ __device__ constexpr int range_part_buckets(bool wide) { return kRangeRowBytes / (wide ? 4 : 2); }
// The parts (workgroups) per head for n items
inline int direct_index_parts(int64_t n, int n_bits, bool wide) {
  if (n_bits >= kRangeMinBits) return (1 << n_bits) / range_part_buckets(wide);
  const int64_t p = (n + kDirectPartItems - 1) / kDirectPartItems;
  return p < 1 ? 1 : (p > kDirectMaxParts ? kDirectMaxParts : (int)p);
}
// whether the direct pass covers n items of n_bits bits with counters of the
// given width
inline bool direct_index_fits_wide(int64_t n, int n_probes, int n_bits, bool wide) {
  if (n_probes < 1 || n_probes > kMaxProbes || n_bits < kDirectMinBits || n_bits > kDirectMaxBits) return false;
  if (n >= ((int64_t)1 << 31) || (!wide && direct_index_wide(n))) return false;
  if (n_bits >= kRangeMinBits) return true;
  return direct_shape(n_bits, wide, direct_index_parts(n, n_bits, wide)).sw >= 1;
}
inline bool direct_index_fits(int64_t n, int n_probes, int n_bits) {
  return direct_index_fits_wide(n, n_probes, n_bits, direct_index_wide(n));
}
// LDS bytes the direct index of n items in nparts parts needs, and whether it
// stages the permutation there
inline size_t direct_index_lds(int64_t n, int n_bits, bool wide, int nparts, int* stage) {
  if (n_bits >= kRangeMinBits) {
    *stage = 0;
    return (size_t)kDirectWaves * kRangeRowBytes;
  }
  const DirectShape sh = direct_shape(n_bits, wide, nparts);
  const size_t counters = (size_t)sh.rows * ((size_t)1 << n_bits) * (wide ? 4u : 2u);
  *stage = nparts == 1 && counters + (size_t)n * sizeof(int32_t) <= kDirectLds ? 1 : 0;
  return counters + (*stage ? (size_t)n * sizeof(int32_t) : 0);
}

// Part `part` of nparts of the index of head h (ids [H][n][P], sorted by
// their smallest probe), by one workgroup of kDirectWaves waves.  lds4: the
// dynamic LDS of direct_index_lds bytes.
template <int NBITS, bool WIDE>
__device__ __forceinline__ void direct_index_body(int h, int part, int nparts,
                                                  const int32_t* __restrict__ bucket, int P, int64_t n,
                                                  const int32_t* __restrict__ n_valid,
                                                  int32_t* __restrict__ offsets,
                                                  int32_t* __restrict__ perm, int stage, int4* lds4) {
  constexpr int nbits = NBITS;
  constexpr int nbk = 1 << nbits;
  // buckets per thread in the scan, in groups of 4
  constexpr int BPT = nbk / kDirectThreads > 4 ? nbk / kDirectThreads : 4;
  constexpr int NG = BPT / 4;
  using CT = typename std::conditional<WIDE, uint32_t, uint16_t>::type;
  using CT4 = typename std::conditional<WIDE, uint4, uint2>::type;  // 4 counters
  static_assert(nbk % 4 == 0, "whole 4-bucket groups");
  // lds4: [rows][2^nbits] counters (the scattering waves' rows, then with
  // several parts the counts of the items before and after this part's
  // slice), then the staged permutation (int32, n entries) when stage is set
  __shared__ int wtot[kDirectWaves];
  int nh = (int)n;
  if (n_valid) {
    const int v = n_valid[h];
    nh = v < 0 ? 0 : (v < nh ? v : nh);
  }
  const bool split = nparts > 1;
  const DirectShape shape = direct_shape(nbits, WIDE, nparts);
  const int sw = shape.sw, rows = shape.rows;
  CT* cnt = reinterpret_cast<CT*>(lds4);
  uint32_t* cnt32 = reinterpret_cast<uint32_t*>(lds4);
  CT4* cnt4 = reinterpret_cast<CT4*>(lds4);
  constexpr int kPerInt4 = 16 / sizeof(CT);
  int32_t* pst = reinterpret_cast<int32_t*>(lds4 + rows * (nbk / kPerInt4));
  const uint32_t bmask = (uint32_t)nbk - 1u;
  const int32_t* ids = bucket + (int64_t)h * n * P;
  int32_t* ph = perm + (int64_t)h * n;
  int32_t* off = offsets + (int64_t)h * (nbk + 1);
  const int wave = threadIdx.x >> 6;
  const int lane = lane_id();
  if (nh == 0) {  // the whole workgroup: every bucket is empty
    if (part == 0)
      for (int B = threadIdx.x; B <= nbk; B += kDirectThreads) off[B] = 0;
    return;
  }
  // one counter up by one (LDS atomics; 16-bit counters in their 32-bit word)
  auto inc = [&](int row, uint32_t b) {
    const int i = row * nbk + (int)b;
    if (WIDE) atomicAdd(&cnt32[i], 1u);
    else atomicAdd(&cnt32[i >> 1], 1u << (16 * (b & 1u)));
  };
  // this part's slice [sb, se), and the share [wbeg, wend) of wave w < sw
  const int pchunk = (nh + nparts - 1) / nparts;
  const int sb = part * pchunk < nh ? part * pchunk : nh;
  const int se = sb + pchunk < nh ? sb + pchunk : nh;
  const int chunk = (se - sb + sw - 1) / sw;
  const int wbeg = wave < sw && sb + wave * chunk < se ? sb + wave * chunk : se;
  const int wend = wbeg + chunk < se ? wbeg + chunk : se;
  const int wrow = wave * nbk;
  // the wave's share is handled in tiles of kTile ids per lane, loaded
  // together; a share of one tile keeps its ids in registers for the scatter
  constexpr int kTile = 16;
  const bool one_tile = wend - wbeg <= kTile * FASTAR_WAVE;
  // the other items (several parts) in batches of kBatch per thread: j walks
  // them with the slice cut out
  constexpr int kBatch = 8;
  const int nother = split ? nh - (se - sb) : 0;
  // loads are unconditional (at an index clamped into the items), so that
  // they all go out before the first wait
  const int last = nh - 1;
  uint32_t b[kTile], ob[kBatch];
  auto load_tile = [&](int t0) {
#pragma unroll
    for (int r = 0; r < kTile; ++r) {
      const int i = t0 + r * FASTAR_WAVE + lane;
      const uint32_t v = index_key(ids, i < last ? i : last, P);
      b[r] = i < wend ? (v & bmask) : 0xFFFFFFFFu;
    }
  };
  auto load_batch = [&](int j0) {
#pragma unroll
    for (int r = 0; r < kBatch; ++r) {
      const int j = j0 + r * kDirectThreads + (int)threadIdx.x;
      const int i = j < sb ? j : j + (se - sb);
      const uint32_t v = index_key(ids, i < last ? i : last, P);
      ob[r] = j < nother ? (v & bmask) : 0xFFFFFFFFu;
    }
  };
  // the first loads are in flight while the counters are cleared (the
  // barriers below order LDS only: this workgroup reads no global memory that
  // it writes)
  load_tile(wbeg);
  load_batch(0);
  for (int i = threadIdx.x; i < rows * (nbk / kPerInt4); i += kDirectThreads) lds4[i] = make_int4(0, 0, 0, 0);
  lds_barrier();
  // counts (order does not matter)
  for (int t0 = wbeg; t0 < wend;) {
#pragma unroll
    for (int r = 0; r < kTile; ++r)
      if (b[r] != 0xFFFFFFFFu) inc(wave, b[r]);
    t0 += kTile * FASTAR_WAVE;
    if (t0 >= wend) break;
    load_tile(t0);
  }
  // before the slice into row sw, after it into row sw + 1
  for (int j0 = 0; j0 < nother;) {
#pragma unroll
    for (int r = 0; r < kBatch; ++r) {
      const int j = j0 + r * kDirectThreads + (int)threadIdx.x;
      if (ob[r] != 0xFFFFFFFFu) inc(j < sb ? sw : sw + 1, ob[r]);
    }
    j0 += kBatch * kDirectThreads;
    if (j0 >= nother) break;
    load_batch(j0);
  }
  lds_barrier();
  // exclusive scan over (bucket, row): thread t owns buckets BPT t .. + BPT,
  // four counters per LDS access
  const int t = threadIdx.x;
  const bool owner = t < nbk / BPT;
  const int g0 = t * NG;  // its first 4-bucket group
  auto get4 = [&](int w, int gi, uint32_t* o) {
    const CT4 c = cnt4[w * (nbk / 4) + g0 + gi];
    if constexpr (WIDE) {
      o[0] = c.x; o[1] = c.y; o[2] = c.z; o[3] = c.w;
    } else {
      o[0] = c.x & 0xFFFFu; o[1] = c.x >> 16; o[2] = c.y & 0xFFFFu; o[3] = c.y >> 16;
    }
  };
  auto put4 = [&](int w, int gi, const uint32_t* v) {
    if constexpr (WIDE) cnt4[w * (nbk / 4) + g0 + gi] = make_uint4(v[0], v[1], v[2], v[3]);
    else cnt4[w * (nbk / 4) + g0 + gi] = make_uint2(v[0] | (v[1] << 16), v[2] | (v[3] << 16));
  };
  uint32_t tot[BPT];
#pragma unroll
  for (int e = 0; e < BPT; ++e) tot[e] = 0u;
  if (owner) {
    for (int w = 0; w < rows; ++w) {
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) {
        uint32_t c[4];
        get4(w, gi, c);
#pragma unroll
        for (int e = 0; e < 4; ++e) tot[4 * gi + e] += c[e];
      }
    }
  }
  uint32_t local = 0u;
#pragma unroll
  for (int e = 0; e < BPT; ++e) local += tot[e];
  const uint32_t incl = wave_incl_scan_dpp(local);
  if (lane == FASTAR_WAVE - 1) wtot[wave] = (int)incl;
  lds_barrier();
  // plus the totals of the waves before (one load per lane, then a sum)
  const int wt = lane < kDirectWaves ? wtot[lane] : 0;
  uint32_t run = incl - local + (uint32_t)wave_sum_dpp(lane < wave ? wt : 0);
  if (owner) {
    uint32_t base[BPT];
#pragma unroll
    for (int e = 0; e < BPT; ++e) {
      base[e] = run;
      run += tot[e];
    }
    // the bucket starts; part 0 writes the offsets
    if (part == 0) {
#pragma unroll
      for (int e = 0; e < BPT; ++e) off[t * BPT + e] = (int)base[e];
      if (t == nbk / BPT - 1) off[nbk] = (int)run;
    }
    if (split) {
      // this part's items follow those before its slice
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) {
        uint32_t c[4];
        get4(sw, gi, c);
#pragma unroll
        for (int e = 0; e < 4; ++e) base[4 * gi + e] += c[e];
      }
    }
    // each wave's base within each bucket (replacing the wave's counts)
    for (int w = 0; w < sw; ++w) {
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) {
        uint32_t c[4];
        get4(w, gi, c);
        put4(w, gi, &base[4 * gi]);
#pragma unroll
        for (int e = 0; e < 4; ++e) base[4 * gi + e] += c[e];
      }
    }
  }
  lds_barrier();
  // stable scatter: each wave walks its share in order, 64 tokens at a time
  for (int t0 = wbeg; t0 < wend; t0 += kTile * FASTAR_WAVE) {
    if (!one_tile) load_tile(t0);
#pragma unroll
    for (int r = 0; r < kTile; ++r) {
      const int i = t0 + r * FASTAR_WAVE + lane;
      if (t0 + r * FASTAR_WAVE >= wend) break;  // uniform
      const bool valid = i < wend;
      const uint32_t bb = b[r] & bmask;
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
        if (rank == 0) cnt[wrow + (int)bb] = (CT)(pos + __popcll(peers));
      }
    }
  }
  // a staged permutation is written out coalesced
  if (stage) {
    lds_barrier();
    for (int p = threadIdx.x; p < nh; p += kDirectThreads) ph[p] = pst[p];
  }
}

// Range mode (13..15 bits): part `part` of nparts of head h owns the buckets
// [part R, part R + R), R = range_part_buckets(WIDE), and reads all of the
// head's items: every wave counts the items of its contiguous slice that fall
// in the range (one LDS counter row per wave) and the ones below it; a scan
// over (bucket, wave) from the count below gives each wave its base in each
// bucket and the range's offsets; then each wave walks its slice in order
// and places its in-range items (ballot ranks among equal buckets), so the
// sort is stable.  No exchange between the parts.
template <int NBITS, bool WIDE>
__device__ __forceinline__ void range_index_body(int h, int part, int nparts,
                                                 const int32_t* __restrict__ bucket, int P, int64_t n,
                                                 const int32_t* __restrict__ n_valid,
                                                 int32_t* __restrict__ offsets,
                                                 int32_t* __restrict__ perm, int4* lds4) {
  constexpr int nbk = 1 << NBITS;
  constexpr int R = range_part_buckets(WIDE);
  constexpr int RB = NBITS - ilog2_c(R);  // bits of the part index
  static_assert(R * (1 << RB) == nbk && R % kDirectThreads == 0 || R < kDirectThreads, "range split");
  constexpr int BPT = R / kDirectThreads > 0 ? R / kDirectThreads : 1;  // buckets per thread
  using CT = typename std::conditional<WIDE, uint32_t, uint16_t>::type;
  __shared__ int wtot[kDirectWaves];
  __shared__ int wbelow[kDirectWaves];
  int nh = (int)n;
  if (n_valid) {
    const int v = n_valid[h];
    nh = v < 0 ? 0 : (v < nh ? v : nh);
  }
  CT* cnt = reinterpret_cast<CT*>(lds4);  // [kDirectWaves][R]
  uint32_t* cnt32 = reinterpret_cast<uint32_t*>(lds4);
  const uint32_t bmask = (uint32_t)nbk - 1u;
  const uint32_t lo = (uint32_t)part * R;
  const int32_t* ids = bucket + (int64_t)h * n * P;
  int32_t* ph = perm + (int64_t)h * n;
  int32_t* off = offsets + (int64_t)h * (nbk + 1);
  const int wave = threadIdx.x >> 6;
  const int lane = lane_id();
  if (nh == 0) {  // the whole workgroup: every bucket is empty
    for (int B = threadIdx.x; B < R; B += kDirectThreads) off[lo + B] = 0;
    if (part == nparts - 1 && threadIdx.x == 0) off[nbk] = 0;
    return;
  }
  auto inc = [&](int row, uint32_t b) {
    const int i = row * R + (int)b;
    if (WIDE) atomicAdd(&cnt32[i], 1u);
    else atomicAdd(&cnt32[i >> 1], 1u << (16 * (b & 1u)));
  };
  // the wave's slice [wbeg, wend), walked in tiles of kTile ids per lane; a
  // slice of at most kResTiles tiles is loaded once, all tiles at a time, and
  // kept in registers for the scatter pass.  Two tiles keep the kernel within
  // 64 VGPRs: a 16-wave workgroup then still finds room on a CU beside the
  // attention waves of the other stream (at 72 it waits for them)
  const int chunk = (nh + kDirectWaves - 1) / kDirectWaves;
  const int wbeg = wave * chunk < nh ? wave * chunk : nh;
  const int wend = wbeg + chunk < nh ? wbeg + chunk : nh;
  constexpr int kTile = 8;
  constexpr int kResTiles = 2;
  const int last = nh - 1;
  const bool resident = wend - wbeg <= kResTiles * kTile * FASTAR_WAVE;
  uint32_t b[kResTiles][kTile];
  auto load_tile = [&](uint32_t* bt, int t0) {
#pragma unroll
    for (int r = 0; r < kTile; ++r) {
      const int i = t0 + r * FASTAR_WAVE + lane;
      const uint32_t v = index_key(ids, i < last ? i : last, P) & bmask;
      bt[r] = i < wend ? v : 0xFFFFFFFFu;
    }
  };
  if (resident) {
#pragma unroll
    for (int u = 0; u < kResTiles; ++u)
      if (wbeg + u * kTile * FASTAR_WAVE < wend) load_tile(b[u], wbeg + u * kTile * FASTAR_WAVE);
  } else {
    load_tile(b[0], wbeg);
  }
  for (int i = threadIdx.x; i < kDirectWaves * R * (int)sizeof(CT) / 16; i += kDirectThreads)
    lds4[i] = make_int4(0, 0, 0, 0);
  lds_barrier();
  int below = 0;  // this lane's items below the range
  auto count_tile = [&](const uint32_t* bt) {
#pragma unroll
    for (int r = 0; r < kTile; ++r) {
      if (bt[r] == 0xFFFFFFFFu) continue;
      const uint32_t d = bt[r] - lo;
      if (d < (uint32_t)R) inc(wave, d);
      else if (bt[r] < lo) ++below;
    }
  };
  if (resident) {
#pragma unroll
    for (int u = 0; u < kResTiles; ++u)
      if (wbeg + u * kTile * FASTAR_WAVE < wend) count_tile(b[u]);
  } else {
    for (int t0 = wbeg; t0 < wend;) {
      count_tile(b[0]);
      t0 += kTile * FASTAR_WAVE;
      if (t0 >= wend) break;
      load_tile(b[0], t0);
    }
  }
  below = wave_sum_dpp(below);
  if (lane == 0) wbelow[wave] = below;
  lds_barrier();
  // the items below the range, all waves
  int base0 = lane < kDirectWaves ? wbelow[lane] : 0;
  base0 = wave_sum_dpp(base0);
  // exclusive scan over (bucket, wave): thread t owns buckets BPT t .. + BPT
  const int t = threadIdx.x;
  const bool owner = t * BPT < R;
  uint32_t tot[BPT];
#pragma unroll
  for (int e = 0; e < BPT; ++e) {
    tot[e] = 0u;
    if (owner)
      for (int w = 0; w < kDirectWaves; ++w) tot[e] += (uint32_t)cnt[w * R + t * BPT + e];
  }
  uint32_t local = 0u;
#pragma unroll
  for (int e = 0; e < BPT; ++e) local += tot[e];
  const uint32_t incl = wave_incl_scan_dpp(local);
  if (lane == FASTAR_WAVE - 1) wtot[wave] = (int)incl;
  lds_barrier();
  const int wt = lane < kDirectWaves ? wtot[lane] : 0;
  uint32_t run = (uint32_t)base0 + incl - local + (uint32_t)wave_sum_dpp(lane < wave ? wt : 0);
  if (owner) {
#pragma unroll
    for (int e = 0; e < BPT; ++e) {
      off[lo + t * BPT + e] = (int)run;
      // each wave's base within the bucket (replacing the wave's count)
      uint32_t bw = run;
      for (int w = 0; w < kDirectWaves; ++w) {
        const uint32_t c = (uint32_t)cnt[w * R + t * BPT + e];
        cnt[w * R + t * BPT + e] = (CT)bw;
        bw += c;
      }
      run += tot[e];
    }
    if (part == nparts - 1 && t * BPT + BPT == R) off[nbk] = (int)run;
  }
  lds_barrier();
  // stable scatter of the in-range items: each wave walks its slice in order
  auto scatter_tile = [&](const uint32_t* bt, int t0) {
#pragma unroll
    for (int r = 0; r < kTile; ++r) {
      if (t0 + r * FASTAR_WAVE >= wend) break;  // uniform
      const int i = t0 + r * FASTAR_WAVE + lane;
      const uint32_t d = bt[r] - lo;  // past the end: 0xFFFFFFFF - lo, not in range
      const bool inr = d < (uint32_t)R;
      // lanes of this row with the same bucket: in range, and agreeing on the
      // bits of d
      uint64_t peers = ballot64(inr);
      if (peers == 0ull) continue;  // uniform
#pragma unroll
      for (int k = 0; k < NBITS - RB; ++k) {
        const uint32_t bit = (d >> k) & 1u;
        const uint64_t bk = ballot64(bit != 0u);
        peers &= ~(bk ^ (0ull - (uint64_t)bit));
      }
      if (inr) {
        const int rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(peers >> 32),
                                                   __builtin_amdgcn_mbcnt_lo((uint32_t)peers, 0u));
        const int pos = (int)cnt[wave * R + (int)d] + rank;
        ph[pos] = (int32_t)i;
        // the lowest peer (rank 0) advances the counter
        if (rank == 0) cnt[wave * R + (int)d] = (CT)(pos + __popcll(peers));
      }
    }
  };
  if (resident) {
#pragma unroll
    for (int u = 0; u < kResTiles; ++u)
      if (wbeg + u * kTile * FASTAR_WAVE < wend) scatter_tile(b[u], wbeg + u * kTile * FASTAR_WAVE);
  } else {
    for (int t0 = wbeg; t0 < wend; t0 += kTile * FASTAR_WAVE) {
      load_tile(b[0], t0);
      scatter_tile(b[0], t0);
    }
  }
}

}  // namespace fastar
