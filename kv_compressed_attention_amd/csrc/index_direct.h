// Stable counting-sort bucket index for one probe, 3..12 bits and at most
// 65535 items per head (see index.hip), as a workgroup-level body, so that
// other launches can run it in workgroups of their own.
#pragma once

#include "common.h"

namespace fastar {

// One probe, 3..12 bits, at most 65535 items: a single stable counting pass.
// Per-wave 16-bit bucket counters (one row of 2^b per scattering wave) fit in
// LDS; one scan over (bucket, row) gives each wave's scatter bases and the
// offsets.  A head may be split into parts, one workgroup each: a part
// scatters its own slice of the items and counts the others (those before
// the slice and those after it, per bucket, in two more rows) to place it,
// so the parts need no exchange.  With `stage` (one part), the permutation is
// assembled in LDS and written out coalesced.
constexpr int kDirectWaves = 16;
// waves that scatter a part's slice when a head has several parts (fewer
// counter rows to clear and scan)
constexpr int kDirectPartWaves = 8;
constexpr int kDirectMinBits = 3;
constexpr int kDirectMaxBits = 12;
constexpr int64_t kDirectMaxItems = 65535;
// parts per head: about this many items each, at most kDirectMaxParts
constexpr int64_t kDirectPartItems = 1536;
constexpr int kDirectMaxParts = 8;
// LDS left for the staged permutation next to the counters
constexpr size_t kDirectLds = 152 * 1024;

// The parts (workgroups) per head for n items
inline int direct_index_parts(int64_t n) {
  const int64_t p = (n + kDirectPartItems - 1) / kDirectPartItems;
  return p < 1 ? 1 : (p > kDirectMaxParts ? kDirectMaxParts : (int)p);
}
// counter rows: one per scattering wave, and two more with several parts
__host__ __device__ inline int direct_index_rows(int nparts) {
  return nparts > 1 ? kDirectPartWaves + 2 : kDirectWaves;
}
// LDS bytes the direct index of n items in nparts parts needs, and whether it
// stages the permutation there
inline size_t direct_index_lds(int64_t n, int n_bits, int nparts, int* stage) {
  const size_t counters = (size_t)direct_index_rows(nparts) * ((size_t)1 << n_bits) * sizeof(uint16_t);
  *stage = nparts == 1 && counters + (size_t)n * sizeof(int32_t) <= kDirectLds ? 1 : 0;
  return counters + (*stage ? (size_t)n * sizeof(int32_t) : 0);
}
inline bool direct_index_fits(int64_t n, int n_probes, int n_bits) {
  return n_probes == 1 && n_bits >= kDirectMinBits && n_bits <= kDirectMaxBits && n <= kDirectMaxItems;
}

// Part `part` of nparts of the index of head h, by one workgroup of
// kDirectWaves waves.  lds4: the dynamic LDS of direct_index_lds bytes.
template <int NBITS>
__device__ __forceinline__ void direct_index_body(int h, int part, int nparts,
                                                  const int32_t* __restrict__ bucket, int64_t n,
                                                  const int32_t* __restrict__ n_valid,
                                                  int32_t* __restrict__ offsets,
                                                  int32_t* __restrict__ perm, int stage, int4* lds4) {
  constexpr int nbits = NBITS;
  // lds4: [sw][2^nbits] uint16 counters of the scattering waves (8 per
  // 128-bit word), then with several parts [2][2^nbits] uint16 counts of the
  // items before and after this part's slice, then the staged permutation
  // (int32, n entries) when stage is set
  __shared__ int wtot[kDirectWaves];
  constexpr int NT = kDirectWaves * FASTAR_WAVE;
  static_assert((1 << kDirectMaxBits) / 4 <= NT, "at most one 4-bucket group per thread");
  static_assert((1 << kDirectMinBits) >= 4, "whole 4-bucket groups");
  // item indices fit in 32 bits (at most kDirectMaxItems)
  int nh = (int)n;
  if (n_valid) {
    const int v = n_valid[h];
    nh = v < 0 ? 0 : (v < nh ? v : nh);
  }
  const bool split = nparts > 1;
  const int sw = split ? kDirectPartWaves : kDirectWaves;
  const int rows = direct_index_rows(nparts);
  const int nbk = 1 << nbits;
  const int nb8 = nbk >> 3;
  uint16_t* cnt = reinterpret_cast<uint16_t*>(lds4);
  uint32_t* cnt32 = reinterpret_cast<uint32_t*>(lds4);
  int32_t* pst = reinterpret_cast<int32_t*>(lds4 + rows * nb8);
  const uint32_t bmask = (uint32_t)nbk - 1u;
  const int32_t* ids = bucket + (int64_t)h * n;
  int32_t* ph = perm + (int64_t)h * n;
  int32_t* off = offsets + (int64_t)h * (nbk + 1);
  const int wave = threadIdx.x >> 6;
  const int lane = lane_id();
  if (nh == 0) {  // the whole workgroup: every bucket is empty
    if (part == 0)
      for (int B = threadIdx.x; B <= nbk; B += NT) off[B] = 0;
    return;
  }
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
      const uint32_t v = (uint32_t)ids[i < last ? i : last];
      b[r] = i < wend ? (v & bmask) : 0xFFFFFFFFu;
    }
  };
  auto load_batch = [&](int j0) {
#pragma unroll
    for (int r = 0; r < kBatch; ++r) {
      const int j = j0 + r * NT + (int)threadIdx.x;
      const int i = j < sb ? j : j + (se - sb);
      const uint32_t v = (uint32_t)ids[i < last ? i : last];
      ob[r] = j < nother ? (v & bmask) : 0xFFFFFFFFu;
    }
  };
  // the first loads are in flight while the counters are cleared (the
  // barriers below order LDS only: this workgroup reads no global memory that
  // it writes)
  load_tile(wbeg);
  load_batch(0);
  for (int i = threadIdx.x; i < rows * nb8; i += NT) lds4[i] = make_int4(0, 0, 0, 0);
  lds_barrier();
  // counts (order does not matter): the 16-bit counter in its 32-bit word
  for (int t0 = wbeg;;) {
#pragma unroll
    for (int r = 0; r < kTile; ++r)
      if (b[r] != 0xFFFFFFFFu) atomicAdd(&cnt32[(wrow + (int)b[r]) >> 1], 1u << (16 * (b[r] & 1u)));
    t0 += kTile * FASTAR_WAVE;
    if (t0 >= wend) break;
    load_tile(t0);
  }
  // before the slice into row sw, after it into row sw + 1
  for (int j0 = 0; j0 < nother;) {
#pragma unroll
    for (int r = 0; r < kBatch; ++r) {
      const int j = j0 + r * NT + (int)threadIdx.x;
      if (ob[r] != 0xFFFFFFFFu) {
        const int row = j < sb ? sw : sw + 1;
        atomicAdd(&cnt32[(row * nbk + (int)ob[r]) >> 1], 1u << (16 * (ob[r] & 1u)));
      }
    }
    j0 += kBatch * NT;
    if (j0 >= nother) break;
    load_batch(j0);
  }
  lds_barrier();
  // exclusive scan over (bucket, row): thread t owns buckets 4t .. 4t + 3,
  // one 64-bit word per row
  const int t = threadIdx.x;
  const int nb4 = nbk >> 2;
  uint2* c64 = reinterpret_cast<uint2*>(lds4);
  uint32_t tot[4] = {0u, 0u, 0u, 0u};
#pragma unroll 2
  for (int w = 0; w < rows; ++w) {
    const uint2 cw = t < nb4 ? c64[w * nb4 + t] : make_uint2(0u, 0u);
    tot[0] += cw.x & 0xFFFFu;
    tot[1] += cw.x >> 16;
    tot[2] += cw.y & 0xFFFFu;
    tot[3] += cw.y >> 16;
  }
  const uint32_t local = tot[0] + tot[1] + tot[2] + tot[3];
  const uint32_t incl = wave_incl_scan_dpp(local);
  if (lane == FASTAR_WAVE - 1) wtot[wave] = (int)incl;
  lds_barrier();
  // plus the totals of the waves before (one load per lane, then a sum)
  const int wt = lane < kDirectWaves ? wtot[lane] : 0;
  uint32_t run = incl - local + (uint32_t)wave_sum_dpp(lane < wave ? wt : 0);
  if (t < nb4) {
    uint32_t base[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      base[e] = run;
      run += tot[e];
    }
    // the bucket starts; part 0 writes the offsets
    if (part == 0) {
#pragma unroll
      for (int e = 0; e < 4; ++e) off[4 * t + e] = (int)base[e];
      if (t == nb4 - 1) off[nbk] = (int)run;
    }
    if (split) {
      // this part's items follow those before its slice
      const uint2 pw = c64[sw * nb4 + t];
      base[0] += pw.x & 0xFFFFu;
      base[1] += pw.x >> 16;
      base[2] += pw.y & 0xFFFFu;
      base[3] += pw.y >> 16;
    }
    // each wave's base within each bucket (replacing the wave's counts)
#pragma unroll 8
    for (int w = 0; w < sw; ++w) {
      const uint2 cw = c64[w * nb4 + t];
      c64[w * nb4 + t] = make_uint2(base[0] | (base[1] << 16), base[2] | (base[3] << 16));
      base[0] += cw.x & 0xFFFFu;
      base[1] += cw.x >> 16;
      base[2] += cw.y & 0xFFFFu;
      base[3] += cw.y >> 16;
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
        if (rank == 0) cnt[wrow + (int)bb] = (uint16_t)(pos + __popcll(peers));
      }
    }
  }
  // a staged permutation is written out coalesced
  if (stage) {
    lds_barrier();
    for (int p = threadIdx.x; p < nh; p += NT) ph[p] = pst[p];
  }
}

}  // namespace fastar
