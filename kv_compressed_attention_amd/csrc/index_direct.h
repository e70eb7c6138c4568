// Stable counting-sort bucket index for one probe, 3..12 bits and at most
// 65535 items per head (see index.hip), as a workgroup-level body, so that
// other launches can run it in workgroups of their own.
#pragma once

#include "common.h"

namespace fastar {

// One probe, 3..12 bits, at most 65535 items: a single stable counting pass.
// Per-wave 16-bit bucket counters (kDirectWaves x 2^b) fit in LDS; one scan
// over (bucket, wave) gives each wave's scatter bases and the offsets.  With
// `stage`, the permutation is assembled in LDS and written out coalesced.
constexpr int kDirectWaves = 16;
constexpr int kDirectMinBits = 3;
constexpr int kDirectMaxBits = 12;
constexpr int64_t kDirectMaxItems = 65535;
// LDS left for the staged permutation next to the counters
constexpr size_t kDirectLds = 152 * 1024;

// LDS bytes the direct index of n items needs, and whether it stages the
// permutation there
inline size_t direct_index_lds(int64_t n, int n_bits, int* stage) {
  const size_t counters = (size_t)kDirectWaves * ((size_t)1 << n_bits) * sizeof(uint16_t);
  *stage = counters + (size_t)n * sizeof(int32_t) <= kDirectLds ? 1 : 0;
  return counters + (*stage ? (size_t)n * sizeof(int32_t) : 0);
}
inline bool direct_index_fits(int64_t n, int n_probes, int n_bits) {
  return n_probes == 1 && n_bits >= kDirectMinBits && n_bits <= kDirectMaxBits && n <= kDirectMaxItems;
}

// The index of head h by one workgroup of kDirectWaves waves.  lds4: the
// dynamic LDS of direct_index_lds bytes.
template <int NBITS>
__device__ __forceinline__ void direct_index_body(int h, const int32_t* __restrict__ bucket, int64_t n,
                                                  const int32_t* __restrict__ n_valid,
                                                  int32_t* __restrict__ offsets,
                                                  int32_t* __restrict__ perm, int stage, int4* lds4) {
  constexpr int nbits = NBITS;
  // lds4: [kDirectWaves][2^nbits] uint16 counters (8 per 128-bit word), then
  // the staged permutation (int32, n entries) when stage is set
  __shared__ int wtot[kDirectWaves];
  constexpr int NT = kDirectWaves * FASTAR_WAVE;
  static_assert((1 << kDirectMaxBits) / 4 <= NT, "at most one 4-bucket group per thread");
  static_assert((1 << kDirectMinBits) >= 4, "whole 4-bucket groups");
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
  // exclusive scan over (bucket, wave): thread t owns buckets 4t .. 4t + 3,
  // one 64-bit word per wave
  const int t = threadIdx.x;
  const int nb4 = nbk >> 2;
  uint2* c64 = reinterpret_cast<uint2*>(lds4);
  uint32_t tot[4] = {0u, 0u, 0u, 0u};
#pragma unroll 8
  for (int w = 0; w < kDirectWaves; ++w) {
    const uint2 cw = t < nb4 ? c64[w * nb4 + t] : make_uint2(0u, 0u);
    tot[0] += cw.x & 0xFFFFu;
    tot[1] += cw.x >> 16;
    tot[2] += cw.y & 0xFFFFu;
    tot[3] += cw.y >> 16;
  }
  const uint32_t local = tot[0] + tot[1] + tot[2] + tot[3];
  const uint32_t incl = wave_incl_scan_dpp(local);
  if (lane == FASTAR_WAVE - 1) wtot[wave] = (int)incl;
  __syncthreads();
  uint32_t run = incl - local;
  for (int w = 0; w < wave; ++w) run += (uint32_t)wtot[w];
  if (t < nb4) {
    uint32_t base[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      base[e] = run;
      run += tot[e];
    }
    // each wave's base within each bucket (replacing the wave's counts)
#pragma unroll 8
    for (int w = 0; w < kDirectWaves; ++w) {
      const uint2 cw = c64[w * nb4 + t];
      c64[w * nb4 + t] = make_uint2(base[0] | (base[1] << 16), base[2] | (base[3] << 16));
      base[0] += cw.x & 0xFFFFu;
      base[1] += cw.x >> 16;
      base[2] += cw.y & 0xFFFFu;
      base[3] += cw.y >> 16;
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

}  // namespace fastar
