// The merge's per-call arrays (workspace), shared by the TempCache launches
// of both match kinds (tempcache.hip, tempcache_quant.hip).
#pragma once

#include "common.h"

namespace fastar {

struct MergeArgs {
  int H, Tf, cap, F, nbits;
  int64_t kb_stride;  // F * Tf
  // per head, tables t = 0..F sorted by bucket: table 0 holds the cache's
  // last frame (the frontier), table f + 1 new frame f
  int32_t* off;       // [H][F+1][2^b + 1] bucket starts, then the number kept
  int32_t* tok;       // [H][F+1][Tf] tokens, bucket by bucket
  int32_t* tbk;       // [H][F+1][Tf] their buckets
  int32_t* candg;     // [H][Tf] groups of table 0's tokens
  int32_t* link;      // [H][F][Tf] f = 0: frontier group the token extends;
                      //            f > 0: frame f - 1 token it extends; -1: opens a group
  int32_t* ocnt;      // [H][nblk + 1] tokens that open groups, per 64 tokens of
                      // (frame, j) order (nblk = ceil(F Tf / 64) blocks), then
                      // the group count before the call
  int32_t* nextj;     // [H][F][Tf] token of frame f + 1 that extends this one, or -1
  int32_t* prop;      // [H][F][3][Tf] proposals of workgroups whose lists stay global
  int32_t* mrange;    // [H][F][match workgroups][4] key positions [p0, p1), candidates [c0, c1)
};

__host__ __device__ __forceinline__ int64_t off_off(const MergeArgs& a, int h, int t) {
  return ((int64_t)h * (a.F + 1) + t) * ((1 << a.nbits) + 1);
}
__host__ __device__ __forceinline__ int64_t tok_off(const MergeArgs& a, int h, int t) {
  return ((int64_t)h * (a.F + 1) + t) * a.Tf;
}
__host__ __device__ __forceinline__ int64_t frame_off(const MergeArgs& a, int h, int f) {
  return ((int64_t)h * a.F + f) * a.Tf;
}
__host__ __device__ __forceinline__ int ocnt_blocks(const MergeArgs& a) { return (a.F * a.Tf + 63) >> 6; }
}  // namespace fastar
