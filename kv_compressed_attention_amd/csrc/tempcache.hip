// TempCache merge on gfx950 (paperlayer.ai section 5 "TempCache", appendix A
// Lemma 5.1, appendix C representative and threshold ablations).
//
// The candidates of a new key of frame f are the previous frame's tokens in
// its bucket: for f = 0 the representatives of the cache's last frame (the
// frontier), for f > 0 the raw keys of new frame f - 1 (each of which is the
// representative of its group after frame f - 1).  A key only ever competes
// with the keys of its own bucket for a candidate, so matching and the
// one-to-one resolution of all frames are independent per (frame, bucket)
// and run in one launch; only the numbering of new groups is sequential.
// Four launches per call:
//   tc_index    per (table, head): the frontier and each new frame sorted by
//               bucket (counting sort in LDS: bucket offsets, tokens, buckets);
//   tc_match    one workgroup per 64 sorted keys of a frame, rounded to whole
//               buckets: cosines of 16 consecutive keys with the candidates of
//               their buckets as 16 x 16 tiles (MFMA for bf16; pairs of
//               different buckets masked), best candidate per key, proposal if
//               it passes tau; then per candidate the proposer of largest
//               cosine (ties: smaller j) wins and links to it; the other keys
//               open groups and are counted per 64 tokens of (frame, j)
//               order;
//   tc_apply    new groups numbered in (frame, j) order from those counts,
//               then 16 lanes per chain of tokens (a token that opens a group or
//               extends a frontier group, then its links through the frames):
//               float32 value sum in frame order, count, mean (rounded once
//               to the cache dtype), last key, its bucket and ln count, the
//               group of every member and the new frontier;
//   then the bucket index of the representatives.
// Cosines are compared in float32 against a certified error bound; a decision
// inside the bound is redone in float64 (where products of the stored values
// are exact) and counted in the diagnostics.

#include <algorithm>

#include "common.h"
#include "hash_body.h"
#include "kernels.h"
#include "merge_args.h"

namespace fastar {

namespace {

// bound on |fl32(cos) - cos| for d exact products accumulated in float32 in
// any order (dot and both norms), then rsqrt and two multiplies; twice the
// first-order estimate
template <int D>
__device__ __forceinline__ float cos_err32() { return (float)(4 * D + 32) * 0x1p-24f; }
// the same for a dot product accumulated by MFMA, taken (as for the hash) at
// four times the float32 worst case: twice (4 D u + D u + 6 u)
template <typename T, int D>
__device__ __forceinline__ float match_err() {
  return sizeof(T) == 2 ? (float)(10 * D + 32) * 0x1p-24f : cos_err32<D>();
}
template <int D>
__device__ __forceinline__ double cos_err64() { return (double)(4 * D + 32) * 0x1p-53; }

__device__ __forceinline__ float sum16(float v) {
  v += shfl_xor_f(v, 1);
  v += shfl_xor_f(v, 2);
  v += shfl_xor_f(v, 4);
  v += shfl_xor_f(v, 8);
  return v;
}
__device__ __forceinline__ double sum16d(double v) {
  v += __shfl_xor(v, 1, FASTAR_WAVE);
  v += __shfl_xor(v, 2, FASTAR_WAVE);
  v += __shfl_xor(v, 4, FASTAR_WAVE);
  v += __shfl_xor(v, 8, FASTAR_WAVE);
  return v;
}

// EPL = D/16 consecutive elements of a row, as float
template <typename T, int EPL>
struct Chunk;
template <int EPL>
struct Chunk<uint16_t, EPL> {
  static __device__ __forceinline__ void load(const uint16_t* p, float* o) {
    static_assert(EPL == 8 || EPL == 4, "EPL");
    if (EPL == 8) {
      const uint4 u = *reinterpret_cast<const uint4*>(p);
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        o[2 * i] = __uint_as_float(w[i] << 16);
        o[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      }
    } else {
      const uint2 u = *reinterpret_cast<const uint2*>(p);
      const uint32_t w[2] = {u.x, u.y};
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        o[2 * i] = __uint_as_float(w[i] << 16);
        o[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      }
    }
  }
};
template <int EPL>
struct Chunk<float, EPL> {
  static __device__ __forceinline__ void load(const float* p, float* o) {
#pragma unroll
    for (int c = 0; c < EPL / 4; ++c) {
      const float4 u = reinterpret_cast<const float4*>(p)[c];
      o[4 * c] = u.x;
      o[4 * c + 1] = u.y;
      o[4 * c + 2] = u.z;
      o[4 * c + 3] = u.w;
    }
  }
};

// running (best, second best); equal values go to the smaller index, so the
// result does not depend on the order the candidates are visited in.  Empty:
// best = -1 and both values -inf (no finite cosine is below that).
template <typename F>
struct Top2 {
  F c1, c2;
  int best;
  __device__ __forceinline__ void init() {
    c1 = -INFINITY;
    c2 = -INFINITY;
    best = -1;
  }
  // the top two of this and (oc1, oc2, ob), branch-free; an empty side never
  // wins (-1 is the largest index unsigned)
  __device__ __forceinline__ void merge(F oc1, F oc2, int ob) {
    const bool o = ob >= 0 && (oc1 > c1 || (oc1 == c1 && (uint32_t)ob < (uint32_t)best));
    const F lo = o ? c1 : oc1;  // the loser's best
    const F w2 = o ? oc2 : c2;  // the winner's second
    c2 = lo > w2 ? lo : w2;
    c1 = o ? oc1 : c1;
    best = o ? ob : best;
  }
  __device__ __forceinline__ void add(F c, int i) { merge(c, (F)-INFINITY, i); }
};

// keys are matched in tiles of this many (one wave each)
constexpr int kKeyTile = 16;

// The tokens of one table that a thread of a 1024-thread workgroup handles
// (i = threadIdx.x + u * blockDim.x, u < kTabPer): bucket b[u] and group g[u]
// (g < 0: left out).  Loads are unconditional, at an index clamped into the
// table, so that all of them go out before the first wait.
constexpr int kTabPer = 2;  // Tf <= 2048
struct TabTok {
  int b[kTabPer], g[kTabPer];
};
// new frame tokens (all kept), buckets kb[0 .. Tf)
__device__ __forceinline__ TabTok tab_frame(const int32_t* kb, int Tf) {
  TabTok r;
#pragma unroll
  for (int u = 0; u < kTabPer; ++u) {
    const int i = threadIdx.x + u * blockDim.x;
    const int v = kb[i < Tf ? i : Tf - 1];
    r.b[u] = v;
    r.g[u] = i < Tf ? 0 : -1;
  }
  return r;
}
// the frontier: token i belongs to group fr[i] (< 0: none), of bucket rb[g]
__device__ __forceinline__ TabTok tab_frontier(const int32_t* fr, const int32_t* rb, bool empty, int Tf) {
  TabTok r;
#pragma unroll
  for (int u = 0; u < kTabPer; ++u) {
    const int i = threadIdx.x + u * blockDim.x;
    const int g = fr[i < Tf ? i : Tf - 1];
    r.g[u] = empty || i >= Tf ? -1 : g;
  }
#pragma unroll
  for (int u = 0; u < kTabPer; ++u) r.b[u] = rb[r.g[u] >= 0 ? r.g[u] : 0];
  return r;
}

// Exclusive scans of st[0 .. nb) and, if given, st2[0 .. nb) in place (whole
// workgroup, one set of barriers for both); st[nb] = total (st2 likewise);
// copy (if given) gets st's starts too.  st and st2 16-byte aligned.  Ends
// with a barrier.
__device__ void scan_buckets(int nb, int32_t* st, int32_t* copy, int32_t* st2 = nullptr) {
  __shared__ int wtot[2][16];
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int per = (nb + nthr - 1) / nthr;
  const int s0 = tid * per;
  // four buckets per thread exactly: one 16-byte access each way
  const bool quad = nb == 4 * nthr;
  int4 q = make_int4(0, 0, 0, 0), q2 = make_int4(0, 0, 0, 0);
  int local = 0, local2 = 0;
  const int nwv = nthr >> 6;
  if (!quad && nb >= 64 * nwv && nb % (64 * nwv) == 0) {
    const int lane = lane_id(), wave = tid >> 6;
    // each wave scans a contiguous segment, 64 buckets per step (lane l:
    // bucket base + l: no bank conflicts, contiguous stores)
    const int seg = nb / nwv, b0 = wave * seg;
    // four consecutive buckets per lane and step where the segment allows
    const bool wide4 = seg % (4 * FASTAR_WAVE) == 0;
    int sum = 0, sum2 = 0;
    if (wide4) {
      for (int i = 4 * lane; i < seg; i += 4 * FASTAR_WAVE) {
        const int4 v = *reinterpret_cast<const int4*>(st + b0 + i);
        sum += v.x + v.y + v.z + v.w;
        if (st2) {
          const int4 v2 = *reinterpret_cast<const int4*>(st2 + b0 + i);
          sum2 += v2.x + v2.y + v2.z + v2.w;
        }
      }
    } else {
      for (int i = lane; i < seg; i += FASTAR_WAVE) {
        sum += st[b0 + i];
        if (st2) sum2 += st2[b0 + i];
      }
    }
    sum = wave_sum_dpp(sum);
    sum2 = wave_sum_dpp(sum2);
    if (lane == 0) {
      wtot[0][wave] = sum;
      wtot[1][wave] = sum2;
    }
    lds_barrier();
    const int wt = lane < nwv ? wtot[0][lane] : 0, wt2 = lane < nwv ? wtot[1][lane] : 0;
    int carry = wave_sum_dpp(lane < wave ? wt : 0), carry2 = wave_sum_dpp(lane < wave ? wt2 : 0);
    auto scan4 = [&](int32_t* a, int b, int& c, int32_t* cp) {
      const int4 v = *reinterpret_cast<const int4*>(a + b);
      const int l4 = v.x + v.y + v.z + v.w;
      const int inc = (int)wave_incl_scan_dpp((uint32_t)l4);
      const int base = c + inc - l4;
      const int4 o = make_int4(base, base + v.x, base + v.x + v.y, base + v.x + v.y + v.z);
      *reinterpret_cast<int4*>(a + b) = o;
      if (cp) {
        cp[b] = o.x;
        cp[b + 1] = o.y;
        cp[b + 2] = o.z;
        cp[b + 3] = o.w;
      }
      c += __builtin_amdgcn_readlane(inc, FASTAR_WAVE - 1);
    };
    for (int i = 0; wide4 && i < seg; i += 4 * FASTAR_WAVE) {
      scan4(st, b0 + i + 4 * lane, carry, copy);
      if (st2) scan4(st2, b0 + i + 4 * lane, carry2, nullptr);
    }
    for (int i = 0; !wide4 && i < seg; i += FASTAR_WAVE) {
      const int b = b0 + i + lane;
      const int v = st[b];
      const int inc = (int)wave_incl_scan_dpp((uint32_t)v);
      st[b] = carry + inc - v;
      if (copy) copy[b] = carry + inc - v;
      carry += __builtin_amdgcn_readlane(inc, FASTAR_WAVE - 1);
      if (st2) {
        const int v2 = st2[b];
        const int inc2 = (int)wave_incl_scan_dpp((uint32_t)v2);
        st2[b] = carry2 + inc2 - v2;
        carry2 += __builtin_amdgcn_readlane(inc2, FASTAR_WAVE - 1);
      }
    }
    if (wave == nwv - 1 && lane == 0) {
      if (copy) copy[nb] = carry;
      st[nb] = carry;
      if (st2) st2[nb] = carry2;
    }
    lds_barrier();
    return;
  }
  if (quad) {
    q = *reinterpret_cast<const int4*>(st + s0);
    local = q.x + q.y + q.z + q.w;
    if (st2) {
      q2 = *reinterpret_cast<const int4*>(st2 + s0);
      local2 = q2.x + q2.y + q2.z + q2.w;
    }
  } else {
    for (int s = s0; s < s0 + per && s < nb; ++s) {
      local += st[s];
      if (st2) local2 += st2[s];
    }
  }
  const int lane = lane_id(), wave = tid >> 6;
  const int incl = (int)wave_incl_scan_dpp((uint32_t)local);
  const int incl2 = (int)wave_incl_scan_dpp((uint32_t)local2);
  if (lane == FASTAR_WAVE - 1) {
    wtot[0][wave] = incl;
    wtot[1][wave] = incl2;
  }
  lds_barrier();
  // plus the totals of the waves before (one load per lane, then a sum)
  const int nw = nthr >> 6;
  const int wt = lane < nw ? wtot[0][lane] : 0, wt2 = lane < nw ? wtot[1][lane] : 0;
  int run = incl - local + wave_sum_dpp(lane < wave ? wt : 0);
  int run2 = incl2 - local2 + wave_sum_dpp(lane < wave ? wt2 : 0);
  if (quad) {
    const int4 o = make_int4(run, run + q.x, run + q.x + q.y, run + q.x + q.y + q.z);
    *reinterpret_cast<int4*>(st + s0) = o;
    if (copy) {
      copy[s0] = o.x;
      copy[s0 + 1] = o.y;
      copy[s0 + 2] = o.z;
      copy[s0 + 3] = o.w;
    }
    run += local;
    if (st2) {
      *reinterpret_cast<int4*>(st2 + s0) =
          make_int4(run2, run2 + q2.x, run2 + q2.x + q2.y, run2 + q2.x + q2.y + q2.z);
      run2 += local2;
    }
  }
  for (int s = s0; !quad && s < s0 + per && s < nb; ++s) {
    const int c = st[s];
    if (copy) copy[s] = run;
    st[s] = run;
    run += c;
    if (st2) {
      const int c2 = st2[s];
      st2[s] = run2;
      run2 += c2;
    }
  }
  if (tid == nthr - 1) {
    if (copy) copy[nb] = run;
    st[nb] = run;
    if (st2) st2[nb] = run2;
  }
  lds_barrier();
}

// Sorts the tokens of one table (up to 2048, whole workgroup of 1024
// threads) by bucket.  Writes off[0 .. 2^nbits] (bucket starts, then the
// number kept), tok (the kept tokens, bucket by bucket; within a bucket in no
// particular order), tbk (their buckets), if given, a copy of tbk in LDS
// (ltbk) and their groups (candg).  lds holds 2^nbits + 1 int32; after the
// call (and a barrier) lds[b] is the end of bucket b.  With a second table
// tc, its bucket starts go to st (2^nbits + 1 int32 of LDS: st[b] = kept
// tokens of buckets < b, st[2^nbits] = all kept), counted and scanned
// together with the first table's.
__device__ void csr_build(int nbits, const TabTok& tt, int32_t* lds, int32_t* off, int32_t* tok,
                          int32_t* tbk, int32_t* ltbk, int32_t* candg, const TabTok* tc = nullptr,
                          int32_t* st = nullptr) {
  const int nb = 1 << nbits;
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  // (lds and st are 16-byte aligned)
  for (int s = 4 * tid; s < nb; s += 4 * nthr) {
    *reinterpret_cast<int4*>(lds + s) = make_int4(0, 0, 0, 0);
    if (tc) *reinterpret_cast<int4*>(st + s) = make_int4(0, 0, 0, 0);
  }
  if (tid == 0) {
    lds[nb] = 0;
    if (tc) st[nb] = 0;
  }
  lds_barrier();
#pragma unroll
  for (int u = 0; u < kTabPer; ++u) {
    if (tt.g[u] >= 0) atomicAdd(&lds[tt.b[u]], 1);
    if (tc && tc->g[u] >= 0) atomicAdd(&st[tc->b[u]], 1);
  }
  lds_barrier();
  // the bucket starts, to off and as the cursors of the fill below
  scan_buckets(nb, lds, off, tc ? st : nullptr);
#pragma unroll
  for (int u = 0; u < kTabPer; ++u) {
    if (tt.g[u] < 0) continue;
    const int k = atomicAdd(&lds[tt.b[u]], 1);
    tok[k] = tid + u * nthr;
    tbk[k] = tt.b[u];
    if (ltbk) ltbk[k] = tt.b[u];
    if (candg) candg[k] = tt.g[u];
  }
}

// dynamic LDS the index launch may take
constexpr size_t kTcIndexLds = 152 * 1024;
// hashing that rides along with the match launch: tiles per wave, and at most
// this many planes of the match grid
constexpr int kMatchHashTiles = 2;
constexpr int kMatchHashPlanes = 2;

// sorted keys per match workgroup (before rounding to whole buckets)
constexpr int kKeysPerGroup = 64;
__host__ __device__ __forceinline__ int match_groups(int Tf) { return (Tf + kKeysPerGroup - 1) / kKeysPerGroup; }

// Table 0 from the frontier (blockIdx.x == 0) or table f + 1 from new frame f.
// One workgroup per (table, head).  Also clears new frame f's nextj links
// and (table 0) the head's opener counts, next to which it keeps the group
// count before the call.
__global__ __launch_bounds__(1024) void tc_index_kernel(
    const int32_t* __restrict__ frontier, const int32_t* __restrict__ rep_bucket,
    const int32_t* __restrict__ n_groups, const int32_t* __restrict__ kbucket, MergeArgs a) {
  extern __shared__ int4 lds_raw[];
  const int h = blockIdx.y;
  const int t = blockIdx.x;
  int32_t* lds = reinterpret_cast<int32_t*>(lds_raw);
  int32_t* off = a.off + off_off(a, h, t);
  int32_t* tok = a.tok + tok_off(a, h, t);
  int32_t* tbk = a.tbk + tok_off(a, h, t);
  const int nb = 1 << a.nbits;
  const bool empty = n_groups[h] <= 0;
  const int32_t* fr = frontier + (int64_t)h * a.Tf;
  const int32_t* rb = rep_bucket + (int64_t)h * a.cap;
  if (t == 0) {
    const TabTok tt = tab_frontier(fr, rb, empty, a.Tf);
    const int nblk = ocnt_blocks(a);
    int32_t* oc = a.ocnt + (int64_t)h * (nblk + 1);
    for (int i = threadIdx.x; i <= nblk; i += blockDim.x) oc[i] = i < nblk ? 0 : n_groups[h];
    csr_build(a.nbits, tt, lds, off, tok, tbk, nullptr, a.candg + (int64_t)h * a.Tf);
    return;
  }
  const int f = t - 1;
  const int32_t* kb = kbucket + (int64_t)h * a.kb_stride + (int64_t)f * a.Tf;
  // this frame's buckets, and those of table f (the frontier's, or frame
  // f - 1's), whose starts give the match workgroups' candidate ranges
  const TabTok tt = tab_frame(kb, a.Tf);
  for (int i = threadIdx.x; i < a.Tf; i += blockDim.x) a.nextj[frame_off(a, h, f) + i] = -1;
  if (!a.mrange) {  // the match workgroups find their ranges themselves
    csr_build(a.nbits, tt, lds, off, tok, tbk, nullptr, nullptr);
    return;
  }
  const TabTok tc = f == 0 ? tab_frontier(fr, rb, empty, a.Tf) : tab_frame(kb - a.Tf, a.Tf);
  // lds: [2^b + 1] cursors, [2^b + 1] starts of table f, [Tf] buckets of the
  // sorted keys (each array from a 16-byte boundary)
  const int nb1 = (nb + 1 + 3) & ~3;
  int32_t* cst = lds + nb1;
  int32_t* ltbk = cst + nb1;
  csr_build(a.nbits, tt, lds, off, tok, tbk, ltbk, nullptr, &tc, cst);
  lds_barrier();
  // The match workgroups of frame f: key positions rounded to whole buckets,
  // and the candidate range of their buckets.  lds[b] is the end of bucket b.
  const int nkt = lds[nb - 1];
  const int nwg = match_groups(a.Tf);
  for (int wi = threadIdx.x; wi < nwg; wi += blockDim.x) {
    int p0 = 0, p1 = 0, c0 = 0, c1 = 0;
    const int a0 = wi * kKeysPerGroup;
    if (a0 < nkt) {
      const int a1 = min(a0 + kKeysPerGroup, nkt);
      const int b0 = ltbk[a0], b1 = ltbk[a1 - 1];
      const bool cut0 = a0 > 0 && ltbk[a0 - 1] == b0;  // a0 inside a bucket owned before
      const bool cut1 = a1 < nkt && ltbk[a1] == b1;    // a1 inside a bucket owned here
      p0 = cut0 ? lds[b0] : a0;
      p1 = cut1 ? lds[b1] : a1;
      c0 = cst[cut0 ? b0 + 1 : b0];
      c1 = cst[b1 + 1];
    }
    reinterpret_cast<int4*>(a.mrange)[((int64_t)h * a.F + f) * nwg + wi] = make_int4(p0, p1, c0, c1);
  }
}

// 16 x 16 tiles of dot products of keys with candidates.  Loads are issued
// (issue_*) before they are used (finish_keys, dots), so that the key rows
// and a tile of candidate rows are in flight together.  Lane l (col = l & 15,
// g = l >> 4) fetches key col and candidate col of a tile; after finish_keys
// it holds the squared norm of key col in kn, cand_norm gives the squared
// norm of candidate col, and dots the dots of key col with candidates 4g + i
// of the tile in s[i].
template <typename T, int D>
struct TileDot;

template <int D>
struct TileDot<uint16_t, D> {
  static constexpr int NC = D / 32;
  struct Rows {
    uint4 u[NC];  // row l & 15, dims 32c + 8g .. +8
  };
  Rows kr;
  float kn;
  __device__ __forceinline__ static float sumsq(const uint4& u) {
    float s = 0.f;
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lo = __uint_as_float(w[i] << 16);
      const float hi = __uint_as_float(w[i] & 0xFFFF0000u);
      s = fmaf(lo, lo, s);
      s = fmaf(hi, hi, s);
    }
    return s;
  }
  __device__ __forceinline__ static Rows issue(const uint16_t* row) {
    const int g = lane_id() >> 4;
    Rows r;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      r.u[c] = make_uint4(0u, 0u, 0u, 0u);
      if (row) r.u[c] = *reinterpret_cast<const uint4*>(row + 32 * c + 8 * g);
    }
    return r;
  }
  __device__ __forceinline__ static float rownorm(const Rows& r) {
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c) s += sumsq(r.u[c]);
    return sum_xor32(sum_xor16(s));
  }
  // row r of an LDS tile whose row r holds 16-byte piece p at position
  // p ^ (r % (D / 8)) (all zero for r >= n)
  __device__ __forceinline__ static Rows from_lds(const uint16_t* rows, int r, int n) {
    constexpr int kPieces = D / 8;
    const int g = lane_id() >> 4;
    Rows o;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      o.u[c] = make_uint4(0u, 0u, 0u, 0u);
      if (r < n)
        o.u[c] = *reinterpret_cast<const uint4*>(rows + r * D + (((4 * c + g) ^ (r % kPieces)) * 8));
    }
    return o;
  }
  __device__ __forceinline__ void issue_keys(const uint16_t* row) { kr = issue(row); }
  __device__ __forceinline__ void finish_keys() { kn = rownorm(kr); }
  // the squared norm of candidate l & 15 (every lane of it)
  __device__ __forceinline__ static float cand_norm(const Rows& cr) { return rownorm(cr); }
  __device__ __forceinline__ void dots(const Rows& cr, float* s) const {
    // candidates as the A operand: acc[i] = cand (4g + i) . key col
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NC; ++c)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, cr.u[c]),
                                                     __builtin_bit_cast(bf16x8_t, kr.u[c]), acc,
                                                     0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) s[i] = acc[i];
  }
};

template <int D>
struct TileDot<float, D> {
  struct Rows {
    const float* p;  // candidate l & 15's row
  };
  const float* own;  // key l & 15's row
  float kn;
  __device__ __forceinline__ static Rows issue(const float* row) { return Rows{row}; }
  __device__ __forceinline__ void issue_keys(const float* row) { own = row; }
  __device__ __forceinline__ void finish_keys() {
    float n = 0.f;
    if (own)
      for (int d = 0; d < D; ++d) n = fmaf(own[d], own[d], n);
    kn = n;
  }
  __device__ __forceinline__ static float cand_norm(const Rows& cr) {
    float n = 0.f;
    if (cr.p)
      for (int k = 0; k < D; ++k) n = fmaf(cr.p[k], cr.p[k], n);
    return n;
  }
  __device__ __forceinline__ void dots(const Rows& cr, float* s) const {
    const int g = lane_id() >> 4;
    const uint64_t u = (uint64_t)cr.p;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = (uint32_t)__shfl((int)(uint32_t)u, 4 * g + i, FASTAR_WAVE);
      const uint32_t hi = (uint32_t)__shfl((int)(uint32_t)(u >> 32), 4 * g + i, FASTAR_WAVE);
      const float* c = (const float*)(((uint64_t)hi << 32) | lo);
      float d = 0.f;
      if (c && own)
        for (int k = 0; k < D; ++k) d = fmaf(own[k], c[k], d);
      s[i] = d;
    }
  }
};

// t merged with the lane a DPP pattern CTRL pairs this lane with
template <int CTRL>
__device__ __forceinline__ void top2_merge_dpp(Top2<float>& t) {
  const float c1 = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(t.c1), CTRL, 0xF, 0xF, false));
  const float c2 = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(t.c2), CTRL, 0xF, 0xF, false));
  const int b = __builtin_amdgcn_update_dpp(0, t.best, CTRL, 0xF, 0xF, false);
  t.merge(c1, c2, b);
}

// float64 cosine of two rows, the whole wave (lane l takes dims l, l + 64, ..);
// every lane returns it.  Products of the stored values are exact in float64.
// exact: the value is the cosine itself, not an estimate: 0 for a zero row,
// 1 for two bitwise-identical nonzero rows.
struct Cos64 {
  double c;
  bool exact;
};
template <typename T, int D>
__device__ Cos64 wave_cos64(const T* x, const T* y) {
  double s = 0.0, na = 0.0, nb = 0.0;
  bool differ = false;
  for (int d = lane_id(); d < D; d += FASTAR_WAVE) {
    const float uf = Elem<T>::load(x, d), vf = Elem<T>::load(y, d);
    differ = differ || __float_as_uint(uf) != __float_as_uint(vf);
    const double u = (double)uf;
    const double v = (double)vf;
    s += u * v;
    na += u * u;
    nb += v * v;
  }
#pragma unroll
  for (int m = 1; m < FASTAR_WAVE; m <<= 1) {
    s += __shfl_xor(s, m, FASTAR_WAVE);
    na += __shfl_xor(na, m, FASTAR_WAVE);
    nb += __shfl_xor(nb, m, FASTAR_WAVE);
  }
  if (na == 0.0 || nb == 0.0) return Cos64{0.0, true};
  if (ballot64(differ) == 0) return Cos64{1.0, true};
  return Cos64{s / sqrt(na * nb), false};
}

// The same with 16 lanes per pair of rows (the lane's group of 16 takes the
// pair, D/16 elements per lane): four cosines per wave at once.  Every lane
// of the group returns its pair's.
template <typename T, int D>
__device__ __forceinline__ Cos64 group_cos64(const T* x, const T* y) {
  constexpr int EPL = D / 16;
  const int sub = threadIdx.x & 15;
  float xv[EPL], yv[EPL];
  Chunk<T, EPL>::load(x + sub * EPL, xv);
  Chunk<T, EPL>::load(y + sub * EPL, yv);
  double s = 0.0, na = 0.0, nb = 0.0;
  bool differ = false;
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    differ = differ || __float_as_uint(xv[e]) != __float_as_uint(yv[e]);
    const double u = (double)xv[e], v = (double)yv[e];
    s += u * v;
    na += u * u;
    nb += v * v;
  }
  s = sum16d(s);
  na = sum16d(na);
  nb = sum16d(nb);
  const bool dif = ((ballot64(differ) >> (lane_id() & 48)) & 0xFFFFull) != 0ull;
  if (na == 0.0 || nb == 0.0) return Cos64{0.0, true};
  if (!dif) return Cos64{1.0, true};
  return Cos64{s / sqrt(na * nb), false};
}

// What one wave needs to match keys of new frame f.
template <typename T, int D>
struct SegCtx {
  const T* kf;          // frame f keys
  const T* kp;          // frame f - 1 keys (f > 0)
  const T* rk;          // the head's representatives
  int64_t k_st;
  int nk, f;            // keys that step 2 compares; the frame
  float tau, e;
  fastar_diag_t* diag;
  // the wave's float64 decisions and the ones float64 could not certify
  // (wave-uniform), added to diag once at the end: an atomic per event that
  // the wave then waits for stalls it
  mutable uint32_t nfb = 0u, nunres = 0u;
  // candidate row: the frontier group's representative (f == 0), else the
  // frame f - 1 key
  __device__ __forceinline__ const T* cand_row(int, int i, int gr) const {
    return f == 0 ? rk + (int64_t)gr * D : kp + (int64_t)i * k_st;
  }
};

// Turns the float32 best / second best of the reporting lanes' keys (m) into
// proposals p (candidate token, -1: none) and cosines c; a key the error
// bound cannot decide is redone in float64 by the whole wave over its
// candidates, which cand_of(lane, list, groups, n) gives for the reporting
// lane `lane`.
template <typename T, int D, typename CandOf>
__device__ __forceinline__ void decide(const SegCtx<T, D>& x, const Top2<float>& m, bool own,
                                       int jrep, CandOf cand_of, int& p, float& c) {
  const int lane = lane_id();
  bool prop = false, amb = false;
  if (own) {
    if (m.c1 < x.tau - x.e) prop = false;                                  // none reaches tau
    else if (m.c1 >= x.tau + x.e && m.c1 - m.c2 > 2.f * x.e) prop = true;  // clear winner
    else amb = true;
  }
  int best = m.best;
  float c1 = m.c1;
  const double e64 = cos_err64<D>();
  uint64_t ab = ballot64(amb);
  while (ab) {
    const int src = __builtin_ctzll(ab);
    ab &= ab - 1;
    const int js = __shfl(jrep, src, FASTAR_WAVE);
    const int32_t* cl;
    const int32_t* gl;
    int n;
    cand_of(src, cl, gl, n);
    const T* key = x.kf + (int64_t)js * x.k_st;
    // four candidates at a time, one per 16-lane group
    const int grp = lane >> 4;
    auto cand_cos = [&](int k0) {
      const int k = k0 + grp < n ? k0 + grp : n - 1;
      return group_cos64<T, D>(key, x.cand_row(k, cl[k], x.f == 0 ? gl[k] : 0));
    };
    Top2<double> u;
    u.init();
    for (int k0 = 0; k0 < n; k0 += 4) {
      const Cos64 r = cand_cos(k0);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const double cq = __shfl(r.c, 16 * q, FASTAR_WAVE);
        if (k0 + q < n) u.add(cq, cl[k0 + q]);
      }
    }
    // certified: the threshold test (an exact best value decides it exactly)
    // and, with a proposal, the winner (every candidate within the bound of
    // the best has an exact value: equal values go to the smaller index).
    // The exactness of values is only looked at when float64 alone leaves
    // either in doubt.
    bool ex1 = false;
    int near = 1, near_exact = 0;
    const bool thr_doubt = fabs(u.c1 - (double)x.tau) <= e64;
    const bool win_doubt = u.c1 >= (double)x.tau - e64 && u.c1 - u.c2 <= 2.0 * e64;
    if (thr_doubt || win_doubt) {
      near = 0;
      for (int k0 = 0; k0 < n; k0 += 4) {
        const Cos64 r = cand_cos(k0);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const double cq = __shfl(r.c, 16 * q, FASTAR_WAVE);
          const bool xq = __shfl((int)r.exact, 16 * q, FASTAR_WAVE) != 0;
          if (k0 + q < n) {
            if (cl[k0 + q] == u.best) ex1 = xq;
            if (cq >= u.c1 - 2.0 * e64) {
              ++near;
              near_exact += xq ? 1 : 0;
            }
          }
        }
      }
    }
    ++x.nfb;
    const bool thr_sure = ex1 || fabs(u.c1 - (double)x.tau) > e64;
    const bool sure = thr_sure && (u.c1 < (double)x.tau || near <= 1 || near == near_exact);
    if (!sure) ++x.nunres;
    if (lane == src) {
      best = u.best;
      prop = u.c1 >= (double)x.tau;
      c1 = (float)u.c1;
    }
  }
  p = -1;
  c = 0.f;
  if (own) {
    p = prop ? best : -1;
    c = c1;
  }
}

// the lane's key's float32 top two over all 16 x 4 candidate slots: the
// four lanes of a key (l, l ^ 16, l ^ 32, l ^ 48) merged with permlane swaps
__device__ __forceinline__ void reduce_top2(Top2<float>& t) {
#pragma unroll
  for (int step = 0; step < 2; ++step) {
    const auto c1 = step == 0 ? __builtin_amdgcn_permlane16_swap(__float_as_uint(t.c1), __float_as_uint(t.c1), false, false)
                              : __builtin_amdgcn_permlane32_swap(__float_as_uint(t.c1), __float_as_uint(t.c1), false, false);
    const auto c2 = step == 0 ? __builtin_amdgcn_permlane16_swap(__float_as_uint(t.c2), __float_as_uint(t.c2), false, false)
                              : __builtin_amdgcn_permlane32_swap(__float_as_uint(t.c2), __float_as_uint(t.c2), false, false);
    const auto bb = step == 0 ? __builtin_amdgcn_permlane16_swap((uint32_t)t.best, (uint32_t)t.best, false, false)
                              : __builtin_amdgcn_permlane32_swap((uint32_t)t.best, (uint32_t)t.best, false, false);
    // each pair is (this lane's, the partner's) in one order or the other,
    // the same order for all three; merging both halves is exact either way
    Top2<float> u;
    u.c1 = __uint_as_float(c1[0]);
    u.c2 = __uint_as_float(c2[0]);
    u.best = (int)bb[0];
    u.merge(__uint_as_float(c1[1]), __uint_as_float(c2[1]), (int)bb[1]);
    t = u;
  }
}

// Step 1 for keys k0 .. k0 + 15 of a bucket-sorted key list ktok / kbk
// (whole wave; keys past kend are empty).  Their candidates are positions
// [c_lo, c_hi) of the bucket-sorted candidate list ctok / cbk / cg, covering
// the buckets from the first key's to the last key's; a (key, candidate)
// cosine counts only when their buckets agree.  The lists may be LDS copies;
// the float64 re-evaluation reads a key's whole bucket from the candidate
// table itself (gtok / gcg, bucket offsets coff).  The lane with
// l < 16 reports key l: jrep (its token, -1: none), p (the candidate token
// it proposes to, -1: none) and c (the cosine).  Candidates are visited in
// tiles of 16, the next tile's rows loading while the current one is used;
// lane l compares its key l & 15 with candidates 4 (l >> 4) .. + 3 of each.
template <typename T, int D, bool LROWS>
__device__ __forceinline__ void match_tile(const SegCtx<T, D>& x, const int32_t* ktok,
                                           const int32_t* kbk, int k0, int kend,
                                           const int32_t* ctok, const int32_t* cbk,
                                           const int32_t* cg, int c_lo, int c_hi,
                                           const int32_t* gtok, const int32_t* gcg,
                                           const int32_t* coff, TileDot<T, D>& td,
                                           const uint16_t* crow, const float* crn, int& jrep, int& p,
                                           float& c) {
  using TD = TileDot<T, D>;
  const int lane = lane_id();
  const int g = lane >> 4, col = lane & 15;
  const bool kv = k0 + col < kend;
  const int jr = kv ? ktok[k0 + col] : -1;  // this lane's key
  const int rb = kv ? kbk[k0 + col] : -1;   // and its bucket
  jrep = lane < 16 ? jr : -1;
  p = -1;
  c = 0.f;
  if (c_hi <= c_lo) return;
  const bool own = lane < 16 && jr >= 0;
  // per wave: the current tile's candidates (token, bucket, 1 / norm), laid
  // out so that lane l reads its four (4 (l >> 4) ..) in one load each
  __shared__ __attribute__((aligned(16))) int32_t tt_tok[4][16];
  __shared__ __attribute__((aligned(16))) int32_t tt_bk[4][16];
  __shared__ __attribute__((aligned(16))) float tt_rn[4][16];
  const int wv = threadIdx.x >> 6;
  // candidate ids of the first tile (the row this lane fetches); the key
  // rows were issued by the caller.  LROWS: the candidate rows are staged in
  // LDS (crow, one row per candidate of the workgroup's range) and so are
  // their 1 / norms (crn).
  bool cv = c_lo + col < c_hi;
  int ci = cv ? ctok[c_lo + col] : 0;
  int cb = cv ? cbk[c_lo + col] : -2;
  int cgi = (cv && x.f == 0) ? cg[c_lo + col] : 0;
  typename TD::Rows cr;
  if constexpr (LROWS) cr = TD::from_lds(crow, c_lo + col, c_hi);
  else cr = TD::issue(cv ? x.cand_row(0, ci, cgi) : nullptr);
  td.finish_keys();
  const float rk = td.kn > 0.f ? rsqrtf(td.kn) : 0.f;
  Top2<float> t;
  t.init();
  for (int c0 = c_lo; c0 < c_hi; c0 += 16) {
    // next tile's ids, then this tile's dots, then the next tile's rows
    const bool nv = c0 + 16 + col < c_hi;
    const int ni = nv ? ctok[c0 + 16 + col] : 0;
    const int nb = nv ? cbk[c0 + 16 + col] : -2;
    const int ng = (nv && x.f == 0) ? cg[c0 + 16 + col] : 0;
    float rn;
    if constexpr (LROWS) {
      rn = crn[c0 + col];
    } else {
      const float cn = TD::cand_norm(cr);
      rn = cn > 0.f ? rsqrtf(cn) : 0.f;
    }
    if (g == 0) {
      tt_tok[wv][col] = ci;
      tt_bk[wv][col] = cb;  // -2 past the end: no key's bucket
      tt_rn[wv][col] = rn;
    }
    const int4 t4 = *reinterpret_cast<const int4*>(&tt_tok[wv][4 * g]);
    const int4 b4 = *reinterpret_cast<const int4*>(&tt_bk[wv][4 * g]);
    const float4 r4 = *reinterpret_cast<const float4*>(&tt_rn[wv][4 * g]);
    float sd[4];
    td.dots(cr, sd);
    const int ti[4] = {t4.x, t4.y, t4.z, t4.w};
    const int bi[4] = {b4.x, b4.y, b4.z, b4.w};
    const float ri[4] = {r4.x, r4.y, r4.z, r4.w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (bi[i] == rb) t.add(sd[i] * rk * ri[i], ti[i]);
    if (c0 + 16 < c_hi) {
      if constexpr (LROWS) cr = TD::from_lds(crow, c0 + 16 + col, c_hi);
      else cr = TD::issue(nv ? x.cand_row(0, ni, ng) : nullptr);
    }
    cv = nv;
    ci = ni;
    cb = nb;
  }
  reduce_top2(t);
  decide<T, D>(x, t, own, jrep,
               [&](int src, const int32_t*& cl, const int32_t*& gl, int& n) {
                 // the key's own bucket
                 const int b = __shfl(rb, src, FASTAR_WAVE);
                 const int s = coff[b];
                 cl = gtok + s;
                 gl = gcg + s;
                 n = coff[b + 1] - s;
               },
               p, c);
}

// Step 2 for the keys this wave holds (one per lane; p < 0: no proposal):
// does the key win its candidate against every other proposer?  other(q, p2,
// c2, j2) gives key q's proposal (q < x.nk); the lane compares with keys
// qlo .. qhi - 1, which must hold every other proposer of its candidate; self
// is the lane's own position (skipped).  Float32 near-ties are redone in
// float64.  Returns whether it wins.
template <typename T, int D, typename Other>
__device__ __forceinline__ bool resolve_keys(const SegCtx<T, D>& x, int self, int p, float c, int j,
                                             int qlo, int qhi, Other other, const int32_t* fr) {
  const int lane = lane_id();
  bool win = p >= 0, amb = false;
  for (int q2 = qlo; q2 < qhi; ++q2) {
    int p2, j2;
    float c2;
    other(q2, p2, c2, j2);
    if (q2 == self || p2 != p || p < 0) continue;
    if (c2 > c + 2.f * x.e) win = false;
    else if (c2 >= c - 2.f * x.e) amb = true;
  }
  const double e64 = cos_err64<D>();
  uint64_t nb = ballot64(win && amb);
  while (nb) {
    const int src = __builtin_ctzll(nb);
    nb &= nb - 1;
    const int ps = __shfl(p, src, FASTAR_WAVE);
    const int js = __shfl(j, src, FASTAR_WAVE);
    const int qs = __shfl(self, src, FASTAR_WAVE);
    const T* prev = x.f == 0 ? x.rk + (int64_t)fr[ps] * D : x.kp + (int64_t)ps * x.k_st;
    const Cos64 cj = wave_cos64<T, D>(x.kf + (int64_t)js * x.k_st, prev);
    const double dj = cj.c;
    bool w = true, unres = false;
    for (int q2 = 0; q2 < x.nk; ++q2) {
      int p2, j2;
      float c2;
      other(q2, p2, c2, j2);
      if (q2 == qs || p2 != ps) continue;
      const Cos64 cd = wave_cos64<T, D>(x.kf + (int64_t)j2 * x.k_st, prev);
      const double dd = cd.c;
      // two exact values compare exactly (equal ones go to the smaller j)
      if (fabs(dd - dj) <= 2.0 * e64 && !(cd.exact && cj.exact)) unres = true;
      if (dd > dj || (dd == dj && j2 < js)) w = false;
    }
    ++x.nfb;
    if (unres) ++x.nunres;
    if (lane == src) win = w;
  }
  return win;
}

// keys and candidates a match workgroup copies to LDS (larger ranges are read
// from the tables directly)
constexpr int kStageKeys = 256;
constexpr int kStageCands = 512;

// number of the first n entries of the ascending list v (LDS) that are < b
// (below) or <= b (!below); whole wave
__device__ __forceinline__ int count_until(const int32_t* v, int n, int b, bool below) {
  int cnt = 0;
  for (int i0 = 0; i0 < n; i0 += FASTAR_WAVE) {
    const int i = i0 + lane_id();
    const bool in = i < n && (below ? v[i] < b : v[i] <= b);
    cnt += __popcll(ballot64(in));
  }
  return cnt;
}

// candidate rows a bf16 workgroup stages in LDS
constexpr int kRowCands = 96;

// LDS int32 words of a match workgroup: proposals and lists, then (bf16)
// the staged candidate rows and their 1 / norms
template <typename T, int D>
constexpr size_t match_lds_words() {
  return 3 * kStageKeys + 2 * kStageKeys + 3 * kStageCands +
         (sizeof(T) == 2 ? (size_t)kRowCands * D / 2 + kRowCands : 0);
}

// One workgroup per kKeysPerGroup positions of frame f's bucket-sorted keys,
// rounded to whole buckets: a workgroup owns the buckets whose first key lies
// in its positions.  MODE 0: the lists and the proposals stay in global
// memory (very large buckets); 1: the workgroup copies its keys' ids and
// buckets and the candidate ids, buckets and groups of its bucket range to
// LDS, and keeps the proposals there; 2 (bf16): also the candidate rows,
// fetched once by the whole workgroup while each wave's first key rows load.
// Then its waves take the tiles of 16 consecutive keys (step 1, each key's
// best candidate and proposal) and, after one barrier, step 2 over all of
// its keys: every candidate keeps its best proposer (ties: smaller j), which
// links to it; the other keys open groups.  A candidate's proposers all
// share its bucket, so they are all in the workgroup.
template <typename T, int D, int MODE>
__device__ __forceinline__ void match_group(const SegCtx<T, D>& x, const MergeArgs& a, int h,
                                            int p0, int p1, int c0, int c1,
                                            const int32_t* __restrict__ frontier, int32_t* lds) {
  constexpr bool STAGED = MODE >= 1;
  const int f = x.f;
  const int lane = lane_id();
  const int col = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int32_t* koff = a.off + off_off(a, h, f + 1);
  const int32_t* gktok = a.tok + tok_off(a, h, f + 1);
  const int32_t* gkbk = a.tbk + tok_off(a, h, f + 1);
  const int32_t* coff = a.off + off_off(a, h, f);
  const int32_t* gctok = a.tok + tok_off(a, h, f);
  const int32_t* gcbk = a.tbk + tok_off(a, h, f);
  const int32_t* gcg = a.candg + (int64_t)h * a.Tf;
  const int nk = p1 - p0;
  const int nc = c1 - c0;
  // proposals of the keys by position: LDS, or the workspace's frame slice
  int32_t* const pbase = STAGED ? lds : a.prop + frame_off(a, h, f) * 3 + p0;
  const int pst = STAGED ? kStageKeys : a.Tf;
  int32_t* lp = pbase;
  float* lc = reinterpret_cast<float*>(pbase + pst);
  int32_t* lj = pbase + 2 * pst;
  // the key and candidate lists, rebased to the workgroup's ranges
  int32_t* sk = lds + 3 * kStageKeys;      // [2][kStageKeys] tokens, buckets
  int32_t* sc = sk + 2 * kStageKeys;       // [3][kStageCands] tokens, buckets, groups
  uint16_t* crow = reinterpret_cast<uint16_t*>(sc + 3 * kStageCands);  // [kRowCands][D]
  float* crn = reinterpret_cast<float*>(crow + kRowCands * D);          // [kRowCands]
  const int32_t* ktok = STAGED ? sk : gktok + p0;
  const int32_t* kbk = STAGED ? sk + kStageKeys : gkbk + p0;
  const int32_t* ctok = STAGED ? sc : gctok + c0;
  const int32_t* cbk = STAGED ? sc + kStageCands : gcbk + c0;
  const int32_t* cg = STAGED ? sc + 2 * kStageCands : gcg + c0;
  if (STAGED) {
    for (int i = threadIdx.x; i < nk; i += blockDim.x) {
      sk[i] = gktok[p0 + i];
      sk[kStageKeys + i] = gkbk[p0 + i];
    }
    for (int i = threadIdx.x; i < nc; i += blockDim.x) {
      sc[i] = gctok[c0 + i];
      sc[kStageCands + i] = gcbk[c0 + i];
      if (f == 0) sc[2 * kStageCands + i] = gcg[c0 + i];
    }
    __syncthreads();
  }
  // the key rows of this wave's first tile, in flight with the candidate rows
  TileDot<T, D> td;
  auto issue_tile_keys = [&](int k0) {
    const int jr = k0 + col < nk ? ktok[k0 + col] : -1;
    td.issue_keys(jr >= 0 ? x.kf + (int64_t)jr * x.k_st : nullptr);
  };
  if (wave * kKeyTile < nk) issue_tile_keys(wave * kKeyTile);
  if constexpr (MODE == 2) {
    // candidate row r: piece p at position p ^ (r % (D / 8)), so that the 16
    // lanes reading one piece of 16 rows hit different banks
    constexpr int kPieces = D / 8;
    constexpr int kDmaRows = 64 / kPieces;
    for (int i0 = wave * kDmaRows; i0 < nc; i0 += 4 * kDmaRows) {
      const int r = i0 + lane / kPieces;
      const int rr = r < nc ? r : nc - 1;  // past the end: a real row, never read
      const T* src = x.cand_row(0, ctok[rr], f == 0 ? cg[rr] : 0);
      __builtin_amdgcn_global_load_lds(
          (const void*)(src + (((lane % kPieces) ^ (r % kPieces)) * 8)),
          (__attribute__((address_space(3))) void*)(crow + i0 * D), 16, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
    // each candidate's 1 / norm, once for the workgroup (16 rows per wave at
    // a time, exactly as a tile would compute them)
    for (int r0 = wave * 16; r0 < nc; r0 += 64) {
      const float cn = TileDot<T, D>::cand_norm(TileDot<T, D>::from_lds(crow, r0 + col, nc));
      if (lane < 16 && r0 + col < nc) crn[r0 + col] = cn > 0.f ? rsqrtf(cn) : 0.f;
    }
    lds_barrier();  // (the first key rows stay in flight)
  }
  for (int k0 = wave * kKeyTile; k0 < nk; k0 += 4 * kKeyTile) {
    if (k0 != wave * kKeyTile) issue_tile_keys(k0);
    const int klast = min(k0 + kKeyTile, nk) - 1;
    int c_lo, c_hi;
    if (STAGED) {
      c_lo = count_until(cbk, nc, kbk[k0], true);
      c_hi = count_until(cbk, nc, kbk[klast], false);
    } else {
      c_lo = coff[kbk[k0]] - c0;
      c_hi = coff[kbk[klast] + 1] - c0;
    }
    int jrep, p;
    float c;
    match_tile<T, D, MODE == 2>(x, ktok, kbk, k0, nk, ctok, cbk, cg, c_lo, c_hi, gctok, gcg, coff,
                                td, crow, crn, jrep, p, c);
    if (lane < 16 && jrep >= 0) {
      const int q = k0 + lane;
      lp[q] = p;
      lc[q] = c;
      lj[q] = jrep;
    }
  }
  __syncthreads();
  const int64_t fo = frame_off(a, h, f);
  const int32_t* fr = frontier + (int64_t)h * a.Tf;
  for (int q0 = wave * FASTAR_WAVE; q0 < nk; q0 += 4 * FASTAR_WAVE) {
    const int q = q0 + lane;
    const bool v = q < nk;
    const int pj = v ? lp[q] : -1;
    const float cj = v ? lc[q] : 0.f;
    const int j = v ? lj[q] : -1;
    // a candidate's proposers all have its bucket: the key's own bucket is
    // the only range to compare with
    int qlo = 0, qhi = 0;
    if (STAGED && nk <= FASTAR_WAVE) {
      // the bucket runs of the (at most 64) keys, from their starts
      const int bq = v ? kbk[q] : -1;
      const bool start = v && (q == 0 || kbk[q - 1] != bq);
      // positions >= nk end a run
      const uint64_t starts = ballot64(start) | (nk >= FASTAR_WAVE ? 0ull : (~0ull << nk));
      const uint64_t below = starts & (lane == 63 ? ~0ull : ((2ull << lane) - 1));
      qlo = 63 - __builtin_clzll(below);
      const uint64_t above = starts & ~((2ull << lane) - 1);
      qhi = above ? __builtin_ctzll(above) : FASTAR_WAVE;
    } else if (v && pj >= 0) {
      const int b = kbk[q];
      qlo = max(koff[b], p0) - p0;
      qhi = min(koff[b + 1], p1) - p0;
    }
    const bool win = resolve_keys<T, D>(
        x, q, pj, cj, j, qlo, qhi,
        [&](int q2, int& p2, float& c2, int& j2) {
          p2 = lp[q2];
          c2 = lc[q2];
          j2 = lj[q2];
        },
        fr);
    if (v) {
      int lk = -1;
      if (win) {
        lk = f == 0 ? fr[pj] : pj;
        if (f > 0) a.nextj[frame_off(a, h, f - 1) + pj] = j;
      }
      a.link[fo + j] = lk;
      if (lk < 0) atomicAdd(&a.ocnt[(int64_t)h * (ocnt_blocks(a) + 1) + ((f * a.Tf + j) >> 6)], 1);
    }
  }
}

// The workgroups of the planes past the frames (blockIdx.z >= F, dispatched
// last; bf16 only) hash the jobs qh instead: flat index ((z - F) * gridDim.y
// + y) * gridDim.x + x < qblocks is hashing block that index (jobs of one
// or two probes).
template <typename T, int D>
__global__ __launch_bounds__(256, 4) void tc_match_kernel(
    const T* __restrict__ rep_k, const T* __restrict__ knew, int64_t k_sh, int64_t k_st,
    const int32_t* __restrict__ frontier, float tau, MergeArgs a,
    fastar_diag_t* __restrict__ diag, HashJobs qh, const uint16_t* __restrict__ qplanes, int qnb,
    int qblocks) {
  extern __shared__ int32_t lds[];  // match_lds_words<T, D>()
  const int h = blockIdx.y;
  const int f = blockIdx.z;
  if (f >= a.F) {
    if constexpr (sizeof(T) == 2) {
      static_assert(hash_bf16_lds<D>() <= match_lds_words<T, D>() * sizeof(int32_t), "hashing fits the LDS");
      const int qb = (int)(((blockIdx.z - a.F) * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x);
      if (qb < qblocks)  // (jobs of at most two probes)
        hash_bf16_body<D, 2>(qh, qplanes, qnb, diag, qb, qblocks, reinterpret_cast<char*>(lds));
    }
    return;  // the whole workgroup
  }
  // the owned key positions [p0, p1) and the candidate range [c0, c1) of
  // their buckets (it may also hold candidates of buckets without keys),
  // worked out by the index launch, or else here
  int p0, p1, c0, c1;
  if (a.mrange) {
    const int4 r = reinterpret_cast<const int4*>(a.mrange)[((int64_t)h * a.F + f) * match_groups(a.Tf) + blockIdx.x];
    p0 = r.x, p1 = r.y, c0 = r.z, c1 = r.w;
  } else {
    const int nb = 1 << a.nbits;
    const int32_t* koff = a.off + off_off(a, h, f + 1);
    const int32_t* kbk = a.tbk + tok_off(a, h, f + 1);
    const int32_t* coff = a.off + off_off(a, h, f);
    const int nkt = koff[nb];
    const int a0 = blockIdx.x * kKeysPerGroup;
    if (a0 >= nkt) return;
    const int a1 = min(a0 + kKeysPerGroup, nkt);
    const int b0 = kbk[a0], b1 = kbk[a1 - 1];
    const bool cut0 = a0 > 0 && kbk[a0 - 1] == b0;  // a0 inside a bucket owned before
    const bool cut1 = a1 < nkt && kbk[a1] == b1;    // a1 inside a bucket owned here
    p0 = cut0 ? koff[b0 + 1] : a0;
    p1 = cut1 ? koff[b1 + 1] : a1;
    c0 = coff[cut0 ? b0 + 1 : b0];
    c1 = coff[b1 + 1];
  }
  if (p0 >= p1) return;  // the whole workgroup: no barrier is reached
  SegCtx<T, D> x;
  x.kf = knew + (int64_t)h * k_sh + (int64_t)f * a.Tf * k_st;
  x.kp = f > 0 ? x.kf - (int64_t)a.Tf * k_st : x.kf;
  x.rk = rep_k + (int64_t)h * a.cap * D;
  x.k_st = k_st;
  x.f = f;
  x.tau = tau;
  x.e = match_err<T, D>();
  x.diag = diag;
  x.nk = p1 - p0;
  if (sizeof(T) == 2 && p1 - p0 <= kStageKeys && c1 - c0 <= kRowCands) {
    if constexpr (sizeof(T) == 2) match_group<T, D, 2>(x, a, h, p0, p1, c0, c1, frontier, lds);
  } else if (p1 - p0 <= kStageKeys && c1 - c0 <= kStageCands)
    match_group<T, D, 1>(x, a, h, p0, p1, c0, c1, frontier, lds);
  else
    match_group<T, D, 0>(x, a, h, p0, p1, c0, c1, frontier, lds);
  if (diag && lane_id() == 0) {
    if (x.nfb) atomicAdd(&diag->merge_fallbacks, x.nfb);
    if (x.nunres) atomicAdd(&diag->unresolved, x.nunres);
  }
}

// The float64 quotient s / n rounded once to the storage dtype T (to nearest,
// ties to even).  q = fl(s / n) is on the same side of every rounding
// midpoint of T as s / n unless q is itself a midpoint; then the sign of
// s - n q, exact from one fma, tells which side s / n lies on.
template <typename T>
__device__ __forceinline__ float mean_round(double s, int n) {
  constexpr int kDrop = sizeof(T) == 2 ? 45 : 29;  // float64 fraction bits T lacks
  const double q = s / (double)n;
  const uint64_t b = (uint64_t)__double_as_longlong(q);
  const uint64_t low = b & ((1ull << kDrop) - 1), base = b - low;
  const uint64_t half = 1ull << (kDrop - 1);
  bool away;  // round the magnitude up
  if (low != half) {
    away = low > half;
  } else {
    const double r = fma(-(double)n, q, s);
    away = r == 0.0 ? ((base >> kDrop) & 1) != 0 : ((r > 0.0) == (q > 0.0));
  }
  return (float)__longlong_as_double((long long)(base + (away ? (1ull << kDrop) : 0ull)));
}

// A mean- or medoid-key group's representative state, held by the 16 lanes
// of its token (D/16 elements each): the group's float64 key sum and the
// current representative.  Adding a key to the sum is checked with an exact
// two-sum; a rounded addition is counted as unresolved.  Mean: the sum over
// the count, rounded once (mean_round).  Medoid: of the previous
// representative r and the new key k, the one of larger cosine with the sum
// S; both cosines are evaluated in float64 with a bound (products and sums of
// D terms: (D + 2) u sum|x_i S_i| on the dot, (D + 8) u |dot| for the norm
// and the square root, doubled); a difference inside the bound keeps r if the
// two are an exact tie (identical keys, or both cosines exactly computed) and
// otherwise takes the float64 answer and counts as unresolved.
template <typename T, int D, int REP>
struct RepState {
  static constexpr int EPL = D / 16;
  double ks[EPL];
  float rk[EPL];
  bool inexact = false;
  int unres = 0;

  __device__ __forceinline__ void open(const float* k) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      ks[e] = (double)k[e];
      rk[e] = k[e];
    }
  }
  __device__ __forceinline__ void load(const T* rep, const double* sum) {
    Chunk<T, EPL>::load(rep, rk);
#pragma unroll
    for (int e = 0; e < EPL; e += 2) {
      const double2 u = *reinterpret_cast<const double2*>(sum + e);
      ks[e] = u.x;
      ks[e + 1] = u.y;
    }
  }
  __device__ __forceinline__ void join(const float* k, int) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const double x = (double)k[e];
      const double t = ks[e] + x;
      const double bb = t - ks[e];
      const double err = (ks[e] - (t - bb)) + (x - bb);
      inexact = inexact || err != 0.0;
      ks[e] = t;
    }
    if (REP != FASTAR_REP_MEDOID) return;
    double dk = 0.0, dr = 0.0, nk = 0.0, nr = 0.0, ak = 0.0, ar = 0.0;
    bool differ = false;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const double x = (double)k[e], r = (double)rk[e], sv = ks[e];
      dk = fma(x, sv, dk);
      dr = fma(r, sv, dr);
      nk = fma(x, x, nk);
      nr = fma(r, r, nr);
      ak += fabs(x * sv);
      ar += fabs(r * sv);
      differ = differ || __float_as_uint(k[e]) != __float_as_uint(rk[e]);
    }
    dk = sum16d(dk);
    dr = sum16d(dr);
    nk = sum16d(nk);
    nr = sum16d(nr);
    ak = sum16d(ak);
    ar = sum16d(ar);
    constexpr double u = 0x1p-53;
    const double sk = sqrt(nk), sr = sqrt(nr);
    const double ck = nk > 0.0 ? dk / sk : 0.0, cr = nr > 0.0 ? dr / sr : 0.0;
    const double ek = nk > 0.0 ? 2.0 * ((D + 2) * u * ak + (D + 8) * u * fabs(dk)) / sk : 0.0;
    const double er = nr > 0.0 ? 2.0 * ((D + 2) * u * ar + (D + 8) * u * fabs(dr)) / sr : 0.0;
    const double diff = ck - cr, bound = ek + er;
    bool take;
    if (diff > bound) {
      take = true;
    } else if (-diff > bound) {
      take = false;
    } else {
      const int lane = lane_id();
      const bool same = ((ballot64(differ) >> (lane & 48)) & 0xFFFFull) == 0;
      if (same || (bound == 0.0 && diff == 0.0)) {
        take = false;  // a tie keeps the previous representative
      } else {
        take = diff > 0.0;
        ++unres;
      }
    }
    if (take) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) rk[e] = k[e];
    }
  }
  __device__ __forceinline__ void store(T* rep, double* sum, int n, fastar_diag_t* diag) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const float r = REP == FASTAR_REP_MEAN ? mean_round<T>(ks[e], n) : rk[e];
      Elem<T>::store(rep, e, r);  // r is a value of T: stored exactly
    }
#pragma unroll
    for (int e = 0; e < EPL; e += 2) *reinterpret_cast<double2*>(sum + e) = make_double2(ks[e], ks[e + 1]);
    const int lane = lane_id();
    const bool any_inexact = ((ballot64(inexact) >> (lane & 48)) & 0xFFFFull) != 0;
    const int total = unres + (any_inexact ? 1 : 0);
    if ((lane & 15) == 0 && total && diag) atomicAdd(&diag->unresolved, (unsigned)total);
  }
};

// Group rows, 16 lanes per chain (D/16 elements each).  A token that opens a
// group gets the group count before the call plus the number of tokens
// before it in (frame, j) order that open groups (the counts of the 64-token
// blocks before its own, then a ballot over its block's links); ids from
// the capacity on are dropped (-1).  A chain starts at a
// token that opens a group, or at a frame-0 token that extends a frontier
// group; it follows nextj through the later frames.  Value sums are
// accumulated frame by frame in float32, exactly as merging the frames one at
// a time would; the representative is the chain's last key (REP =
// FASTAR_REP_LAST), or is updated at every member from the group's float64
// key sum (RepState).  Every member's group goes to group_of_new, last-frame
// members' to the frontier.
template <typename T, int D, int REP>
__device__ __forceinline__ void tc_apply_body(
    T* __restrict__ rep_k, T* __restrict__ v_mean, float* __restrict__ v_sum,
    int32_t* __restrict__ count, float* __restrict__ log_count, int32_t* __restrict__ rep_bucket,
    int32_t* __restrict__ n_groups, int32_t* __restrict__ frontier, int32_t* __restrict__ group_of_new,
    const T* __restrict__ knew, int64_t k_sh, int64_t k_st, const T* __restrict__ vnew,
    int64_t v_sh, int64_t v_st, const int32_t* __restrict__ kbucket, MergeArgs a,
    int32_t* __restrict__ status, fastar_diag_t* __restrict__ diag, double* __restrict__ k_sum) {
  constexpr int EPL = D / 16;
  const int h = blockIdx.y;
  const int64_t idx = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  const int total = a.F * a.Tf;
  // the workgroup's 16 tokens lie in one 64-token block; with all lanes
  // present: openers in the blocks before it and in it, up to each token
  const int nblk = ocnt_blocks(a);
  const int32_t* oc = a.ocnt + (int64_t)h * (nblk + 1);
  const int blk = (int)((blockIdx.x * 16) >> 6);
  const int lane = lane_id();
  const int ng0 = oc[nblk];
  int before = 0;
  for (int i = lane; i < blk; i += FASTAR_WAVE) before += oc[i];
  const int bpos = blk * 64 + lane;
  const int lk_b = bpos < total ? a.link[frame_off(a, h, 0) + bpos] : 0;
  const uint64_t openers = ballot64(bpos < total && lk_b < 0);
  // this lane group's token's link, from the block's (every lane is here)
  const int lk = __shfl(lk_b, (int)(((int64_t)blockIdx.x * 16 + (threadIdx.x >> 4)) & 63), FASTAR_WAVE);
  before = wave_sum_dpp(before);
  if (blockIdx.x == 0 && threadIdx.x < FASTAR_WAVE) {
    // the new group count
    int all = 0;
    for (int i = lane; i < nblk; i += FASTAR_WAVE) all += oc[i];
    all = wave_sum_dpp(all);
    if (lane == 0) {
      const int64_t ng = (int64_t)ng0 + all;
      n_groups[h] = ng < a.cap ? (int32_t)ng : a.cap;
    }
  }
  if (idx >= total) return;
  int f = (int)(idx / a.Tf);
  int j = (int)(idx - (int64_t)f * a.Tf);
  if (lk >= 0 && f > 0) return;  // continuation of a chain that starts earlier
  const T* kh = knew + (int64_t)h * k_sh + sub * EPL;
  const T* vh = vnew + (int64_t)h * v_sh + sub * EPL;
  const int32_t* kbh = kbucket + (int64_t)h * a.kb_stride;
  // everything the chain's first token needs, in flight together: its
  // successor, its value and key rows and its bucket
  // meaningful when lk < 0
  const int64_t gd64 = (int64_t)ng0 + before +
                       __popcll(openers & ((1ull << (int)(idx - (int64_t)blk * 64)) - 1ull));
  const int gd = gd64 < a.cap ? (int32_t)gd64 : -1;
  int nx = f + 1 < a.F ? a.nextj[frame_off(a, h, f) + j] : -1;
  float vv[EPL], kk[EPL];
  Chunk<T, EPL>::load(vh + ((int64_t)f * a.Tf + j) * v_st, vv);
  Chunk<T, EPL>::load(kh + ((int64_t)f * a.Tf + j) * k_st, kk);
  int kb = kbh[(int64_t)f * a.Tf + j];
  const int g = lk < 0 ? gd : lk;
  auto member = [&](int ff, int jj) {
    if (sub != 0) return;
    if (group_of_new) group_of_new[(int64_t)h * a.kb_stride + (int64_t)ff * a.Tf + jj] = g;
    if (ff == a.F - 1) frontier[(int64_t)h * a.Tf + jj] = g;
    if (g < 0) {
      // the cache's status word (benign race: every writer stores the same bit)
      *status = FASTAR_CACHE_OVERFLOW;
      if (diag) atomicAdd(&diag->capacity_overflow, 1u);
    }
  };
  member(f, j);
  if (g < 0) {
    // no room: the whole chain is left out
    while (nx >= 0) {
      ++f;
      j = nx;
      member(f, j);
      nx = f + 1 < a.F ? a.nextj[frame_off(a, h, f) + j] : -1;
    }
    return;
  }
  const int64_t gi = (int64_t)h * a.cap + g;
  float sum[EPL];
  int cnt;
  RepState<T, D, REP> rs;
  if (lk < 0) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) sum[e] = vv[e];
    cnt = 1;
    if (REP != FASTAR_REP_LAST) rs.open(kk);
  } else {
    const float* vs = v_sum + gi * D + sub * EPL;
#pragma unroll
    for (int e = 0; e < EPL; ++e) sum[e] = vs[e] + vv[e];
    cnt = count[gi] + 1;
    if (REP != FASTAR_REP_LAST) {
      rs.load(rep_k + gi * D + sub * EPL, k_sum + gi * D + sub * EPL);
      rs.join(kk, cnt);
    }
  }
  // the successors: each hop loads the member's rows, bucket and successor at once
  while (nx >= 0) {
    ++f;
    j = nx;
    nx = f + 1 < a.F ? a.nextj[frame_off(a, h, f) + j] : -1;
    Chunk<T, EPL>::load(vh + ((int64_t)f * a.Tf + j) * v_st, vv);
    Chunk<T, EPL>::load(kh + ((int64_t)f * a.Tf + j) * k_st, kk);
    kb = kbh[(int64_t)f * a.Tf + j];
    member(f, j);
#pragma unroll
    for (int e = 0; e < EPL; ++e) sum[e] += vv[e];
    ++cnt;
    if (REP != FASTAR_REP_LAST) rs.join(kk, cnt);
  }
  T* rkr = rep_k + gi * D + sub * EPL;
  T* vmr = v_mean + gi * D + sub * EPL;
  float* vsr = v_sum + gi * D + sub * EPL;
  const float fc = (float)cnt;
  if (REP != FASTAR_REP_LAST) rs.store(rkr, k_sum + gi * D + sub * EPL, cnt, diag);
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    vsr[e] = sum[e];
    // the last key, exactly (stored values round-trip)
    if (REP == FASTAR_REP_LAST) Elem<T>::store(rkr, e, kk[e]);
    if (cnt == 1) Elem<T>::store(vmr, e, sum[e]);  // exact copy of the value
    else Elem<T>::store(vmr, e, sum[e] / fc);
  }
  if (sub == 0) {
    count[gi] = cnt;
    log_count[gi] = logf(fc);
    rep_bucket[gi] = kb;
  }
}

template <typename T, int D, int REP>
__global__ __launch_bounds__(256) void tc_apply_kernel(
    T* __restrict__ rep_k, T* __restrict__ v_mean, float* __restrict__ v_sum,
    int32_t* __restrict__ count, float* __restrict__ log_count, int32_t* __restrict__ rep_bucket,
    int32_t* __restrict__ n_groups, int32_t* __restrict__ frontier, int32_t* __restrict__ group_of_new,
    const T* __restrict__ knew, int64_t k_sh, int64_t k_st, const T* __restrict__ vnew,
    int64_t v_sh, int64_t v_st, const int32_t* __restrict__ kbucket, MergeArgs a,
    int32_t* __restrict__ status, fastar_diag_t* __restrict__ diag, double* __restrict__ k_sum) {
  tc_apply_body<T, D, REP>(rep_k, v_mean, v_sum, count, log_count, rep_bucket, n_groups, frontier, group_of_new,
                           knew, k_sh, k_st, vnew, v_sh, v_st, kbucket, a, status, diag, k_sum);
}

// the group updates of a merge, for the representative kind rep
template <typename T, int D>
void apply_launch(const fastar_cache_t& c, const fastar_tensor_t& kn, const fastar_tensor_t& vn,
                  const int32_t* kb, const MergeArgs& a, int32_t* group_of_new, int rep,
                  fastar_diag_t* diag, hipStream_t s) {
  auto kern = rep == FASTAR_REP_MEAN     ? tc_apply_kernel<T, D, FASTAR_REP_MEAN>
              : rep == FASTAR_REP_MEDOID ? tc_apply_kernel<T, D, FASTAR_REP_MEDOID>
                                         : tc_apply_kernel<T, D, FASTAR_REP_LAST>;
  hipLaunchKernelGGL(kern, dim3((unsigned)(((int64_t)a.F * a.Tf + 15) / 16), (unsigned)a.H), dim3(256), 0, s,
                     (T*)c.rep_k, (T*)c.v_mean, c.v_sum, c.count, c.log_count, c.rep_bucket, c.n_groups,
                     c.frontier, group_of_new, (const T*)kn.data, kn.stride_head, kn.stride_token,
                     (const T*)vn.data, vn.stride_head, vn.stride_token, kb, a, c.status, diag, c.k_sum);
}

template <typename T, int D>
hipError_t merge_td(const fastar_cache_t& c, const fastar_tensor_t& kn, const fastar_tensor_t& vn,
                    const int32_t* kb, int F, float tau, int32_t* group_of_new, int32_t* rep_offsets,
                    int32_t* rep_perm, const MergeWs& ws, fastar_diag_t* diag, hipStream_t s) {
  const int H = c.heads, Tf = c.tokens_per_frame;
  MergeArgs a;
  a.H = H;
  a.Tf = Tf;
  a.cap = c.capacity;
  a.F = F;
  a.nbits = c.n_bits;
  a.kb_stride = ws.kb_stride > 0 ? ws.kb_stride : (int64_t)F * Tf;
  a.off = ws.off;
  a.tok = ws.tok;
  a.tbk = ws.tbk;
  a.candg = ws.candg;
  a.link = ws.link;
  a.ocnt = ws.ocnt;
  a.nextj = ws.nextj;
  a.prop = ws.prop;
  {
    // the index launch works out the match ranges when its LDS allows
    const size_t nb1 = ((((size_t)1 << c.n_bits) + 1) + 3) & ~(size_t)3;
    const size_t full_lds = (nb1 * 2 + (size_t)Tf) * sizeof(int32_t);
    const bool ranges = full_lds <= kTcIndexLds;
    a.mrange = ranges ? ws.mrange : nullptr;
    const size_t tc_lds = ranges ? full_lds : nb1 * sizeof(int32_t);
    hipLaunchKernelGGL(tc_index_kernel, dim3(F + 1, H), dim3(1024), tc_lds, s, c.frontier, c.rep_bucket,
                       c.n_groups, kb, a);
  }
  // extra workgroups (planes after the frames', dispatched last) hash the
  // jobs that come with the merge: about kMatchHashTiles tiles per wave, at
  // most kMatchHashPlanes planes
  HashJobs qh;
  qh.count = 0;
  int qblocks = 0, qz = 0;
  if (ws.also_hash && sizeof(T) == 2) {
    const int64_t tiles = hash_tiles(*ws.also_hash, &qh);
    // tiles are numbered in 32 bits; the riding hash takes one or two probes
    if (tiles >= (int64_t)1 << 31 || hash_probe_class(qh) != 2) return hipErrorInvalidValue;
    const int64_t plane = (int64_t)match_groups(Tf) * H;
    const int64_t want = (tiles + 4 * kMatchHashTiles - 1) / (4 * kMatchHashTiles);
    qblocks = (int)(want < kMatchHashPlanes * plane ? want : kMatchHashPlanes * plane);
    qz = (int)((qblocks + plane - 1) / plane);
  }
  hipLaunchKernelGGL((tc_match_kernel<T, D>),
                     dim3((unsigned)match_groups(Tf), (unsigned)H, (unsigned)(F + qz)),
                     dim3(256),
                     (match_lds_words<T, D>() * sizeof(int32_t)), s,
                     (const T*)c.rep_k,
                     (const T*)kn.data, kn.stride_head, kn.stride_token, c.frontier, tau, a, diag, qh,
                     (const uint16_t*)ws.hash_planes, ws.hash_bits, qblocks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ws.after_match && (e = hipEventRecord(ws.after_match, s)) != hipSuccess) return e;
  apply_launch<T, D>(c, kn, vn, kb, a, group_of_new, ws.rep, diag, s);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ws.index_after) {
    // the job riding on the index launch is produced on another stream
    e = hipStreamWaitEvent(s, ws.index_after, 0);
    if (e != hipSuccess) return e;
  }
  if (rep_offsets && rep_perm)
    return launch_bucket_index(c.rep_bucket, H, c.capacity, 1, c.n_bits, c.n_groups, rep_offsets,
                               rep_perm, ws.index_ws, s, ws.also_index);
  return hipSuccess;
}

template <typename T, int D>
hipError_t apply_td(const fastar_cache_t& c, const fastar_tensor_t& kn, const fastar_tensor_t& vn,
                    const int32_t* kb, const MergeArgs& a, int32_t* group_of_new, int32_t* rep_offsets,
                    int32_t* rep_perm, const MergeWs& ws, fastar_diag_t* diag, hipStream_t s) {
  apply_launch<T, D>(c, kn, vn, kb, a, group_of_new, ws.rep, diag, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ws.index_after) {
    e = hipStreamWaitEvent(s, ws.index_after, 0);
    if (e != hipSuccess) return e;
  }
  if (rep_offsets && rep_perm)
    return launch_bucket_index(c.rep_bucket, a.H, c.capacity, 1, c.n_bits, c.n_groups, rep_offsets,
                               rep_perm, ws.index_ws, s, ws.also_index);
  return hipSuccess;
}

}  // namespace

hipError_t launch_merge_apply(const fastar_cache_t& c, const fastar_tensor_t& kn, const fastar_tensor_t& vn,
                              const int32_t* kb, const MergeArgs& a, int32_t* group_of_new,
                              int32_t* rep_offsets, int32_t* rep_perm, const MergeWs& ws,
                              fastar_diag_t* diag, hipStream_t s) {
  if (c.dtype == FASTAR_BF16)
    return c.dim == 64 ? apply_td<uint16_t, 64>(c, kn, vn, kb, a, group_of_new, rep_offsets, rep_perm, ws, diag, s)
                       : apply_td<uint16_t, 128>(c, kn, vn, kb, a, group_of_new, rep_offsets, rep_perm, ws, diag, s);
  return c.dim == 64 ? apply_td<float, 64>(c, kn, vn, kb, a, group_of_new, rep_offsets, rep_perm, ws, diag, s)
                     : apply_td<float, 128>(c, kn, vn, kb, a, group_of_new, rep_offsets, rep_perm, ws, diag, s);
}

hipError_t launch_tempcache_merge(const fastar_cache_t& c, const fastar_tensor_t& k_new,
                                  const fastar_tensor_t& v_new, const int32_t* k_new_bucket,
                                  int n_frames, float tau, int32_t* group_of_new,
                                  int32_t* rep_offsets, int32_t* rep_perm, const MergeWs& ws,
                                  fastar_diag_t* diag, hipStream_t s) {
  if (c.heads == 0 || n_frames == 0) return hipSuccess;
  if (c.dtype == FASTAR_BF16)
    return c.dim == 64
               ? merge_td<uint16_t, 64>(c, k_new, v_new, k_new_bucket, n_frames, tau, group_of_new, rep_offsets, rep_perm, ws, diag, s)
               : merge_td<uint16_t, 128>(c, k_new, v_new, k_new_bucket, n_frames, tau, group_of_new, rep_offsets, rep_perm, ws, diag, s);
  return c.dim == 64
             ? merge_td<float, 64>(c, k_new, v_new, k_new_bucket, n_frames, tau, group_of_new, rep_offsets, rep_perm, ws, diag, s)
             : merge_td<float, 128>(c, k_new, v_new, k_new_bucket, n_frames, tau, group_of_new, rep_offsets, rep_perm, ws, diag, s);
}

}  // namespace fastar
