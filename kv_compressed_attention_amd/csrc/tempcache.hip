// TempCache merge on gfx950 (paperlayer.ai section 5 "TempCache", appendix A
// Lemma 5.1, appendix C representative and threshold ablations).
//
// The candidates of a new key of frame f are the previous frame's tokens in
// its bucket: for f = 0 the representatives of the cache's last frame (the
// frontier), for f > 0 the raw keys of new frame f - 1 (each of which is the
// representative of its group after frame f - 1).  The matches of all frames
// therefore do not depend on each other and run in one launch; only the group
// bookkeeping is sequential.  Four launches per call:
//   tc_index    per (table, head): the frontier and each new frame grouped by
//               bucket (LDS open-addressing table -> contiguous segments);
//   tc_match    16 lanes per new key, all frames: cosine with every candidate
//               of its bucket, keep the best, propose if it passes tau;
//   tc_resolve  one workgroup per head, frames in order: a candidate with
//               several proposers keeps the one of largest cosine (ties: smaller
//               j); the other keys open groups numbered in ascending j;
//   tc_apply    16 lanes per touched group: follow the group's chain of tokens
//               through the frames, accumulate the float32 value sum in frame
//               order, write count, sum, mean (rounded once to the cache
//               dtype), last key, its bucket and ln count.
// Cosines are compared in float32 against a certified error bound; a decision
// inside the bound is redone in float64 (where products of the stored values
// are exact) and counted in the diagnostics.

#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace fastar {

namespace {

// bound on |fl32(cos) - cos| for d exact products accumulated in float32 in
// any order (dot and both norms), then rsqrt and two multiplies; twice the
// first-order estimate
template <int D>
__device__ __forceinline__ float cos_err32() { return (float)(4 * D + 32) * 0x1p-24f; }
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
// result does not depend on the order the candidates are visited in
template <typename F>
struct Top2 {
  F c1, c2;
  int best;
  __device__ __forceinline__ void init() {
    c1 = -INFINITY;
    c2 = -INFINITY;
    best = -1;
  }
  __device__ __forceinline__ void add(F c, int i) {
    if (best < 0) {
      c1 = c;
      best = i;
    } else if (c > c1 || (c == c1 && i < best)) {
      c2 = c1 > c2 ? c1 : c2;
      c1 = c;
      best = i;
    } else if (c > c2) {
      c2 = c;
    }
  }
};

__device__ __forceinline__ uint32_t slot_hash(int b, uint32_t mask) {
  return ((uint32_t)b * 2654435761u >> 7) & mask;
}

// Groups Tf tokens by bucket for one head.  get(i, b, g) gives token i's
// bucket and group (g < 0: token left out).  Writes cand (tokens, bucket
// segments contiguous), optionally candg (their groups) and the table
// tkey/tstart/tcount (slot -> bucket + 1, segment).  Whole workgroup; lds
// must hold 2 * tsize int32 + 2 * Tf int16.
template <typename Get>
__device__ void group_by_bucket(int Tf, int tsize, Get get, int32_t* lds, int32_t* tkey,
                                int32_t* tstart, int32_t* tcount, int32_t* cand, int32_t* candg) {
  int32_t* skey = lds;
  int32_t* scnt = skey + tsize;
  int16_t* slot_of = reinterpret_cast<int16_t*>(scnt + tsize);
  int16_t* pos_of = slot_of + Tf;
  __shared__ int wtot[16];
  const uint32_t mask = (uint32_t)tsize - 1u;
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  for (int s = tid; s < tsize; s += nthr) {
    skey[s] = 0;
    scnt[s] = 0;
  }
  __syncthreads();
  for (int i = tid; i < Tf; i += nthr) {
    int b, g;
    get(i, b, g);
    if (g < 0) {
      slot_of[i] = -1;
      continue;
    }
    uint32_t slot = slot_hash(b, mask);
    while (true) {
      const int w = skey[slot];
      if (w == b + 1) break;
      if (w == 0) {
        const int old = atomicCAS(&skey[slot], 0, b + 1);
        if (old == 0 || old == b + 1) break;
      } else {
        slot = (slot + 1u) & mask;
      }
    }
    slot_of[i] = (int16_t)slot;
    pos_of[i] = (int16_t)atomicAdd(&scnt[slot], 1);
  }
  __syncthreads();
  // exclusive scan of the segment lengths over the slots
  const int per = (tsize + nthr - 1) / nthr;
  const int s0 = tid * per;
  int local = 0;
  for (int s = s0; s < s0 + per && s < tsize; ++s) local += scnt[s];
  const int lane = lane_id(), wave = tid >> 6;
  int incl = local;
#pragma unroll
  for (int off = 1; off < FASTAR_WAVE; off <<= 1) {
    const int y = __shfl_up(incl, off, FASTAR_WAVE);
    if (lane >= off) incl += y;
  }
  if (lane == FASTAR_WAVE - 1) wtot[wave] = incl;
  __syncthreads();
  int run = incl - local;
  for (int w = 0; w < wave; ++w) run += wtot[w];
  for (int s = s0; s < s0 + per && s < tsize; ++s) {
    const int c = scnt[s];
    if (tkey) {
      tkey[s] = skey[s];
      tcount[s] = c;
      tstart[s] = run;
    }
    scnt[s] = run;  // segment start, for the fill below
    run += c;
  }
  __syncthreads();
  for (int i = tid; i < Tf; i += nthr) {
    const int slot = slot_of[i];
    if (slot < 0) continue;
    int b, g;
    get(i, b, g);
    const int k = scnt[slot] + pos_of[i];
    cand[k] = i;
    if (candg) candg[k] = g;
  }
}

struct MergeArgs {
  int H, Tf, cap, F, tsize;
  int64_t kb_stride;  // F * Tf
  // per-head tables t = 0..F: table 0 indexes the cache's last frame (the
  // frontier), table f + 1 indexes new frame f, each by bucket
  int32_t* tkey;      // [H][F+1][tsize] bucket + 1, 0 = empty slot
  int32_t* tstart;    // [H][F+1][tsize] segment start in cand
  int32_t* tcount;    // [H][F+1][tsize] segment length
  int32_t* cand;      // [H][F+1][Tf] token indices, bucket segments contiguous
  int32_t* candg;     // [H][Tf] groups of table 0's tokens
  int32_t* target;    // [H][F][Tf] proposed previous-frame token, or -1
  float* tcos;        // [H][F][Tf] its cosine
  int32_t* mgroup;    // [H][F][Tf] group a token extends, -1 if it opens one
  int32_t* gid;       // [H][F][Tf] final group of each token (-1: dropped)
  int32_t* nextj;     // [H][F][Tf] token of the next frame that extends this
                      //            token's group, or -1
};

__device__ __forceinline__ int64_t tab_off(const MergeArgs& a, int h, int t) {
  return ((int64_t)h * (a.F + 1) + t) * a.tsize;
}
__device__ __forceinline__ int64_t cand_off(const MergeArgs& a, int h, int t) {
  return ((int64_t)h * (a.F + 1) + t) * a.Tf;
}
__device__ __forceinline__ int64_t frame_off(const MergeArgs& a, int h, int f) {
  return ((int64_t)h * a.F + f) * a.Tf;
}

// Table 0 from the frontier (blockIdx.x == 0) or table f + 1 from new frame f.
// One workgroup per (table, head).
__global__ __launch_bounds__(1024) void tc_index_kernel(
    const int32_t* __restrict__ frontier, const int32_t* __restrict__ rep_bucket,
    const int32_t* __restrict__ n_groups, const int32_t* __restrict__ kbucket, MergeArgs a) {
  extern __shared__ int32_t lds[];
  const int h = blockIdx.y;
  const int t = blockIdx.x;
  int32_t* tk = a.tkey + tab_off(a, h, t);
  int32_t* ts = a.tstart + tab_off(a, h, t);
  int32_t* tc = a.tcount + tab_off(a, h, t);
  int32_t* cd = a.cand + cand_off(a, h, t);
  if (t == 0) {
    const bool empty = n_groups[h] <= 0;
    const int32_t* fr = frontier + (int64_t)h * a.Tf;
    const int32_t* rb = rep_bucket + (int64_t)h * a.cap;
    group_by_bucket(
        a.Tf, a.tsize,
        [&](int i, int& b, int& g) {
          g = empty ? -1 : fr[i];
          b = g >= 0 ? rb[g] : 0;
        },
        lds, tk, ts, tc, cd, a.candg + (int64_t)h * a.Tf);
  } else {
    const int32_t* kb = kbucket + (int64_t)h * a.kb_stride + (int64_t)(t - 1) * a.Tf;
    group_by_bucket(
        a.Tf, a.tsize,
        [&](int i, int& b, int& g) {
          b = kb[i];
          g = 0;
        },
        lds, tk, ts, tc, cd, nullptr);
  }
}

// Best previous-frame candidate of every new key of every frame, 16 lanes per
// key (each lane d/16 dims).  Frame f's candidates are the frontier (f = 0)
// or new frame f - 1's tokens with the key's bucket; keys are visited in
// bucket order so that neighbouring groups of lanes share candidate rows.
template <typename T, int D>
__global__ __launch_bounds__(256) void tc_match_kernel(
    const T* __restrict__ rep_k, const T* __restrict__ knew, int64_t k_sh, int64_t k_st,
    const int32_t* __restrict__ kbucket, const int32_t* __restrict__ n_groups, float tau,
    MergeArgs a, fastar_diag_t* __restrict__ diag) {
  constexpr int EPL = D / 16;
  const int h = blockIdx.y;
  const int f = blockIdx.z;
  const int sub = threadIdx.x & 15;
  const int p = blockIdx.x * 16 + (threadIdx.x >> 4);
  if (p >= a.Tf) return;  // whole 16-lane group
  const int j = a.cand[cand_off(a, h, f + 1) + p];
  const T* kj = knew + (int64_t)h * k_sh + ((int64_t)f * a.Tf + j) * k_st + sub * EPL;
  float av[EPL];
  Chunk<T, EPL>::load(kj, av);
  int start = 0, cnt = 0;
  if (f > 0 || n_groups[h] > 0) {
    const int bj = kbucket[(int64_t)h * a.kb_stride + (int64_t)f * a.Tf + j];
    const uint32_t mask = (uint32_t)a.tsize - 1u;
    const int32_t* tk = a.tkey + tab_off(a, h, f);
    uint32_t slot = slot_hash(bj, mask);
    int w;
    while ((w = tk[slot]) != 0 && w != bj + 1) slot = (slot + 1u) & mask;
    if (w != 0) {
      start = a.tstart[tab_off(a, h, f) + slot];
      cnt = a.tcount[tab_off(a, h, f) + slot];
    }
  }
  int best = -1;
  float cb = 0.f;
  bool prop = false;
  if (cnt > 0) {
    const int32_t* ci = a.cand + cand_off(a, h, f) + start;
    const int32_t* cg = a.candg + (int64_t)h * a.Tf + start;
    // candidate row k: the representative of its group (f == 0) or the raw key
    // of new frame f - 1 (it is the representative of whatever group it is in)
    const T* base0 = rep_k + (int64_t)h * a.cap * D + sub * EPL;
    const T* base1 = knew + (int64_t)h * k_sh + (int64_t)(f - 1) * a.Tf * k_st + sub * EPL;
    auto row = [&](int k) -> const T* {
      return f == 0 ? base0 + (int64_t)cg[k] * D : base1 + (int64_t)ci[k] * k_st;
    };
    float nj2 = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) nj2 = fmaf(av[e], av[e], nj2);
    nj2 = sum16(nj2);
    const float rj = nj2 > 0.f ? rsqrtf(nj2) : 0.f;
    Top2<float> t;
    t.init();
    constexpr int U = 4;  // candidates per batch, so that their row loads overlap
    for (int k0 = 0; k0 < cnt; k0 += U) {
      const T* rp[U];
      int ik[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int kk = k0 + u < cnt ? k0 + u : k0;
        rp[u] = row(kk);
        ik[u] = ci[kk];
      }
      float r[U][EPL];
#pragma unroll
      for (int u = 0; u < U; ++u) Chunk<T, EPL>::load(rp[u], r[u]);
      float dt[U], ni2[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        dt[u] = 0.f;
        ni2[u] = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          dt[u] = fmaf(av[e], r[u][e], dt[u]);
          ni2[u] = fmaf(r[u][e], r[u][e], ni2[u]);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        dt[u] = sum16(dt[u]);
        ni2[u] = sum16(ni2[u]);
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (k0 + u < cnt) t.add((nj2 > 0.f && ni2[u] > 0.f) ? dt[u] * rj * rsqrtf(ni2[u]) : 0.f, ik[u]);
    }
    const float e32 = cos_err32<D>();
    best = t.best;
    cb = t.c1;
    if (t.c1 < tau - e32) {
      prop = false;  // no candidate can reach tau
    } else if (t.c1 >= tau + e32 && t.c1 - t.c2 > 2.f * e32) {
      prop = true;   // clear winner, clearly above tau
    } else {
      // float64: products of the stored values are exact
      if (diag && sub == 0) atomicAdd(&diag->merge_fallbacks, 1u);
      double ad[EPL];
      double n1 = 0.0;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        ad[e] = (double)av[e];
        n1 += ad[e] * ad[e];
      }
      n1 = sum16d(n1);
      Top2<double> u;
      u.init();
      for (int k = 0; k < cnt; ++k) {
        float r[EPL];
        Chunk<T, EPL>::load(row(k), r);
        double dt = 0.0, n2 = 0.0;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          dt += ad[e] * (double)r[e];
          n2 += (double)r[e] * (double)r[e];
        }
        dt = sum16d(dt);
        n2 = sum16d(n2);
        u.add((n1 > 0.0 && n2 > 0.0) ? dt / sqrt(n1 * n2) : 0.0, ci[k]);
      }
      const double e64 = cos_err64<D>();
      const bool sure = (u.c1 < (double)tau - e64) ||
                        (u.c1 >= (double)tau + e64 && u.c1 - u.c2 > 2.0 * e64);
      if (!sure && diag && sub == 0) atomicAdd(&diag->unresolved, 1u);
      best = u.best;
      prop = u.c1 >= (double)tau;
      cb = (float)u.c1;
    }
  }
  if (sub == 0) {
    a.target[frame_off(a, h, f) + j] = prop ? best : -1;
    a.tcos[frame_off(a, h, f) + j] = cb;
  }
}

template <typename T, int D>
__device__ double cos64(const T* x, const T* y) {
  double s = 0.0, na = 0.0, nb = 0.0;
  for (int d = 0; d < D; ++d) {
    const double u = (double)Elem<T>::load(x, d);
    const double v = (double)Elem<T>::load(y, d);
    s += u * v;
    na += u * u;
    nb += v * v;
  }
  if (na == 0.0 || nb == 0.0) return 0.0;
  return s / sqrt(na * nb);
}

// One workgroup per head walks the frames in order.  Per frame: a candidate
// proposed to by several keys keeps the proposer of largest cosine (ties to
// smaller j); winners extend the candidate's group (mgroup, and the chain link
// nextj of the candidate); the others are numbered as new groups in ascending
// j (gid, group_of_new).  At the end: the frontier and the group count.
template <typename T, int D>
__global__ __launch_bounds__(1024) void tc_resolve_kernel(
    const T* __restrict__ rep_k, int32_t* __restrict__ frontier,
    int32_t* __restrict__ n_groups, const T* __restrict__ knew, int64_t k_sh, int64_t k_st,
    int32_t* __restrict__ group_of_new, MergeArgs a, fastar_diag_t* __restrict__ diag) {
  extern __shared__ int32_t lds[];
  const int Tf = a.Tf;
  int32_t* plist = lds;                              // [Tf] proposer list heads
  float* tcl = reinterpret_cast<float*>(plist + Tf); // [Tf]
  int16_t* tg = reinterpret_cast<int16_t*>(tcl + Tf);// [Tf]
  int16_t* nxt = tg + Tf;                            // [Tf]
  __shared__ int wsum[16];
  __shared__ int running;
  const int h = blockIdx.x;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = lane_id();
  const float e = cos_err32<D>();
  const double e64 = cos_err64<D>();
  int ng = n_groups[h];
  const T* kh = knew + (int64_t)h * k_sh;
  for (int f = 0; f < a.F; ++f) {
    const int64_t fo = frame_off(a, h, f);
    for (int i = tid; i < Tf; i += blockDim.x) {
      plist[i] = -1;
      tg[i] = (int16_t)a.target[fo + i];
      tcl[i] = a.tcos[fo + i];
      a.nextj[fo + i] = -1;
    }
    if (tid == 0) running = 0;
    __syncthreads();
    for (int j = tid; j < Tf; j += blockDim.x) {
      const int i = tg[j];
      if (i >= 0) nxt[j] = (int16_t)atomicExch(&plist[i], j);
    }
    __syncthreads();
    for (int j = tid; j < Tf; j += blockDim.x) {
      const int i = tg[j];
      bool win = i >= 0;
      if (win) {
        const float cj = tcl[j];
        bool amb = false;
        for (int j2 = plist[i]; j2 >= 0; j2 = nxt[j2]) {
          if (j2 == j) continue;
          const float c = tcl[j2];
          if (c > cj + 2.f * e) win = false;
          else if (c >= cj - 2.f * e) amb = true;
        }
        if (win && amb) {
          if (diag) atomicAdd(&diag->merge_fallbacks, 1u);
          const T* prev = f == 0 ? rep_k + ((int64_t)h * a.cap + frontier[(int64_t)h * Tf + i]) * D
                                 : kh + ((int64_t)(f - 1) * Tf + i) * k_st;
          const double dj = cos64<T, D>(kh + ((int64_t)f * Tf + j) * k_st, prev);
          bool unres = false;
          for (int j2 = plist[i]; j2 >= 0; j2 = nxt[j2]) {
            if (j2 == j) continue;
            const double dd = cos64<T, D>(kh + ((int64_t)f * Tf + j2) * k_st, prev);
            if (fabs(dd - dj) <= 2.0 * e64) unres = true;
            if (dd > dj || (dd == dj && j2 < j)) win = false;
          }
          if (unres && diag) atomicAdd(&diag->unresolved, 1u);
        }
      }
      int mg = -1;
      if (win) {
        // the candidate's group; a token dropped for capacity has none
        mg = f == 0 ? frontier[(int64_t)h * Tf + i] : a.gid[frame_off(a, h, f - 1) + i];
        if (mg >= 0 && f > 0) a.nextj[frame_off(a, h, f - 1) + i] = j;
      }
      a.mgroup[fo + j] = mg;
    }
    __threadfence_block();
    __syncthreads();
    // number the new groups in ascending j
    for (int base = 0; base < Tf; base += blockDim.x) {
      const int j = base + tid;
      const int mg = j < Tf ? a.mgroup[fo + j] : 0;
      const bool isnew = j < Tf && mg < 0;
      const uint64_t bal = ballot64(isnew);
      if (lane == 0) wsum[wave] = __popcll(bal);
      __syncthreads();
      int rank = running + __popcll(bal & lanemask_lt());
      for (int w = 0; w < wave; ++w) rank += wsum[w];
      if (j < Tf) {
        int g = isnew ? ng + rank : mg;
        if (isnew && g >= a.cap) {
          g = -1;
          if (diag) atomicAdd(&diag->capacity_overflow, 1u);
        }
        a.gid[fo + j] = g;
        if (group_of_new) group_of_new[(int64_t)h * a.kb_stride + (int64_t)f * Tf + j] = g;
      }
      __syncthreads();
      if (tid == 0) {
        int sum = 0;
        for (int w = 0; w < (int)(blockDim.x >> 6); ++w) sum += wsum[w];
        running += sum;
      }
      __syncthreads();
    }
    ng = ng + running < a.cap ? ng + running : a.cap;
    __threadfence_block();
    __syncthreads();
  }
  for (int j = tid; j < Tf; j += blockDim.x) frontier[(int64_t)h * Tf + j] = a.gid[frame_off(a, h, a.F - 1) + j];
  if (tid == 0) n_groups[h] = ng;
}

// Group rows, 16 lanes per group touched by the chunk (D/16 elements each).
// A chain starts at a token that opens a new group, or at a frame-0 token that
// extends an existing group; it follows nextj through the later frames.  Value
// sums are accumulated frame by frame in float32, exactly as merging the
// frames one at a time would; the representative is the chain's last key.
template <typename T, int D>
__global__ __launch_bounds__(256) void tc_apply_kernel(
    T* __restrict__ rep_k, T* __restrict__ v_mean, float* __restrict__ v_sum,
    int32_t* __restrict__ count, float* __restrict__ log_count, int32_t* __restrict__ rep_bucket,
    const T* __restrict__ knew, int64_t k_sh, int64_t k_st, const T* __restrict__ vnew,
    int64_t v_sh, int64_t v_st, const int32_t* __restrict__ kbucket, MergeArgs a) {
  constexpr int EPL = D / 16;
  const int h = blockIdx.y;
  const int64_t idx = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  if (idx >= (int64_t)a.F * a.Tf) return;
  int f = (int)(idx / a.Tf);
  int j = (int)(idx - (int64_t)f * a.Tf);
  const int g = a.gid[frame_off(a, h, f) + j];
  if (g < 0) return;
  const int mg = a.mgroup[frame_off(a, h, f) + j];
  if (mg >= 0 && f > 0) return;  // continuation of a chain that starts earlier
  const int64_t gi = (int64_t)h * a.cap + g;
  float sum[EPL];
  int cnt;
  {
    float vv[EPL];
    Chunk<T, EPL>::load(vnew + (int64_t)h * v_sh + ((int64_t)f * a.Tf + j) * v_st + sub * EPL, vv);
    if (mg < 0) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) sum[e] = vv[e];
      cnt = 1;
    } else {
      const float* vs = v_sum + gi * D + sub * EPL;
#pragma unroll
      for (int e = 0; e < EPL; ++e) sum[e] = vs[e] + vv[e];
      cnt = count[gi] + 1;
    }
  }
  while (f + 1 < a.F) {
    const int nx = a.nextj[frame_off(a, h, f) + j];
    if (nx < 0) break;
    ++f;
    j = nx;
    float vv[EPL];
    Chunk<T, EPL>::load(vnew + (int64_t)h * v_sh + ((int64_t)f * a.Tf + j) * v_st + sub * EPL, vv);
#pragma unroll
    for (int e = 0; e < EPL; ++e) sum[e] += vv[e];
    ++cnt;
  }
  const T* kr = knew + (int64_t)h * k_sh + ((int64_t)f * a.Tf + j) * k_st + sub * EPL;
  T* rkr = rep_k + gi * D + sub * EPL;
  T* vmr = v_mean + gi * D + sub * EPL;
  float* vsr = v_sum + gi * D + sub * EPL;
  const float fc = (float)cnt;
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    vsr[e] = sum[e];
    rkr[e] = kr[e];
    if (cnt == 1) Elem<T>::store(vmr, e, sum[e]);  // exact copy of the value
    else Elem<T>::store(vmr, e, sum[e] / fc);
  }
  if (sub == 0) {
    count[gi] = cnt;
    log_count[gi] = logf(fc);
    rep_bucket[gi] = kbucket[(int64_t)h * a.kb_stride + (int64_t)f * a.Tf + j];
  }
}

int table_size(int Tf) {
  int t = 16;
  while (t < 2 * Tf) t <<= 1;
  return t;
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
  a.tsize = table_size(Tf);
  a.kb_stride = (int64_t)F * Tf;
  a.tkey = ws.tkey;
  a.tstart = ws.tstart;
  a.tcount = ws.tcount;
  a.cand = ws.cand;
  a.candg = ws.candg;
  a.target = ws.target;
  a.tcos = ws.tcos;
  a.mgroup = ws.mgroup;
  a.gid = ws.gid;
  a.nextj = ws.nextj;
  const size_t index_lds = (size_t)2 * a.tsize * sizeof(int32_t) + (size_t)2 * Tf * sizeof(int16_t);
  const size_t resolve_lds = (size_t)Tf * (2 * sizeof(int32_t) + 2 * sizeof(int16_t));
  hipLaunchKernelGGL(tc_index_kernel, dim3(F + 1, H), dim3(1024), index_lds, s, c.frontier,
                     c.rep_bucket, c.n_groups, kb, a);
  hipLaunchKernelGGL((tc_match_kernel<T, D>), dim3((unsigned)((Tf + 15) / 16), (unsigned)H, F),
                     dim3(256), 0, s, (const T*)c.rep_k, (const T*)kn.data, kn.stride_head,
                     kn.stride_token, kb, c.n_groups, tau, a, diag);
  hipLaunchKernelGGL((tc_resolve_kernel<T, D>), dim3(H), dim3(1024), resolve_lds, s,
                     (const T*)c.rep_k, c.frontier, c.n_groups, (const T*)kn.data, kn.stride_head,
                     kn.stride_token, group_of_new, a, diag);
  hipLaunchKernelGGL((tc_apply_kernel<T, D>), dim3((unsigned)(((int64_t)F * Tf + 15) / 16), (unsigned)H),
                     dim3(256), 0, s, (T*)c.rep_k, (T*)c.v_mean, c.v_sum, c.count, c.log_count,
                     c.rep_bucket, (const T*)kn.data, kn.stride_head, kn.stride_token,
                     (const T*)vn.data, vn.stride_head, vn.stride_token, kb, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (rep_offsets && rep_perm)
    return launch_bucket_index(c.rep_bucket, H, c.capacity, 1, c.n_bits, c.n_groups, rep_offsets,
                               rep_perm, ws.index_ws, s);
  return hipSuccess;
}

}  // namespace

int tempcache_table_size(int tokens_per_frame) { return table_size(tokens_per_frame); }

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
