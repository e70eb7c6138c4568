// TempCache merge on gfx950 (paperlayer.ai section 5 "TempCache", appendix A
// Lemma 5.1, appendix C representative and threshold ablations).
//
// Frames are merged one after another.  The candidates of a new key are the
// previous frame's tokens in its bucket; they are kept per head as a small
// bucket index (an open-addressing table from bucket id to a segment of a
// candidate array, built in LDS by one workgroup and stored in the
// workspace).  Per frame:
//   tc_match    16 lanes per new key: walk the key's candidate segment, cosine
//               of each (lanes split the dims, shuffles reduce), keep the best;
//               propose if it passes tau;
//   tc_resolve  one workgroup per head: a candidate proposed to by several
//               keys keeps the proposer of largest cosine (ties: smaller j);
//               the other keys are numbered as new groups in ascending j; the
//               candidate index for the next frame is built from this frame;
//   tc_apply    group row updates (count, float32 value sum, value mean
//               rounded once to the cache dtype, representative key and
//               bucket, ln count), 16 lanes per row.
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

struct PrevIndexArgs {
  int32_t* tkey;    // [H][tsize] bucket + 1, 0 = empty slot
  int32_t* tstart;  // [H][tsize] segment start in cand
  int32_t* tcount;  // [H][tsize] segment length
  int32_t* cand;    // [H][Tf] previous-frame token index
  int32_t* candg;   // [H][Tf] its group
};

// Builds head h's candidate index from Tf tokens; get(i, b, g) gives token
// i's bucket and group (g < 0: token has no group).  Whole workgroup; lds
// must hold 2 * tsize int32 + 2 * Tf int16.
template <typename Get>
__device__ void build_prev_index(int h, int Tf, int tsize, Get get, int32_t* lds,
                                 const PrevIndexArgs& ix) {
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
  int32_t* gk = ix.tkey + (int64_t)h * tsize;
  int32_t* gs = ix.tstart + (int64_t)h * tsize;
  int32_t* gc = ix.tcount + (int64_t)h * tsize;
  for (int s = s0; s < s0 + per && s < tsize; ++s) {
    const int c = scnt[s];
    gk[s] = skey[s];
    gc[s] = c;
    gs[s] = run;
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
    ix.cand[(int64_t)h * Tf + k] = i;
    ix.candg[(int64_t)h * Tf + k] = g;
  }
}

// Candidate index of the cache's last frame (the frontier), for the first
// frame of a merge call.  One workgroup per head.
__global__ __launch_bounds__(1024) void tc_index_frontier_kernel(
    const int32_t* __restrict__ frontier, const int32_t* __restrict__ rep_bucket, int cap, int Tf,
    int tsize, const int32_t* __restrict__ ng_in, PrevIndexArgs ix) {
  extern __shared__ int32_t lds[];
  const int h = blockIdx.x;
  const bool empty = ng_in[h] <= 0;
  const int32_t* fr = frontier + (int64_t)h * Tf;
  const int32_t* rb = rep_bucket + (int64_t)h * cap;
  build_prev_index(
      h, Tf, tsize,
      [&](int i, int& b, int& g) {
        g = empty ? -1 : fr[i];
        b = g >= 0 ? rb[g] : 0;
      },
      lds, ix);
}

template <typename T, int D>
__global__ __launch_bounds__(256) void tc_match_kernel(
    const T* __restrict__ rep_k, int cap, int Tf, int tsize, PrevIndexArgs ix,
    const T* __restrict__ knew, int64_t k_sh, int64_t k_st, int64_t frame_off,
    const int32_t* __restrict__ kbucket, int64_t kb_stride, const int32_t* __restrict__ ng_in,
    float tau, int32_t* __restrict__ target, float* __restrict__ tcos,
    fastar_diag_t* __restrict__ diag) {
  constexpr int EPL = D / 16;
  const int h = blockIdx.y;
  const int sub = threadIdx.x & 15;
  const int j = blockIdx.x * 16 + (threadIdx.x >> 4);
  if (j >= Tf) return;  // whole 16-lane group
  int best = -1;
  float cb = 0.f;
  bool prop = false;
  int start = 0, cnt = 0;
  if (ng_in[h] > 0) {
    const int bj = kbucket[(int64_t)h * kb_stride + frame_off + j];
    const uint32_t mask = (uint32_t)tsize - 1u;
    const int32_t* tk = ix.tkey + (int64_t)h * tsize;
    uint32_t slot = slot_hash(bj, mask);
    int w;
    while ((w = tk[slot]) != 0 && w != bj + 1) slot = (slot + 1u) & mask;
    if (w != 0) {
      start = ix.tstart[(int64_t)h * tsize + slot];
      cnt = ix.tcount[(int64_t)h * tsize + slot];
    }
  }
  if (cnt > 0) {
    const T* kj = knew + (int64_t)h * k_sh + (frame_off + j) * k_st + sub * EPL;
    const T* rk = rep_k + (int64_t)h * cap * D + sub * EPL;
    const int32_t* ci = ix.cand + (int64_t)h * Tf + start;
    const int32_t* cg = ix.candg + (int64_t)h * Tf + start;
    float a[EPL];
    Chunk<T, EPL>::load(kj, a);
    float nj2 = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) nj2 = fmaf(a[e], a[e], nj2);
    nj2 = sum16(nj2);
    const float rj = nj2 > 0.f ? rsqrtf(nj2) : 0.f;
    Top2<float> t;
    t.init();
    // candidates in batches of 4, so that their row loads overlap
    constexpr int U = 4;
    for (int k0 = 0; k0 < cnt; k0 += U) {
      int gk[U], ik[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int kk = k0 + u < cnt ? k0 + u : k0;
        gk[u] = cg[kk];
        ik[u] = ci[kk];
      }
      float r[U][EPL];
#pragma unroll
      for (int u = 0; u < U; ++u) Chunk<T, EPL>::load(rk + (int64_t)gk[u] * D, r[u]);
      float dt[U], ni2[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        dt[u] = 0.f;
        ni2[u] = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          dt[u] = fmaf(a[e], r[u][e], dt[u]);
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
        ad[e] = (double)a[e];
        n1 += ad[e] * ad[e];
      }
      n1 = sum16d(n1);
      Top2<double> u;
      u.init();
      for (int k = 0; k < cnt; ++k) {
        float r[EPL];
        Chunk<T, EPL>::load(rk + (int64_t)cg[k] * D, r);
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
    target[(int64_t)h * Tf + j] = prop ? best : -1;
    tcos[(int64_t)h * Tf + j] = cb;
  }
}

template <typename T, int D>
__device__ double cos64(const T* a, const T* b) {
  double s = 0.0, na = 0.0, nb = 0.0;
  for (int d = 0; d < D; ++d) {
    const double x = (double)Elem<T>::load(a, d);
    const double y = (double)Elem<T>::load(b, d);
    s += x * y;
    na += x * x;
    nb += y * y;
  }
  if (na == 0.0 || nb == 0.0) return 0.0;
  return s / sqrt(na * nb);
}

// One workgroup per head: settles conflicts (a candidate keeps the proposer of
// largest cosine, ties to smaller j), numbers the new groups in ascending j,
// writes each token's group (gid), the group it extends (mgroup, -1 for a new
// group), the frontier and group_of_new, and builds the candidate index of
// this frame for the next one.
template <typename T, int D>
__global__ __launch_bounds__(1024) void tc_resolve_kernel(
    const T* __restrict__ rep_k, int cap, int32_t* __restrict__ frontier, int Tf, int tsize,
    const T* __restrict__ knew, int64_t k_sh, int64_t k_st, int64_t frame_off,
    const int32_t* __restrict__ kbucket, int64_t kb_stride, const int32_t* __restrict__ target,
    const float* __restrict__ tcos, const int32_t* __restrict__ ng_in,
    int32_t* __restrict__ ng_out, int32_t* __restrict__ mgroup, int32_t* __restrict__ gid,
    int32_t* __restrict__ group_of_new, int build_next, PrevIndexArgs ix,
    fastar_diag_t* __restrict__ diag) {
  extern __shared__ int32_t lds[];
  int32_t* plist = lds;                              // [Tf] proposer list heads
  float* tc = reinterpret_cast<float*>(plist + Tf);  // [Tf]
  int16_t* tg = reinterpret_cast<int16_t*>(tc + Tf); // [Tf]
  int16_t* nxt = tg + Tf;                            // [Tf]
  __shared__ int wsum[16];
  __shared__ int running;
  const int h = blockIdx.x;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = lane_id();
  const int ng0 = ng_in[h];
  for (int i = tid; i < Tf; i += blockDim.x) {
    plist[i] = -1;
    tg[i] = (int16_t)target[(int64_t)h * Tf + i];
    tc[i] = tcos[(int64_t)h * Tf + i];
  }
  if (tid == 0) running = 0;
  __syncthreads();
  for (int j = tid; j < Tf; j += blockDim.x) {
    const int i = tg[j];
    if (i >= 0) nxt[j] = (int16_t)atomicExch(&plist[i], j);
  }
  __syncthreads();
  int32_t* mg_h = mgroup + (int64_t)h * Tf;
  const float e = cos_err32<D>();
  for (int j = tid; j < Tf; j += blockDim.x) {
    const int i = tg[j];
    bool win = i >= 0;
    if (win) {
      const float cj = tc[j];
      bool amb = false;
      for (int j2 = plist[i]; j2 >= 0; j2 = nxt[j2]) {
        if (j2 == j) continue;
        const float c = tc[j2];
        if (c > cj + 2.f * e) win = false;
        else if (c >= cj - 2.f * e) amb = true;
      }
      if (win && amb) {
        if (diag) atomicAdd(&diag->merge_fallbacks, 1u);
        const T* kh = knew + (int64_t)h * k_sh;
        const T* prev = rep_k + ((int64_t)h * cap + frontier[(int64_t)h * Tf + i]) * D;
        const double dj = cos64<T, D>(kh + (frame_off + j) * k_st, prev);
        const double e64 = cos_err64<D>();
        bool unres = false;
        for (int j2 = plist[i]; j2 >= 0; j2 = nxt[j2]) {
          if (j2 == j) continue;
          const double d = cos64<T, D>(kh + (frame_off + j2) * k_st, prev);
          if (fabs(d - dj) <= 2.0 * e64) unres = true;
          if (d > dj || (d == dj && j2 < j)) win = false;
        }
        if (unres && diag) atomicAdd(&diag->unresolved, 1u);
      }
    }
    mg_h[j] = win ? frontier[(int64_t)h * Tf + i] : -1;
  }
  __threadfence_block();
  __syncthreads();
  // number the new groups in ascending j
  int32_t* gid_h = gid + (int64_t)h * Tf;
  for (int base = 0; base < Tf; base += blockDim.x) {
    const int j = base + tid;
    const int mg = j < Tf ? mg_h[j] : 0;
    const bool isnew = j < Tf && mg < 0;
    const uint64_t bal = ballot64(isnew);
    if (lane == 0) wsum[wave] = __popcll(bal);
    __syncthreads();
    int rank = running + __popcll(bal & lanemask_lt());
    for (int w = 0; w < wave; ++w) rank += wsum[w];
    if (j < Tf) {
      int g = isnew ? ng0 + rank : mg;
      if (isnew && g >= cap) {
        g = -1;
        if (diag) atomicAdd(&diag->capacity_overflow, 1u);
      }
      gid_h[j] = g;
      frontier[(int64_t)h * Tf + j] = g;
      if (group_of_new) group_of_new[(int64_t)h * kb_stride + frame_off + j] = g;
    }
    __syncthreads();
    if (tid == 0) {
      int s = 0;
      for (int w = 0; w < (int)(blockDim.x >> 6); ++w) s += wsum[w];
      running += s;
    }
    __syncthreads();
  }
  if (tid == 0) {
    const int ng1 = ng0 + running;
    ng_out[h] = ng1 < cap ? ng1 : cap;
  }
  if (build_next) {
    __threadfence_block();
    __syncthreads();
    const int32_t* kb = kbucket + (int64_t)h * kb_stride + frame_off;
    build_prev_index(
        h, Tf, tsize,
        [&](int i, int& b, int& g) {
          g = gid_h[i];
          b = kb[i];
        },
        lds, ix);
  }
}

// Row updates, 16 lanes per new token, D/16 contiguous elements per lane.
template <typename T, int D>
__global__ __launch_bounds__(256) void tc_apply_kernel(
    T* __restrict__ rep_k, T* __restrict__ v_mean, float* __restrict__ v_sum,
    int32_t* __restrict__ count, float* __restrict__ log_count, int32_t* __restrict__ rep_bucket,
    int cap, int Tf, const T* __restrict__ knew, int64_t k_sh, int64_t k_st,
    const T* __restrict__ vnew, int64_t v_sh, int64_t v_st, int64_t frame_off,
    const int32_t* __restrict__ kbucket, int64_t kb_stride, const int32_t* __restrict__ mgroup,
    const int32_t* __restrict__ gid) {
  constexpr int EPL = D / 16;
  const int h = blockIdx.y;
  const int64_t jj = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  if (jj >= Tf) return;
  const int gg = gid[(int64_t)h * Tf + jj];
  if (gg < 0) return;
  const bool isnew = mgroup[(int64_t)h * Tf + jj] < 0;
  const int64_t gi = (int64_t)h * cap + gg;
  const T* kr = knew + (int64_t)h * k_sh + (frame_off + jj) * k_st + sub * EPL;
  const T* vr = vnew + (int64_t)h * v_sh + (frame_off + jj) * v_st + sub * EPL;
  T* rkr = rep_k + gi * D + sub * EPL;
  T* vmr = v_mean + gi * D + sub * EPL;
  float* vsr = v_sum + gi * D + sub * EPL;
  const int bkt = kbucket[(int64_t)h * kb_stride + frame_off + jj];
  if (isnew) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      rkr[e] = kr[e];
      vmr[e] = vr[e];
      vsr[e] = Elem<T>::load(vr, e);
    }
    if (sub == 0) {
      count[gi] = 1;
      log_count[gi] = 0.f;
      rep_bucket[gi] = bkt;
    }
  } else {
    const int cnt = count[gi] + 1;
    const float fc = (float)cnt;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const float s = vsr[e] + Elem<T>::load(vr, e);
      vsr[e] = s;
      Elem<T>::store(vmr, e, s / fc);
      rkr[e] = kr[e];
    }
    if (sub == 0) {
      count[gi] = cnt;
      log_count[gi] = logf(fc);
      rep_bucket[gi] = bkt;
    }
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
  const int H = c.heads, Tf = c.tokens_per_frame, cap = c.capacity;
  const int64_t kb_stride = (int64_t)F * Tf;
  const int tsize = table_size(Tf);
  PrevIndexArgs ix{ws.tkey, ws.tstart, ws.tcount, ws.cand, ws.candg};
  const size_t index_lds = (size_t)2 * tsize * sizeof(int32_t) + (size_t)2 * Tf * sizeof(int16_t);
  const size_t resolve_lds =
      std::max(index_lds, (size_t)Tf * (2 * sizeof(int32_t) + 2 * sizeof(int16_t)));
  hipLaunchKernelGGL(tc_index_frontier_kernel, dim3(H), dim3(1024), index_lds, s, c.frontier,
                     c.rep_bucket, cap, Tf, tsize, c.n_groups, ix);
  for (int f = 0; f < F; ++f) {
    const int64_t foff = (int64_t)f * Tf;
    // group counts: the cache's for the first frame in, the cache's for the last
    // frame out (each resolve reads its input count before writing its output)
    const int32_t* ng_in = f == 0 ? c.n_groups : ws.ng + (int64_t)f * H;
    int32_t* ng_out = f == F - 1 ? c.n_groups : ws.ng + (int64_t)(f + 1) * H;
    hipLaunchKernelGGL((tc_match_kernel<T, D>), dim3((unsigned)((Tf + 15) / 16), (unsigned)H),
                       dim3(256), 0, s, (const T*)c.rep_k, cap, Tf, tsize, ix, (const T*)kn.data,
                       kn.stride_head, kn.stride_token, foff, kb, kb_stride, ng_in, tau, ws.target,
                       ws.tcos, diag);
    hipLaunchKernelGGL((tc_resolve_kernel<T, D>), dim3(H), dim3(1024), resolve_lds, s,
                       (const T*)c.rep_k, cap, c.frontier, Tf, tsize, (const T*)kn.data,
                       kn.stride_head, kn.stride_token, foff, kb, kb_stride, ws.target, ws.tcos,
                       ng_in, ng_out, ws.mgroup, ws.gid, group_of_new, f < F - 1 ? 1 : 0, ix, diag);
    hipLaunchKernelGGL((tc_apply_kernel<T, D>), dim3((unsigned)((Tf + 15) / 16), (unsigned)H),
                       dim3(256), 0, s, (T*)c.rep_k, (T*)c.v_mean, c.v_sum, c.count, c.log_count,
                       c.rep_bucket, cap, Tf, (const T*)kn.data, kn.stride_head, kn.stride_token,
                       (const T*)vn.data, vn.stride_head, vn.stride_token, foff, kb, kb_stride,
                       ws.mgroup, ws.gid);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (rep_offsets && rep_perm)
    return launch_bucket_index(c.rep_bucket, H, cap, 1, c.n_bits, c.n_groups, rep_offsets, rep_perm,
                               ws.index_ws, s);
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
