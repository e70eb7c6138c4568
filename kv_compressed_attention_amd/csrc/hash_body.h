// SimHash hashing of bf16 rows as a workgroup-level body (the hash launch
// runs it, and so may other launches in workgroups of their own), and the
// float64 re-evaluation of rows float32 cannot certify.  See hash.hip for the
// method and its error bounds.
#pragma once

#include "common.h"
#include "exact_int.h"
#include "kernels.h"

namespace fastar {


// the sum of squares of 8 bf16 values (two per dot step; it only feeds the
// error bounds, which allow for its rounding)
__device__ __forceinline__ float sumsq_bf16x8(uint4 u) {
  float s = 0.f;
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i)
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[i]), __builtin_bit_cast(bf16x2_t, w[i]),
                                        s, false);
  return s;
}

// a wave's counts of the diag events (wave-uniform), added to the device
// counters once when its rows are done (one atomic per counter, not one per
// event: a wave that waited for such an atomic before its next tile's rows
// stalled)
struct HashCounts {
  uint32_t rows = 0u, signs = 0u, unresolved = 0u;
};
__device__ __forceinline__ void hash_counts_flush(const HashCounts& c, fastar_diag_t* __restrict__ diag) {
  if (!diag || lane_id() != 0) return;
  if (c.rows) atomicAdd(&diag->hash_fallback_rows, c.rows);
  if (c.signs) atomicAdd(&diag->hash_exact_signs, c.signs);
  if (c.unresolved) atomicAdd(&diag->unresolved, c.unresolved);
}

// best / second-best hyperplane distance, merged across lanes
struct Nearest {
  float d1, d2;
  int j1;
};

__device__ __forceinline__ void nearest_merge(Nearest& a, int xor_mask) {
  const float pd1 = shfl_xor_f(a.d1, xor_mask);
  const float pd2 = shfl_xor_f(a.d2, xor_mask);
  const int pj1 = shfl_xor_i(a.j1, xor_mask);
  if (pd1 < a.d1 || (pd1 == a.d1 && pj1 < a.j1)) {
    a.d2 = fminf(a.d1, pd2);
    a.d1 = pd1;
    a.j1 = pj1;
  } else {
    a.d2 = fminf(a.d2, pd1);
  }
}

template <int D>
__device__ __forceinline__ float kcert() {
  return (float)D * 0x1p-22f * (1.0f + 0x1p-10f);
}

__device__ __forceinline__ double dswap16(double v) {  // the value of lane ^ 16
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const auto lo = __builtin_amdgcn_permlane16_swap((uint32_t)u, (uint32_t)u, false, false);
  const auto hi = __builtin_amdgcn_permlane16_swap((uint32_t)(u >> 32), (uint32_t)(u >> 32), false, false);
  // each pair holds this lane's and the partner's word, in the same order
  const uint32_t l0 = lo[0], l1 = lo[1], h0 = hi[0], h1 = hi[1];
  const uint64_t a0 = ((uint64_t)h0 << 32) | l0, a1 = ((uint64_t)h1 << 32) | l1;
  return __builtin_bit_cast(double, a0 == u ? a1 : a0);
}
__device__ __forceinline__ double dswap32(double v) {  // the value of lane ^ 32
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const auto lo = __builtin_amdgcn_permlane32_swap((uint32_t)u, (uint32_t)u, false, false);
  const auto hi = __builtin_amdgcn_permlane32_swap((uint32_t)(u >> 32), (uint32_t)(u >> 32), false, false);
  const uint32_t l0 = lo[0], l1 = lo[1], h0 = hi[0], h1 = hi[1];
  const uint64_t a0 = ((uint64_t)h0 << 32) | l0, a1 = ((uint64_t)h1 << 32) | l1;
  return __builtin_bit_cast(double, a0 == u ? a1 : a0);
}
// v summed over lanes l, l ^ 16, l ^ 32 and l ^ 48 (the same value in all four)
__device__ __forceinline__ double sum4_d(double v) {
  const double w = v + dswap16(v);
  return w + dswap32(w);
}

// Re-evaluates one row in float64 and writes its ids (o: the row's output,
// the same in every lane).  Lane 16s + p takes the dims [s D/4, (s+1) D/4)
// of hyperplane p: serial sums of exact products, then added over the four
// slices.  The row (xr: [D], LDS) and the hyperplanes (ps, row stride pst;
// LDS or global memory) are read through generic pointers.  A sign float64
// cannot certify is settled exactly with an expansion sum in E (D + 2
// doubles of LDS), and so is an order of two probe distances (integers in
// E's words: exact_ratio_cmp); the distances and their error bounds go
// through DE (32 doubles of LDS).
template <typename T, int D>
__device__ inline void hash_fixup_row(const T* xr, const T* ps, int pst, int32_t* __restrict__ o, int P,
                               int nb, HashCounts& hc, double* E, double* DE) {
  constexpr int DS = D / 4;
  const int lane = lane_id();
  const int sl = lane >> 4, p = lane & 15;
  const bool active = p < nb;
  const T* rp = ps + (active ? p : 0) * pst;
  double s = 0.0, a = 0.0, n2 = 0.0;
  if (active) {
#pragma unroll 8
    for (int d = sl * DS; d < sl * DS + DS; ++d) {
      const double xv = (double)Elem<T>::load(xr, d);
      const double rv = (double)Elem<T>::load(rp, d);
      const double pr = xv * rv;  // exact: at most 48 significant bits
      s += pr;
      a += fabs(pr);
      n2 += rv * rv;
    }
  }
  s = sum4_d(s);
  a = sum4_d(a);
  n2 = sum4_d(n2);
  // any order of the D additions is within this bound
  const double bound = 2.0 * (D + 8) * 0x1p-53 * a;
  int sg = 0;
  bool need_exact = false;
  if (active) {
    if (fabs(s) > bound) sg = s > 0.0 ? 1 : -1;
    else need_exact = a != 0.0 && sl == 0;
  }
  uint64_t exact = ballot64(need_exact);
  while (exact) {
    const int src = __builtin_ctzll(exact);
    exact &= exact - 1;
    int sx = 0;
    if (lane == src) {
      int m = 0;
      for (int d = 0; d < D; ++d)
        m = grow_expansion(E, m, (double)Elem<T>::load(xr, d) * (double)Elem<T>::load(rp, d));
      sx = expansion_sign(E, m);
    }
    ++hc.signs;
    sx = __shfl(sx, src, FASTAR_WAVE);
    if (p == src) sg = sx;
  }
  const uint32_t bits = (uint32_t)(ballot64(sg > 0) & 0xFFFFu);
  bool unresolved = false;
  if (P >= 2) {
    if (sl == 0) {
      double dist = 0.0, derr = 0.0;
      if (active) {
        const double rn = sqrt(n2);
        dist = rn > 0.0 ? fabs(s) / rn : 0.0;
        derr = (a == 0.0) ? 0.0 : (rn > 0.0 ? bound / rn : 0.0) + dist * (2 * D + 8) * 0x1p-53;
      }
      DE[p] = dist;
      DE[16 + p] = derr;
    }
  }
  if (lane == 0) {
    o[0] = (int32_t)bits;
    // probes 1 .. P - 1: the P - 1 nearest hyperplanes in ascending distance
    // (ties to the smaller index).  Two distances are compared by their
    // float64 intervals where those are apart, else exactly (the sign
    // expansions in E are done with: its words hold the integers)
    const double* dist = DE;
    const double* derr = DE + 16;
    uint32_t used = 0u;
    for (int r = 0; r + 1 < P; ++r) {
      int jb = -1;
      for (int q = 0; q < nb; ++q) {
        if ((used >> q) & 1u) continue;
        if (jb < 0) {
          jb = q;
          continue;
        }
        // is q strictly nearer than jb (jb < q: a tie keeps jb)?
        bool nearer;
        if (dist[q] + derr[q] < dist[jb] - derr[jb]) {
          nearer = true;
        } else if (dist[q] - derr[q] > dist[jb] + derr[jb]) {
          nearer = false;
        } else {
          const int c = exact_ratio_cmp<T, D>(xr, ps + q * pst, ps + jb * pst, reinterpret_cast<uint32_t*>(E),
                                              2 * (D + 2), nullptr, nullptr);
          if (c == 2) unresolved = true;
          nearer = c == 2 ? dist[q] < dist[jb] : c < 0;
        }
        if (nearer) jb = q;
      }
      used |= 1u << jb;
      o[r + 1] = (int32_t)(bits ^ (1u << jb));
    }
  }
  ++hc.rows;
  if (ballot64(unresolved) != 0ull) ++hc.unresolved;
}

// Ranks of a row's hyperplane distances (ascending, ties to the smaller
// index) for probes beyond the second: dl[i] is this lane's plane p0 + i
// distance (INFINITY past nb), da[16] all of the row's.  Returns in rk[i] the
// rank of plane p0 + i and whether a plane of rank < P - 1 lies within err
// of another plane (err: the float32 distances' bound, e0 + (d + d') 2^-20).
__device__ __forceinline__ bool probe_ranks(const float* dl, const float* da, int p0, int nb, int P, float e0,
                                            int* rk) {
  bool amb = false;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int r = 0;
    bool near = false;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      if (q < nb && q != p0 + i) {
        r += (da[q] < dl[i] || (da[q] == dl[i] && q < p0 + i)) ? 1 : 0;
        near = near || fabsf(da[q] - dl[i]) <= e0 + (da[q] + dl[i]) * 0x1p-20f;
      }
    }
    rk[i] = r;
    amb = amb || (p0 + i < nb && r < P - 1 && near);
  }
  return amb;
}

// (row, hyperplane) projections a wave re-evaluates together in float64
// for one tile (hash_bf16_body, one and two probes)
constexpr int kRefinePairs = 64;
// a row with more uncertain hyperplanes than this takes the whole-row pass
constexpr int kRefineRowMax = 8;

// LDS bytes of hash_bf16_body<D, PT>
template <int D>
constexpr size_t hash_bf16_lds() {
  return 4 * (D + 2 + 32 + 2 * kRefinePairs + 16) * sizeof(double) + 16 * (D + 8) * sizeof(uint16_t) +
         4 * 16 * D * sizeof(uint16_t) + 4 * kRefinePairs + 4 * sizeof(uint32_t);
}

// The jobs with rows, with tile_end filled in (16-row tiles in job order);
// returns the number of tiles.
inline int64_t hash_tiles(const HashJobs& jobs, HashJobs* js) {
  js->count = 0;
  int64_t tiles = 0;
  for (int i = 0; i < jobs.count; ++i) {
    const HashJob& j = jobs.j[i];
    if ((int64_t)j.H * j.N == 0) continue;
    js->j[js->count] = j;
    tiles += (int64_t)j.H * ((j.N + 15) / 16);
    js->tile_end[js->count] = tiles;
    ++js->count;
  }
  return tiles;
}

// the probe class of a launch's jobs: 2 when every job has at most two
// probes, else 3 (the template argument PT of hash_bf16_body)
__host__ __device__ inline int hash_probe_class(const HashJobs& js) {
  int pt = 2;
  for (int i = 0; i < js.count; ++i) pt = js.j[i].P > 2 ? 3 : pt;
  return pt;
}

// v summed over the 16 lanes of its DPP row (the same value in all of them:
// every step adds a lane's value and its partner's, which commutes)
__device__ __forceinline__ double row16_sum_d(double v) {
  auto step = [](double x, auto dpp) {
    const uint64_t u = __builtin_bit_cast(uint64_t, x);
    const uint32_t lo = (uint32_t)dpp((int)(uint32_t)u), hi = (uint32_t)dpp((int)(uint32_t)(u >> 32));
    return x + __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
  };
  v = step(v, [](int w) { return __builtin_amdgcn_update_dpp(w, w, 0xB1, 0xF, 0xF, false); });   // quad_perm [1,0,3,2]
  v = step(v, [](int w) { return __builtin_amdgcn_update_dpp(w, w, 0x4E, 0xF, 0xF, false); });   // quad_perm [2,3,0,1]
  v = step(v, [](int w) { return __builtin_amdgcn_update_dpp(w, w, 0x141, 0xF, 0xF, false); });  // row_half_mirror
  v = step(v, [](int w) { return __builtin_amdgcn_update_dpp(w, w, 0x140, 0xF, 0xF, false); });  // row_mirror
  return v;
}

// the value of lane l ^ 32 (as xor16_word)
__device__ __forceinline__ uint32_t xor32_word(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return r[0] == v ? r[1] : r[0];
}
// Nearest of lane ^ 16 (X = 16) or lane ^ 32 (X = 32) merged in, without
// LDS: the same (d1, d2, j1) in both lanes of a pair
template <int X>
__device__ __forceinline__ void nearest_merge_pl(Nearest& a) {
  auto other = [](uint32_t w) { return X == 16 ? xor16_word(w) : xor32_word(w); };
  const float pd1 = __uint_as_float(other(__float_as_uint(a.d1)));
  const float pd2 = __uint_as_float(other(__float_as_uint(a.d2)));
  const int pj1 = (int)other((uint32_t)a.j1);
  const bool take = (pd1 < a.d1) | ((pd1 == a.d1) & (pj1 < a.j1));
  const float nd2 = take ? (pd2 < a.d1 ? pd2 : a.d1) : (pd1 < a.d2 ? pd1 : a.d2);
  a.d1 = take ? pd1 : a.d1;
  a.j1 = take ? pj1 : a.j1;
  a.d2 = nd2;
}

// Workgroup `block` of nblocks (256 threads) of a bf16 hashing: one wave per
// tile of 16 rows of one of the jobs' tensors (tiles of tensor i are numbered
// from jobs.tile_end[i - 1]; tile_end filled by hash_tiles, fewer than 2^31
// tiles); the first tile's rows and the hyperplanes are requested together.
// PT: hash_probe_class of the jobs (2: every job has one or two probes).
// lds: hash_bf16_lds<D>() bytes, 16-byte aligned.
//
// Rows float32 cannot certify.  With one or two probes a tile's uncertain
// (row, hyperplane) pairs -- the signs within the float32 bound, and for a
// second probe the hyperplanes whose distance may be the row's smallest --
// are re-evaluated in float64 together, 16 lanes per pair and four pairs at
// a time; a row those cannot settle (a float64 sign within its bound, a
// nearest hyperplane float64 cannot separate, too many uncertain pairs) and
// every uncertain row with more probes take the whole-row float64 / exact
// pass of hash_fixup_row, one row at a time.
template <int D, int PT>
__device__ __forceinline__ void hash_bf16_body(const HashJobs& jobs, const uint16_t* __restrict__ planes, int nb,
                                               fastar_diag_t* __restrict__ diag, int block, int nblocks,
                                               char* lds) {
  static_assert(PT == 2 || PT == 3, "probe class 2 (one or two probes) or 3");
  constexpr int NC = D / 32;
  constexpr int kPst = D + 8;  // padded hyperplane rows: lanes reading 16 planes hit different banks
  constexpr int EPL = D / 16;  // dims per lane when 16 lanes share one projection
  // lds, per wave: [4][D + 2] doubles (exact sums), [4][32] doubles (second
  // probe), [4][2][kRefinePairs] doubles (refined sums and absolute sums),
  // [4][16] doubles (the hyperplanes' norms); then [16][kPst] hyperplanes,
  // [4][16][D] the waves' tiles' rows, [4][kRefinePairs] bytes (row | plane
  // << 4), and the workgroup's 3 diag counts
  double (*ex)[D + 2] = reinterpret_cast<double (*)[D + 2]>(lds);
  double (*de)[32] = reinterpret_cast<double (*)[32]>(lds + 4 * (D + 2) * sizeof(double));
  double (*rs)[2][kRefinePairs] =
      reinterpret_cast<double (*)[2][kRefinePairs]>(lds + 4 * (D + 2 + 32) * sizeof(double));
  double (*rn64)[16] =
      reinterpret_cast<double (*)[16]>(lds + 4 * (D + 2 + 32 + 2 * kRefinePairs) * sizeof(double));
  uint16_t* spl = reinterpret_cast<uint16_t*>(rn64 + 4);
  uint16_t (*trow)[16][D] = reinterpret_cast<uint16_t (*)[16][D]>(spl + 16 * kPst);
  uint8_t (*pairs)[kRefinePairs] = reinterpret_cast<uint8_t (*)[kRefinePairs]>(trow + 4);
  uint32_t* wgcount = reinterpret_cast<uint32_t*>(pairs + 4);
  const int l = lane_id();
  const int col = l & 15;
  const int g = l >> 4;
  const int wv = threadIdx.x >> 6;
  const int total = (int)jobs.tile_end[jobs.count - 1];
  const int nwaves = nblocks * (int)(blockDim.x >> 6);
  // wave-uniform (scalar tile bookkeeping)
  const int first = __builtin_amdgcn_readfirstlane(block * (int)(blockDim.x >> 6) + (int)(threadIdx.x >> 6));
  // tile -> tensor, head, first row (wave-uniform)
  struct Where {
    const uint16_t* x;
    int64_t sh, st, N, r0;
    int h, P;
    int32_t* bucket;
  };
  auto where = [&](int tile) {
    int ji = 0;
#pragma unroll
    for (int i = 1; i < kMaxHashJobs; ++i)
      if (i < jobs.count && tile >= jobs.tile_end[i - 1]) ji = i;
    Where w;
    int t0 = 0;
    // field-wise selects: no dynamic indexing of the argument block
#pragma unroll
    for (int i = 0; i < kMaxHashJobs; ++i)
      if (i == ji) {
        w.x = (const uint16_t*)jobs.j[i].x;
        w.sh = jobs.j[i].sh;
        w.st = jobs.j[i].st;
        w.N = jobs.j[i].N;
        w.P = jobs.j[i].P;
        w.bucket = jobs.j[i].bucket;
        t0 = i > 0 ? (int)jobs.tile_end[i - 1] : 0;
      }
    const uint32_t tph = (uint32_t)((w.N + 15) >> 4);
    const uint32_t local = (uint32_t)(tile - t0);
    w.h = (int)(local / tph);
    w.r0 = (int64_t)(local - (uint32_t)w.h * tph) << 4;
    return w;
  };
  auto load_rows = [&](const Where& w, uint4* u) {
    const int64_t row = w.r0 + col;
    const bool valid = row < w.N;
    const uint16_t* xr = w.x + (int64_t)w.h * w.sh + (valid ? row : w.r0) * w.st;
#pragma unroll
    for (int c = 0; c < NC; ++c) u[c] = *reinterpret_cast<const uint4*>(xr + 32 * c + 8 * g);
  };
  // The first tile's rows, the A operand and this thread's share of the
  // hyperplanes for the LDS copy are all in flight together; the copy is
  // written once the A operand has landed (its barrier orders LDS only).
  uint4 xu[NC];
  Where w{};
  if (first < total) {
    w = where(first);
    load_rows(w, xu);
  }

  // A operand: hyperplane `col`, dims 32c + 8g .. +8 of chunk c
  uint4 au[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    au[c] = make_uint4(0u, 0u, 0u, 0u);
    if (col < nb) au[c] = *reinterpret_cast<const uint4*>(planes + (int64_t)col * D + 32 * c + 8 * g);
  }
  static_assert(16 * D / 8 <= 256, "one 16-byte piece of the hyperplanes per thread");
  const int pi = threadIdx.x, pp = pi / (D / 8), p8 = pi % (D / 8);
  uint4 pu = make_uint4(0u, 0u, 0u, 0u);
  if (pi < 16 * D / 8 && pp < nb) pu = *reinterpret_cast<const uint4*>(planes + (int64_t)pp * D + 8 * p8);
  bf16x8_t aop[NC];
  float r2 = 0.f;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    r2 += sumsq_bf16x8(au[c]);
    aop[c] = __builtin_bit_cast(bf16x8_t, au[c]);
  }
  if (pi < 16 * D / 8) *reinterpret_cast<uint4*>(&spl[pp * kPst + 8 * p8]) = pu;
  if (threadIdx.x < 3) wgcount[threadIdx.x] = 0u;
  lds_barrier();
  bool have_rn64 = false;  // this wave's copy of the hyperplanes' float64 norms
  r2 += shfl_xor_f(r2, 16);
  r2 += shfl_xor_f(r2, 32);
  // the lane's four hyperplanes 4g + i: reciprocal norms and the factor of
  // |x| in their sign bounds; for hyperplanes past nb (projections 0) NaN and
  // -inf, which no comparison below takes: such a hyperplane is never
  // uncertain and never nearest
  const float kc = kcert<D>();
  float irn[4], kb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float rnorm = sqrtf(__shfl(r2, 4 * g + i, FASTAR_WAVE));
    const bool pv = 4 * g + i < nb;
    irn[i] = pv ? (rnorm > 0.f ? 1.f / rnorm : 0.f) : __builtin_nanf("");
    kb[i] = pv ? kc * rnorm : -INFINITY;
  }
  HashCounts hc;
  for (int tile = first; tile < total; tile += nwaves) {
    // the next tile's rows load while this one is hashed
    uint4 xn[NC];
    Where wn = w;
    if (tile + nwaves < total) {
      wn = where(tile + nwaves);
      load_rows(wn, xn);
    }
    const int64_t row = w.r0 + col;
    const bool valid = row < w.N;
    const int P = w.P;
    bf16x8_t bop[NC];
    float x2 = 0.f;
    uint32_t nzb = 0u;  // any element nonzero (from the bits)
    // (a row past N holds row r0's values: hashed, never written)
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const uint4 u = xu[c];
      x2 += sumsq_bf16x8(u);
      nzb |= (u.x | u.y | u.z | u.w) & 0x7FFF7FFFu;
      bop[c] = __builtin_bit_cast(bf16x8_t, u);
    }
    x2 = sum_xor32(sum_xor16(x2));
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NC; ++c) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop[c], bop[c], acc, 0, 0, 0);
    // acc[i] = x_row(col) . r_(4g+i) (0 for hyperplanes past nb: their A rows are 0)
    const float xnorm = __builtin_amdgcn_sqrtf(x2);  // (within the bounds' slack)
    uint32_t bits = 0u, am = 0u;  // sign bits; hyperplanes whose sign float32 cannot certify
    float dl[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = 4 * g + i;
      const float s = acc[i];
      bits |= (s > 0.f ? 1u : 0u) << p;
      am |= fabsf(s) <= fmaf(kb[i], xnorm, 0x1p-90f) ? 1u << p : 0u;
      dl[i] = fabsf(s) * irn[i];  // within 2^-22 relative of the quotient
    }
    bits = or_xor32(or_xor16(bits));
    am = or_xor32(or_xor16(am));
    // a zero row (every element +-0, from the bits: no underflow question):
    // every projection is exactly 0 (id 0) and every distance 0, so the
    // probes flip bits 0, 1, .. in order (ties to the smaller index);
    // nothing to certify
    const bool zero = or_xor32(or_xor16(nzb)) == 0u;
    Nearest nr{INFINITY, INFINITY, 0};
    bool near_amb = false;
    uint32_t nearu = 0u;  // hyperplanes whose distance may be the row's smallest
    if (PT == 3 || P == 2) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool lt = dl[i] < nr.d1;  // (a NaN distance, past nb, is never taken)
        nr.d2 = lt ? nr.d1 : (dl[i] < nr.d2 ? dl[i] : nr.d2);
        nr.j1 = lt ? 4 * g + i : nr.j1;
        nr.d1 = lt ? dl[i] : nr.d1;
      }
      nearest_merge_pl<16>(nr);
      nearest_merge_pl<32>(nr);
      // each distance is known to within kc*|x| (plus the rounding of the
      // reciprocal norm and of the product)
      const float e0 = 2.f * kc * xnorm + 0x1p-90f;
      near_amb = P == 2 && nr.d2 - nr.d1 <= e0 + (nr.d1 + nr.d2) * 0x1p-20f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        nearu |= (dl[i] - nr.d1 <= e0 + (nr.d1 + dl[i]) * 0x1p-20f) ? 1u << (4 * g + i) : 0u;
      nearu = or_xor32(or_xor16(nearu));
    }
    // more probes: every lane of the row gathers the row's 16 distances and
    // ranks its own 4 planes
    int rk[4] = {0, 0, 0, 0};
    bool amb = am != 0u || near_amb;
    if constexpr (PT == 3) {
      if (P > 2) {
        float da[16];
#pragma unroll
        for (int g2 = 0; g2 < 4; ++g2)
#pragma unroll
          for (int i = 0; i < 4; ++i) da[4 * g2 + i] = __shfl(dl[i], 16 * g2 + col, FASTAR_WAVE);
        const bool a2 = probe_ranks(dl, da, 4 * g, nb, P, 2.f * kc * xnorm + 0x1p-90f, rk);
        amb = or_xor32(or_xor16(amb || a2 ? 1u : 0u)) != 0u;
        if (zero) {
#pragma unroll
          for (int i = 0; i < 4; ++i) rk[i] = 4 * g + i;
        }
      }
    }
    if (zero) {
      amb = false;
      nr.j1 = 0;
    }
    int32_t* const orow = w.bucket + ((int64_t)w.h * w.N + row) * P;
    if (valid && g == 0 && !amb) {
      orow[0] = (int32_t)bits;
      if (P == 2) orow[1] = (int32_t)(bits ^ (1u << nr.j1));
    }
    if constexpr (PT == 3) {
      if (P > 2 && valid && !amb) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (4 * g + i < nb && rk[i] < P - 1) orow[1 + rk[i]] = (int32_t)(bits ^ (1u << (4 * g + i)));
      }
    }
    uint64_t ab = ballot64(valid && g == 0 && amb);  // bit = the row's column
    if (ab) {
      // the tile's rows to LDS (read by the re-evaluations; in order within the wave)
#pragma unroll
      for (int c = 0; c < NC; ++c) *reinterpret_cast<uint4*>(&trow[wv][col][32 * c + 8 * g]) = xu[c];
      uint64_t whole = ab;  // rows for the whole-row pass
      if (PT == 2 || P <= 2) {
        // (row, hyperplane) pairs in row order, each row's in hyperplane order
        const uint32_t um = am | (near_amb ? nearu : 0u);
        const int cnt = (g == 0 && valid && amb && __builtin_popcount(um) <= kRefineRowMax) ? __builtin_popcount(um) : 0;
        const int incl = (int)wave_incl_scan_dpp((uint32_t)cnt);  // lanes 0..15: within their row
        const int excl = incl - cnt;
        const bool fits = cnt > 0 && incl <= kRefinePairs;
        if (fits) {
          uint32_t m = um;
          for (int k = excl; m; ++k) {
            pairs[wv][k] = (uint8_t)(col | (__builtin_ctz(m) << 4));
            m &= m - 1u;
          }
        }
        const int npairs = __builtin_amdgcn_readfirstlane(wave_reduce_dpp(fits ? incl : 0, [](int a, int b) { return max(a, b); }));
        if (!have_rn64) {
          // the hyperplanes' norms in float64 (squares of bf16 values are
          // exact), from the A operand: lane (p, g) holds a quarter of plane p
          double n2 = 0.0;
#pragma unroll
          for (int c = 0; c < NC; ++c) {
            const uint4 u = __builtin_bit_cast(uint4, aop[c]);
            const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const double lo = (double)bf16_bits_to_f32(wd[k] & 0xFFFFu);
              const double hi = (double)__uint_as_float(wd[k] & 0xFFFF0000u);
              n2 = fma(lo, lo, n2);
              n2 = fma(hi, hi, n2);
            }
          }
          n2 = sum4_d(n2);
          if (g == 0) rn64[wv][col] = sqrt(n2);
          have_rn64 = true;
        }
        // four pairs at a time: lane j of quarter q takes dims EPL j .. +EPL
        const int q = l >> 4, j = l & 15;
        for (int k0 = 0; k0 < npairs; k0 += 4) {
          const int k = k0 + q;
          double s = 0.0, a = 0.0;
          if (k < npairs) {
            const int pr = pairs[wv][k];
            const uint16_t* xp = &trow[wv][pr & 15][EPL * j];
            const uint16_t* rp = &spl[(pr >> 4) * kPst + EPL * j];
            uint32_t xw[EPL / 2], rw[EPL / 2];
            if constexpr (EPL == 8) {
              const uint4 xv = *reinterpret_cast<const uint4*>(xp), rv = *reinterpret_cast<const uint4*>(rp);
              xw[0] = xv.x, xw[1] = xv.y, xw[2] = xv.z, xw[3] = xv.w;
              rw[0] = rv.x, rw[1] = rv.y, rw[2] = rv.z, rw[3] = rv.w;
            } else {
              const uint2 xv = *reinterpret_cast<const uint2*>(xp), rv = *reinterpret_cast<const uint2*>(rp);
              xw[0] = xv.x, xw[1] = xv.y;
              rw[0] = rv.x, rw[1] = rv.y;
            }
#pragma unroll
            for (int e = 0; e < EPL / 2; ++e) {
              // products of bf16 values are exact in float64
              const double x0 = (double)bf16_bits_to_f32(xw[e] & 0xFFFFu), x1 = (double)__uint_as_float(xw[e] & 0xFFFF0000u);
              const double r0 = (double)bf16_bits_to_f32(rw[e] & 0xFFFFu), r1 = (double)__uint_as_float(rw[e] & 0xFFFF0000u);
              s = fma(x0, r0, s);
              s = fma(x1, r1, s);
              a = fma(fabs(x0), fabs(r0), a);
              a = fma(fabs(x1), fabs(r1), a);
            }
          }
          s = row16_sum_d(s);
          a = row16_sum_d(a);
          if (j == 0 && k < npairs) {
            rs[wv][0][k] = s;
            rs[wv][1][k] = a;
          }
        }
        // each refined row's decisions, by its lane of g == 0
        bool settled = false;
        if (fits) {
          uint32_t fb = bits;
          bool ok = true;
          int m = -1;
          double dm = 0.0, em = 0.0, lb = INFINITY;  // nearest so far, its error; the others' lower bound
          for (int k = excl; k < incl; ++k) {
            const int p = pairs[wv][k] >> 4;
            const double s = rs[wv][0][k];
            // any order of the D additions is within this bound
            const double bound = 2.0 * (D + 8) * 0x1p-53 * rs[wv][1][k];
            if ((am >> p) & 1u) {
              if (fabs(s) > bound) fb = (fb & ~(1u << p)) | ((s > 0.0 ? 1u : 0u) << p);
              else ok = false;
            }
            if (near_amb && ((nearu >> p) & 1u)) {
              const double rn = rn64[wv][p];
              if (!(rn > 0.0)) {
                ok = false;
              } else {
                const double dp = fabs(s) / rn;
                const double ep = bound / rn + dp * (2 * D + 8) * 0x1p-53;
                if (m < 0 || dp < dm) {  // hyperplanes come in index order: ties stay with the smaller
                  if (m >= 0) lb = fmin(lb, dm - em);
                  m = p, dm = dp, em = ep;
                } else {
                  lb = fmin(lb, dp - ep);
                }
              }
            }
          }
          // the hyperplanes outside nearu are farther than the row's
          // nearest by the float32 bounds; the float64 nearest must stand
          // apart from the other candidates
          if (near_amb && ok && !(lb > dm + em)) ok = false;
          if (ok) {
            orow[0] = (int32_t)fb;
            if (P == 2) orow[1] = (int32_t)(fb ^ (1u << (near_amb ? m : nr.j1)));
            settled = true;
          }
        }
        whole = ballot64(settled) ^ ab;
      }
      hc.rows += (uint32_t)(__builtin_popcountll(ab) - __builtin_popcountll(whole));
      while (whole) {
        const int r = __builtin_ctzll(whole);  // wave-uniform
        whole &= whole - 1;
        hash_fixup_row<uint16_t, D>(&trow[wv][r][0], spl, kPst, w.bucket + ((int64_t)w.h * w.N + w.r0 + r) * P,
                                    P, nb, hc, ex[wv], de[wv]);
      }
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) xu[c] = xn[c];
    w = wn;
  }
  // the workgroup's counts, then one device atomic per counter: many waves
  // adding to the same word at the end of a launch held it up
  if (diag) {
    if (lane_id() == 0) {
      if (hc.rows) atomicAdd(&wgcount[0], hc.rows);
      if (hc.signs) atomicAdd(&wgcount[1], hc.signs);
      if (hc.unresolved) atomicAdd(&wgcount[2], hc.unresolved);
    }
    lds_barrier();
    if (threadIdx.x == 0) {
      HashCounts wc;
      wc.rows = wgcount[0], wc.signs = wgcount[1], wc.unresolved = wgcount[2];
      hash_counts_flush(wc, diag);
    }
  }
}


}  // namespace fastar
