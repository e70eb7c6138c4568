// SimHash hashing of bf16 rows as a workgroup-level body (the hash launch
// runs it, and so may other launches in workgroups of their own), and the
// float64 re-evaluation of rows float32 cannot certify.  See hash.hip for the
// method and its error bounds.
#pragma once

#include "common.h"
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
// doubles of LDS); the second probe's distances and error bounds go through
// DE (32 doubles of LDS).
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
    // (ties to the smaller index), each certified apart from every other
    const double* dist = DE;
    const double* derr = DE + 16;
    uint32_t used = 0u;
    for (int r = 0; r + 1 < P; ++r) {
      int jb = -1;
      for (int q = 0; q < nb; ++q)
        if (!((used >> q) & 1u) && (jb < 0 || dist[q] < dist[jb])) jb = q;
      used |= 1u << jb;
      for (int q = 0; q < nb; ++q) {
        const double err = derr[q] + derr[jb];
        if (q != jb && err > 0.0 && fabs(dist[q] - dist[jb]) <= err) unresolved = true;
      }
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

// LDS bytes of hash_bf16_body<D>
template <int D>
constexpr size_t hash_bf16_lds() {
  return 4 * (D + 2 + 32) * sizeof(double) + 16 * (D + 8) * sizeof(uint16_t) + 4 * D * sizeof(uint16_t);
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

// Workgroup `block` of nblocks (256 threads) of a bf16 hashing: one wave per
// tile of 16 rows of one of the jobs' tensors (tiles of tensor i are numbered
// from jobs.tile_end[i - 1]; tile_end filled by hash_tiles); the first tile's
// rows and the hyperplanes are requested together.  256 threads.  lds:
// hash_bf16_lds<D>()
// bytes, 16-byte aligned.
template <int D>
__device__ __forceinline__ void hash_bf16_body(const HashJobs& jobs, const uint16_t* __restrict__ planes, int nb,
                                               fastar_diag_t* __restrict__ diag, int block, int nblocks,
                                               char* lds) {
  constexpr int NC = D / 32;
  constexpr int kPst = D + 8;  // padded hyperplane rows: lanes reading 16 planes hit different banks
  // lds: [4][D + 2] doubles (exact sums), [4][32] doubles (second probe),
  // [16][kPst] hyperplanes (for rows float32 cannot certify), [4][D] per
  // wave the row being re-evaluated
  double (*ex)[D + 2] = reinterpret_cast<double (*)[D + 2]>(lds);
  double (*de)[32] = reinterpret_cast<double (*)[32]>(lds + 4 * (D + 2) * sizeof(double));
  uint16_t* spl = reinterpret_cast<uint16_t*>(lds + 4 * (D + 2 + 32) * sizeof(double));
  uint16_t (*sxr)[D] = reinterpret_cast<uint16_t (*)[D]>(spl + 16 * kPst);
  const int l = lane_id();
  const int col = l & 15;
  const int g = l >> 4;
  const int wv = threadIdx.x >> 6;
  const int64_t total = jobs.tile_end[jobs.count - 1];
  const int64_t nwaves = (int64_t)nblocks * (blockDim.x >> 6);
  const int64_t first = (int64_t)block * (blockDim.x >> 6) + (threadIdx.x >> 6);
  // tile -> tensor, head, first row (wave-uniform)
  struct Where {
    const uint16_t* x;
    int64_t sh, st, N, r0;
    int h, P;
    int32_t* bucket;
  };
  auto where = [&](int64_t tile) {
    int ji = 0;
#pragma unroll
    for (int i = 1; i < kMaxHashJobs; ++i)
      if (i < jobs.count && tile >= jobs.tile_end[i - 1]) ji = i;
    Where w;
    int64_t t0 = 0;
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
        t0 = i > 0 ? jobs.tile_end[i - 1] : 0;
      }
    const int64_t tph = (w.N + 15) >> 4;
    const int64_t local = tile - t0;
    w.h = (int)(local / tph);
    w.r0 = (local - (int64_t)w.h * tph) << 4;
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
  if (first < total) load_rows(where(first), xu);

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
  lds_barrier();
  r2 += shfl_xor_f(r2, 16);
  r2 += shfl_xor_f(r2, 32);
  float rnorm[4], irn[4];  // the lane's four hyperplanes' norms and their reciprocals
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    rnorm[i] = sqrtf(__shfl(r2, 4 * g + i, FASTAR_WAVE));
    irn[i] = rnorm[i] > 0.f ? 1.f / rnorm[i] : 0.f;
  }

  const float kc = kcert<D>();
  HashCounts hc;
  for (int64_t tile = first; tile < total; tile += nwaves) {
    const Where w = where(tile);
    // the next tile's rows load while this one is hashed
    uint4 xn[NC];
    if (tile + nwaves < total) load_rows(where(tile + nwaves), xn);
    const int64_t row = w.r0 + col;
    const bool valid = row < w.N;
    const int P = w.P;
    bf16x8_t bop[NC];
    float x2 = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      uint4 u = xu[c];
      if (!valid) u = make_uint4(0u, 0u, 0u, 0u);
      x2 += sumsq_bf16x8(u);
      bop[c] = __builtin_bit_cast(bf16x8_t, u);
    }
    x2 = sum_xor32(sum_xor16(x2));
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NC; ++c) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop[c], bop[c], acc, 0, 0, 0);
    // acc[i] = x_row(col) . r_(4g+i)
    const float xnorm = sqrtf(x2);
    uint32_t bits = 0;
    int amb = 0;
    Nearest nr{INFINITY, INFINITY, 0};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = 4 * g + i;
      if (p < nb) {
        const float s = acc[i];
        const float bound = kc * xnorm * rnorm[i] + 0x1p-90f;
        amb |= fabsf(s) <= bound;
        if (s > 0.f) bits |= 1u << p;
        if (P == 2) {
          const float dist = fabsf(s) * irn[i];  // within 2^-22 relative of the quotient
          if (dist < nr.d1) {
            nr.d2 = nr.d1;
            nr.d1 = dist;
            nr.j1 = p;
          } else if (dist < nr.d2) {
            nr.d2 = dist;
          }
        }
      }
    }
    bits = or_xor32(or_xor16(bits));
    amb = (int)or_xor32(or_xor16((uint32_t)amb));
    // a zero row (every element +-0, from the bits: no underflow question):
    // every projection is exactly 0 (id 0) and every distance 0, so the
    // probes flip bits 0, 1, .. in order (ties to the smaller index);
    // nothing to certify
    uint32_t nzb = 0u;
#pragma unroll
    for (int c = 0; c < NC; ++c) nzb |= (xu[c].x | xu[c].y | xu[c].z | xu[c].w) & 0x7FFF7FFFu;
    const bool zero = valid && or_xor32(or_xor16(nzb)) == 0u;
    if (P == 2) {
      nearest_merge(nr, 16);
      nearest_merge(nr, 32);
      // each distance is known to within kc*|x| (plus the rounding of the
      // reciprocal norm and of the product)
      const float err = 2.f * kc * xnorm + (nr.d1 + nr.d2) * 0x1p-20f + 0x1p-90f;
      if (nr.d2 - nr.d1 <= err) amb = 1;
    }
    if (zero) {
      amb = 0;
      nr.j1 = 0;
    }
    // more probes: every lane of the row gathers the row's 16 distances and
    // ranks its own 4 planes
    int rk[4] = {0, 0, 0, 0};
    if (P > 2) {
      float dl[4], da[16];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        dl[i] = (4 * g + i < nb) ? fabsf(acc[i]) * irn[i] : INFINITY;
#pragma unroll
      for (int g2 = 0; g2 < 4; ++g2)
#pragma unroll
        for (int i = 0; i < 4; ++i) da[4 * g2 + i] = __shfl(dl[i], 16 * g2 + col, FASTAR_WAVE);
      const bool a2 = probe_ranks(dl, da, 4 * g, nb, P, 2.f * kc * xnorm + 0x1p-90f, rk);
      amb = (int)or_xor32(or_xor16((uint32_t)(amb | (a2 ? 1 : 0))));
      if (zero) {
        amb = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) rk[i] = 4 * g + i;
      }
    }
    if (valid && g == 0 && !amb) {
      int32_t* o = w.bucket + ((int64_t)w.h * w.N + row) * P;
      o[0] = (int32_t)bits;
      if (P == 2) o[1] = (int32_t)(bits ^ (1u << nr.j1));
    }
    if (P > 2 && valid && !amb) {
      int32_t* o = w.bucket + ((int64_t)w.h * w.N + row) * P;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (4 * g + i < nb && rk[i] < P - 1) o[1 + rk[i]] = (int32_t)(bits ^ (1u << (4 * g + i)));
    }
    // rows float32 cannot certify: float64 by the whole wave, one at a
    // time, from an LDS copy
    uint64_t ab = ballot64(valid && g == 0 && amb);  // bit = the row's column
    while (ab) {
      const int r = __builtin_ctzll(ab);  // wave-uniform
      ab &= ab - 1;
      if (col == r) {
        // the 4 lanes holding row r copy its dims 32c + 8g .. +8
#pragma unroll
        for (int c = 0; c < NC; ++c) *reinterpret_cast<uint4*>(&sxr[wv][32 * c + 8 * g]) = xu[c];
      }
      hash_fixup_row<uint16_t, D>(sxr[wv], spl, kPst, w.bucket + ((int64_t)w.h * w.N + w.r0 + r) * P,
                                  P, nb, hc, ex[wv], de[wv]);
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) xu[c] = xn[c];
  }
  hash_counts_flush(hc, diag);
}


}  // namespace fastar
