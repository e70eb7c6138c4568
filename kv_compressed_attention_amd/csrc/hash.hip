// SimHash bucket ids on gfx950.
//
// Bucket id bit j is the sign of x . r_j (hyperplane hashing, paperlayer.ai
// section 5 "ANN Attention"); the optional second probe flips the bit of the
// hyperplane nearest to x.
//
// bf16 inputs: the projection X[N x d] . R^T[d x b] runs on MFMA
// (v_mfma_f32_16x16x32_bf16) with the hyperplanes as the A operand (16 rows,
// b <= 15 of them used) and 16 rows of X as the B operand, so each lane ends
// up holding 4 projections of one row and the sign bits of a row are OR-ed
// over 4 lanes.  fp32 inputs use the vector ALUs (one row per lane).
//
// A float32 projection is trusted only when its magnitude exceeds an a-priori
// bound on its rounding error, Kd * |x| * |r_j| with Kd = d * 2^-22 (four times
// the worst case of a d-term float32 accumulation of exact products).  A row
// with any untrusted sign or second-probe choice is re-evaluated on the spot
// by its whole wave in float64 (products of bf16/fp32 values are exact there),
// and a sign float64 still cannot certify is settled exactly with an
// error-free expansion sum.

#include "common.h"
#include "kernels.h"

namespace fastar {

namespace {

__device__ __forceinline__ float sumsq_bf16x8(uint4 u) {
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
// slices.  The row (xr: [D]) and the hyperplanes (ps, row stride pst) are
// read from LDS.  A sign float64 cannot certify is settled exactly with an
// expansion sum in E (D + 2 doubles of LDS); the second probe's distances
// and error bounds go through DE (32 doubles of LDS).
template <typename T, int D>
__device__ void hash_fixup_row(const T* xr, const T* ps, int pst, int32_t* __restrict__ o, int P,
                               int nb, fastar_diag_t* __restrict__ diag, double* E, double* DE) {
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
      if (diag) atomicAdd(&diag->hash_exact_signs, 1u);
    }
    sx = __shfl(sx, src, FASTAR_WAVE);
    if (p == src) sg = sx;
  }
  const uint32_t bits = (uint32_t)(ballot64(sg > 0) & 0xFFFFu);
  int j1 = 0;
  bool unresolved = false;
  if (P == 2) {
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
    if (lane == 0) {
      const double* dist = DE;
      const double* derr = DE + 16;
      double d1 = dist[0], e1 = derr[0];
      for (int q = 1; q < nb; ++q) {
        if (dist[q] < d1) {
          j1 = q;
          d1 = dist[q];
          e1 = derr[q];
        }
      }
      for (int q = 0; q < nb; ++q) {
        if (q != j1) {
          const double gap = dist[q] - d1;
          const double err = derr[q] + e1;
          if (err > 0.0 && gap <= err) unresolved = true;
        }
      }
    }
  }
  if (lane == 0) {
    o[0] = (int32_t)bits;
    if (P == 2) o[1] = (int32_t)(bits ^ (1u << j1));
    if (diag) {
      atomicAdd(&diag->hash_fallback_rows, 1u);
      if (unresolved) atomicAdd(&diag->unresolved, 1u);
    }
  }
}

// One wave per tile of 16 rows of one of the launch's tensors (tiles of
// tensor i are numbered from jobs.tile_end[i - 1]); the first tile's rows
// are requested before the hyperplanes are read.
template <int D>
__global__ __launch_bounds__(256, 4) void hash_bf16_kernel(HashJobs jobs, const uint16_t* __restrict__ planes,
                                                        int nb, fastar_diag_t* __restrict__ diag) {
  constexpr int NC = D / 32;
  constexpr int kPst = D + 8;  // padded hyperplane rows: lanes reading 16 planes hit different banks
  __shared__ __attribute__((aligned(16))) uint16_t spl[16 * kPst];
  __shared__ __attribute__((aligned(16))) uint16_t sxr[4][D];  // per wave: the row being re-evaluated
  __shared__ double ex[4][D + 2];
  __shared__ double de[4][32];
  const int l = lane_id();
  const int col = l & 15;
  const int g = l >> 4;
  const int wv = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < 16 * D / 8; i += blockDim.x) {
    const int pp = i / (D / 8), c8 = i % (D / 8);
    uint4 u = make_uint4(0u, 0u, 0u, 0u);
    if (pp < nb) u = *reinterpret_cast<const uint4*>(planes + (int64_t)pp * D + 8 * c8);
    *reinterpret_cast<uint4*>(&spl[pp * kPst + 8 * c8]) = u;
  }
  __syncthreads();
  const int64_t total = jobs.tile_end[jobs.count - 1];
  const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
  const int64_t first = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
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
  uint4 xu[NC];
  if (first < total) load_rows(where(first), xu);

  // A operand: hyperplane `col`, dims 32c + 8g .. +8 of chunk c
  bf16x8_t aop[NC];
  float r2 = 0.f;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    uint4 u = make_uint4(0u, 0u, 0u, 0u);
    if (col < nb) u = *reinterpret_cast<const uint4*>(planes + (int64_t)col * D + 32 * c + 8 * g);
    r2 += sumsq_bf16x8(u);
    aop[c] = __builtin_bit_cast(bf16x8_t, u);
  }
  r2 += shfl_xor_f(r2, 16);
  r2 += shfl_xor_f(r2, 32);
  float rnorm[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) rnorm[i] = sqrtf(__shfl(r2, 4 * g + i, FASTAR_WAVE));

  const float kc = kcert<D>();
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
          const float dist = rnorm[i] > 0.f ? fabsf(s) / rnorm[i] : 0.f;
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
    if (P == 2) {
      nearest_merge(nr, 16);
      nearest_merge(nr, 32);
      // each distance is known to within kc*|x| (plus division rounding)
      const float err = 2.f * kc * xnorm + (nr.d1 + nr.d2) * 0x1p-20f + 0x1p-90f;
      if (nr.d2 - nr.d1 <= err) amb = 1;
    }
    if (valid && g == 0 && !amb) {
      int32_t* o = w.bucket + ((int64_t)w.h * w.N + row) * P;
      o[0] = (int32_t)bits;
      if (P == 2) o[1] = (int32_t)(bits ^ (1u << nr.j1));
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
                                  P, nb, diag, ex[wv], de[wv]);
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) xu[c] = xn[c];
  }
}

template <int D, int P>
__global__ __launch_bounds__(256) void hash_f32_kernel(
    const float* __restrict__ x, int64_t sh, int64_t st, int H, int64_t N,
    const float* __restrict__ planes, int nb, int32_t* __restrict__ bucket,
    fastar_diag_t* __restrict__ diag) {
  __shared__ float sp[16][D];
  __shared__ float sxr[4][D];  // per wave: the row being re-evaluated
  __shared__ double ex[4][D + 2];
  __shared__ double de[4][32];
  __shared__ float srn[16];
  for (int i = threadIdx.x; i < 16 * D; i += blockDim.x) {
    const int p = i / D;
    sp[p][i % D] = p < nb ? planes[i] : 0.f;
  }
  __syncthreads();
  if (threadIdx.x < 16) {
    float r2 = 0.f;
    for (int d = 0; d < D; ++d) r2 = fmaf(sp[threadIdx.x][d], sp[threadIdx.x][d], r2);
    srn[threadIdx.x] = sqrtf(r2);
  }
  __syncthreads();
  const float kc = kcert<D>();
  const int64_t total = (int64_t)H * N;
  // the loop is uniform per wave so that the wave can settle rows together
  for (int64_t base = (int64_t)blockIdx.x * blockDim.x + (threadIdx.x & ~63); base < total;
       base += (int64_t)gridDim.x * blockDim.x) {
    const int64_t idx = base + lane_id();
    const bool valid = idx < total;
    const int h = valid ? (int)(idx / N) : 0;
    const int64_t row = valid ? idx - (int64_t)h * N : 0;
    const float* xr = x + (int64_t)h * sh + row * st;
    float s[16];
#pragma unroll
    for (int p = 0; p < 16; ++p) s[p] = 0.f;
    float x2 = 0.f;
    for (int d = 0; d < D; ++d) {
      const float xv = xr[d];
      x2 = fmaf(xv, xv, x2);
#pragma unroll
      for (int p = 0; p < 16; ++p) s[p] = fmaf(xv, sp[p][d], s[p]);
    }
    const float xnorm = sqrtf(x2);
    uint32_t bits = 0;
    bool amb = false;
    Nearest nr{INFINITY, INFINITY, 0};
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      if (p < nb) {
        const float bound = kc * xnorm * srn[p] + 0x1p-90f;
        amb |= fabsf(s[p]) <= bound;
        if (s[p] > 0.f) bits |= 1u << p;
        if (P == 2) {
          const float dist = srn[p] > 0.f ? fabsf(s[p]) / srn[p] : 0.f;
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
    if (P == 2) {
      const float err = 2.f * kc * xnorm + (nr.d1 + nr.d2) * 0x1p-20f + 0x1p-90f;
      if (nr.d2 - nr.d1 <= err) amb = true;
    }
    if (valid && !amb) {
      int32_t* o = bucket + idx * P;
      o[0] = (int32_t)bits;
      if (P == 2) o[1] = (int32_t)(bits ^ (1u << nr.j1));
    }
    // rows float32 cannot certify: float64 by the whole wave, one at a
    // time, from an LDS copy
    uint64_t ab = ballot64(valid && amb);
    const int wv = threadIdx.x >> 6;
    while (ab) {
      const int r = __builtin_ctzll(ab);  // wave-uniform
      ab &= ab - 1;
      if (lane_id() == r)
        for (int d = 0; d < D; ++d) sxr[wv][d] = xr[d];
      hash_fixup_row<float, D>(sxr[wv], &sp[0][0], D, bucket + (base + r) * P, P, nb, diag, ex[wv],
                               de[wv]);
    }
  }
}

template <int D, int P>
hipError_t launch_hash_f32(const HashJob& j, const void* planes, int nb, fastar_diag_t* diag,
                           hipStream_t s) {
  const int64_t total = (int64_t)j.H * j.N;
  const int64_t blocks = (total + 255) / 256 < 8192 ? (total + 255) / 256 : 8192;
  hipLaunchKernelGGL((hash_f32_kernel<D, P>), dim3((unsigned)blocks), dim3(256), 0, s,
                     (const float*)j.x, j.sh, j.st, j.H, j.N, (const float*)planes, nb, j.bucket, diag);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_hash_multi(HashJobs jobs, int dim, int dtype, const void* planes, int n_bits,
                             fastar_diag_t* diag, hipStream_t s) {
  // drop empty tensors; tile ranges in launch order
  HashJobs js;
  js.count = 0;
  int64_t tiles = 0;
  for (int i = 0; i < jobs.count; ++i) {
    const HashJob& j = jobs.j[i];
    if ((int64_t)j.H * j.N == 0) continue;
    js.j[js.count] = j;
    tiles += (int64_t)j.H * ((j.N + 15) / 16);
    js.tile_end[js.count] = tiles;
    ++js.count;
  }
  if (js.count == 0) return hipSuccess;
  if (dtype == FASTAR_BF16) {
    // two tiles per wave: the second tile's rows load during the first
    const int64_t blocks = (tiles + 7) / 8 < 8192 ? (tiles + 7) / 8 : 8192;
    if (dim == 64)
      hipLaunchKernelGGL((hash_bf16_kernel<64>), dim3((unsigned)blocks), dim3(256), 0, s, js,
                         (const uint16_t*)planes, n_bits, diag);
    else
      hipLaunchKernelGGL((hash_bf16_kernel<128>), dim3((unsigned)blocks), dim3(256), 0, s, js,
                         (const uint16_t*)planes, n_bits, diag);
    return hipGetLastError();
  }
  for (int i = 0; i < js.count; ++i) {
    const HashJob& j = js.j[i];
    hipError_t e;
    if (dim == 64)
      e = j.P == 1 ? launch_hash_f32<64, 1>(j, planes, n_bits, diag, s) : launch_hash_f32<64, 2>(j, planes, n_bits, diag, s);
    else
      e = j.P == 1 ? launch_hash_f32<128, 1>(j, planes, n_bits, diag, s) : launch_hash_f32<128, 2>(j, planes, n_bits, diag, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_hash(const fastar_tensor_t& x, const void* planes, int n_bits, int n_probes,
                       int32_t* bucket, fastar_diag_t* diag, hipStream_t s) {
  HashJobs jobs;
  jobs.count = 1;
  jobs.j[0] = HashJob{x.data, x.stride_head, x.stride_token, x.tokens, x.heads, n_probes, bucket};
  return launch_hash_multi(jobs, x.dim, x.dtype, planes, n_bits, diag, s);
}

}  // namespace fastar
