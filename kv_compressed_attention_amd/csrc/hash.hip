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

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int m = 1; m < FASTAR_WAVE; m <<= 1) v += __shfl_xor(v, m, FASTAR_WAVE);
  return v;
}

// Re-evaluates one row in float64, the whole wave (each lane holds D/64
// dims), and writes its ids; a sign float64 cannot certify is settled
// exactly by lane 0 with an expansion sum in E (D + 2 doubles of LDS).
template <typename T, int D, int P>
__device__ void hash_fixup_row(const T* __restrict__ xr, const T* __restrict__ planes, int nb,
                               int32_t* __restrict__ o, fastar_diag_t* __restrict__ diag,
                               double* E) {
  constexpr int L = D / FASTAR_WAVE;
  const int lane = lane_id();
  double xv[L];
#pragma unroll
  for (int k = 0; k < L; ++k) xv[k] = (double)Elem<T>::load(xr, lane + FASTAR_WAVE * k);
  uint32_t bits = 0;
  double dist[16], derr[16];
  bool unresolved = false;
#pragma unroll
  for (int p = 0; p < 16; ++p) {
    dist[p] = 0.0;
    derr[p] = 0.0;
    if (p < nb) {
      double s = 0.0, a = 0.0, n2 = 0.0;
#pragma unroll
      for (int k = 0; k < L; ++k) {
        const double rv = (double)Elem<T>::load(planes, (int64_t)p * D + lane + FASTAR_WAVE * k);
        const double pr = xv[k] * rv;  // exact: at most 48 significant bits
        s += pr;
        a += fabs(pr);
        n2 += rv * rv;
      }
      s = wave_sum_d(s);
      a = wave_sum_d(a);
      n2 = wave_sum_d(n2);
      const double bound = 2.0 * (D + 8) * 0x1p-53 * a;
      int sg;
      if (fabs(s) > bound) {
        sg = s > 0.0 ? 1 : -1;
      } else if (a == 0.0) {
        sg = 0;
      } else {
        int sg0 = 0;
        if (lane == 0) {
          int m = 0;
          for (int d = 0; d < D; ++d) {
            const double xd = (double)Elem<T>::load(xr, d);
            const double rd = (double)Elem<T>::load(planes, (int64_t)p * D + d);
            m = grow_expansion(E, m, xd * rd);
          }
          sg0 = expansion_sign(E, m);
          if (diag) atomicAdd(&diag->hash_exact_signs, 1u);
        }
        sg = __shfl(sg0, 0, FASTAR_WAVE);
      }
      if (sg > 0) bits |= 1u << p;
      if (P == 2) {
        const double rn = sqrt(n2);
        dist[p] = rn > 0.0 ? fabs(s) / rn : 0.0;
        derr[p] = (a == 0.0) ? 0.0 : (rn > 0.0 ? bound / rn : 0.0) + dist[p] * (2 * D + 8) * 0x1p-53;
      }
    }
  }
  int j1 = 0;
  if (P == 2) {
    double d1 = dist[0], e1 = derr[0];
#pragma unroll
    for (int p = 1; p < 16; ++p) {
      if (p < nb && dist[p] < d1) {
        j1 = p;
        d1 = dist[p];
        e1 = derr[p];
      }
    }
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      if (p < nb && p != j1) {
        const double gap = dist[p] - d1;
        const double err = derr[p] + e1;
        if (err > 0.0 && gap <= err) unresolved = true;
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

template <int D, int P>
__global__ __launch_bounds__(256) void hash_bf16_kernel(
    const uint16_t* __restrict__ x, int64_t sh, int64_t st, int H, int64_t N,
    const uint16_t* __restrict__ planes, int nb, int32_t* __restrict__ bucket,
    fastar_diag_t* __restrict__ diag) {
  constexpr int NC = D / 32;
  __shared__ double ex[4][D + 2];
  const int l = lane_id();
  const int col = l & 15;
  const int g = l >> 4;

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
  const int64_t tiles_per_head = (N + 15) >> 4;
  const int64_t total = (int64_t)H * tiles_per_head;
  const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
  for (int64_t tile = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6); tile < total;
       tile += nwaves) {
    const int h = (int)(tile / tiles_per_head);
    const int64_t r0 = (tile - (int64_t)h * tiles_per_head) << 4;
    const int64_t row = r0 + col;
    const bool valid = row < N;
    const uint16_t* xr = x + (int64_t)h * sh + (valid ? row : r0) * st;
    bf16x8_t bop[NC];
    float x2 = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      uint4 u = *reinterpret_cast<const uint4*>(xr + 32 * c + 8 * g);
      if (!valid) u = make_uint4(0u, 0u, 0u, 0u);
      x2 += sumsq_bf16x8(u);
      bop[c] = __builtin_bit_cast(bf16x8_t, u);
    }
    x2 += shfl_xor_f(x2, 16);
    x2 += shfl_xor_f(x2, 32);
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
    bits |= (uint32_t)shfl_xor_i((int)bits, 16);
    bits |= (uint32_t)shfl_xor_i((int)bits, 32);
    amb |= shfl_xor_i(amb, 16);
    amb |= shfl_xor_i(amb, 32);
    if (P == 2) {
      nearest_merge(nr, 16);
      nearest_merge(nr, 32);
      // each distance is known to within kc*|x| (plus division rounding)
      const float err = 2.f * kc * xnorm + (nr.d1 + nr.d2) * 0x1p-20f + 0x1p-90f;
      if (nr.d2 - nr.d1 <= err) amb = 1;
    }
    if (valid && g == 0 && !amb) {
      int32_t* o = bucket + ((int64_t)h * N + row) * P;
      o[0] = (int32_t)bits;
      if (P == 2) o[1] = (int32_t)(bits ^ (1u << nr.j1));
    }
    // rows float32 cannot certify: float64 by the whole wave, one at a time
    uint64_t ab = ballot64(valid && g == 0 && amb);
    while (ab) {
      const int src = __builtin_ctzll(ab);  // = the row's column (g == 0)
      ab &= ab - 1;
      const int64_t rr = r0 + src;
      hash_fixup_row<uint16_t, D, P>(x + (int64_t)h * sh + rr * st, planes, nb,
                                     bucket + ((int64_t)h * N + rr) * P, diag,
                                     ex[threadIdx.x >> 6]);
    }
  }
}

template <int D, int P>
__global__ __launch_bounds__(256) void hash_f32_kernel(
    const float* __restrict__ x, int64_t sh, int64_t st, int H, int64_t N,
    const float* __restrict__ planes, int nb, int32_t* __restrict__ bucket,
    fastar_diag_t* __restrict__ diag) {
  __shared__ float sp[16][D];
  __shared__ double ex[4][D + 2];
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
    uint64_t ab = ballot64(valid && amb);
    while (ab) {
      const int src = __builtin_ctzll(ab);
      ab &= ab - 1;
      const int64_t e = base + src;
      const int hh = (int)(e / N);
      const int64_t rr = e - (int64_t)hh * N;
      hash_fixup_row<float, D, P>(x + (int64_t)hh * sh + rr * st, planes, nb, bucket + e * P, diag,
                                  ex[threadIdx.x >> 6]);
    }
  }
}

template <int D, int P>
hipError_t launch_hash_dp(const fastar_tensor_t& x, const void* planes, int nb, int32_t* bucket,
                          fastar_diag_t* diag, hipStream_t s) {
  const int H = x.heads;
  const int64_t N = x.tokens;
  if (x.dtype == FASTAR_BF16) {
    const int64_t tiles = (int64_t)H * ((N + 15) / 16);
    const int64_t blocks = (tiles + 3) / 4 < 8192 ? (tiles + 3) / 4 : 8192;
    hipLaunchKernelGGL((hash_bf16_kernel<D, P>), dim3((unsigned)blocks), dim3(256), 0, s,
                       (const uint16_t*)x.data, x.stride_head, x.stride_token, H, N,
                       (const uint16_t*)planes, nb, bucket, diag);
  } else {
    const int64_t total = (int64_t)H * N;
    const int64_t blocks = (total + 255) / 256 < 8192 ? (total + 255) / 256 : 8192;
    hipLaunchKernelGGL((hash_f32_kernel<D, P>), dim3((unsigned)blocks), dim3(256), 0, s,
                       (const float*)x.data, x.stride_head, x.stride_token, H, N,
                       (const float*)planes, nb, bucket, diag);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_hash(const fastar_tensor_t& x, const void* planes, int n_bits, int n_probes,
                       int32_t* bucket, fastar_diag_t* diag, hipStream_t s) {
  if ((int64_t)x.heads * x.tokens == 0) return hipSuccess;
  if (x.dim == 64)
    return n_probes == 1 ? launch_hash_dp<64, 1>(x, planes, n_bits, bucket, diag, s)
                         : launch_hash_dp<64, 2>(x, planes, n_bits, bucket, diag, s);
  return n_probes == 1 ? launch_hash_dp<128, 1>(x, planes, n_bits, bucket, diag, s)
                       : launch_hash_dp<128, 2>(x, planes, n_bits, bucket, diag, s);
}

}  // namespace fastar
