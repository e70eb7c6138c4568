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
// the worst case of a d-term float32 accumulation of exact products).  With
// bf16 inputs and one or two probes, the untrusted projections of a tile (a
// sign, or the distances that may be a row's smallest) are re-evaluated in
// float64 together (products of bf16 values are exact there); a row that
// still cannot be certified, every uncertain row with more probes and every
// uncertain fp32 row are re-evaluated whole by their wave in float64; a
// sign float64 still cannot certify is settled exactly with an error-free
// expansion sum, and an order of two probe distances by integer arithmetic.

#include "common.h"
#include "hash_body.h"
#include "kernels.h"

namespace fastar {

namespace {

// One workgroup of 256 threads per hash_bf16_body block.
template <int D, int PT>
__global__ __launch_bounds__(256, 4) void hash_bf16_kernel(HashJobs jobs, const uint16_t* __restrict__ planes,
                                                        int nb, fastar_diag_t* __restrict__ diag) {
  __shared__ __attribute__((aligned(16))) char lds[hash_bf16_lds<D>()];
  hash_bf16_body<D, PT>(jobs, planes, nb, diag, blockIdx.x, gridDim.x, lds);
}

// PT: 1, 2, or 3 for any P >= 3 (given by P)
template <int D, int PT>
__global__ __launch_bounds__(256) void hash_f32_kernel(
    const float* __restrict__ x, int64_t sh, int64_t st, int H, int64_t N,
    const float* __restrict__ planes, int nb, int32_t* __restrict__ bucket,
    fastar_diag_t* __restrict__ diag, int P) {
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
  HashCounts hc;
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
    uint32_t nzb = 0u;  // any element nonzero (from the bits)
    for (int d = 0; d < D; ++d) {
      const float xv = xr[d];
      nzb |= __float_as_uint(xv) & 0x7FFFFFFFu;
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
    // more probes: rank the row's distances, four planes at a time
    int rk[16];
    if (P > 2) {
      float da[16];
#pragma unroll
      for (int p = 0; p < 16; ++p) da[p] = p < nb ? (srn[p] > 0.f ? fabsf(s[p]) / srn[p] : 0.f) : INFINITY;
#pragma unroll
      for (int p0 = 0; p0 < 16; p0 += 4)
        amb = probe_ranks(da + p0, da, p0, nb, P, 2.f * kc * xnorm + 0x1p-90f, rk + p0) || amb;
    }
    // a zero row: id 0, probes flip bits 0, 1, .. in order (every distance 0)
    if (nzb == 0u) {
      amb = false;
      nr.j1 = 0;
#pragma unroll
      for (int p = 0; p < 16; ++p) rk[p] = p;
    }
    if (valid && !amb) {
      int32_t* o = bucket + idx * P;
      o[0] = (int32_t)bits;
      if (P == 2) o[1] = (int32_t)(bits ^ (1u << nr.j1));
      if (P > 2) {
#pragma unroll
        for (int p = 0; p < 16; ++p)
          if (p < nb && rk[p] < P - 1) o[1 + rk[p]] = (int32_t)(bits ^ (1u << p));
      }
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
      hash_fixup_row<float, D>(sxr[wv], &sp[0][0], D, bucket + (base + r) * P, P, nb, hc, ex[wv],
                               de[wv]);
    }
  }
  hash_counts_flush(hc, diag);
}

template <int D>
hipError_t launch_hash_f32(const HashJob& j, const void* planes, int nb, fastar_diag_t* diag,
                           hipStream_t s) {
  const int64_t total = (int64_t)j.H * j.N;
  const int64_t blocks = (total + 255) / 256 < 8192 ? (total + 255) / 256 : 8192;
  auto kern = j.P == 1 ? hash_f32_kernel<D, 1> : j.P == 2 ? hash_f32_kernel<D, 2> : hash_f32_kernel<D, 3>;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(256), 0, s, (const float*)j.x, j.sh, j.st, j.H, j.N,
                     (const float*)planes, nb, j.bucket, diag, j.P);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_hash_multi(HashJobs jobs, int dim, int dtype, const void* planes, int n_bits,
                             fastar_diag_t* diag, hipStream_t s) {
  // drop empty tensors; tile ranges in launch order
  HashJobs js;
  const int64_t tiles = hash_tiles(jobs, &js);
  if (js.count == 0) return hipSuccess;
  if (dtype == FASTAR_BF16) {
    // tiles per wave: a wave with more loads the next tile's rows while it
    // hashes one, and amortises its hyperplane set-up; but at least about
    // 800 workgroups (three per CU) keep the loads spread.  Measured best:
    // up to 4
    int64_t tpw = tiles / (4 * 800);
    tpw = tpw < 1 ? 1 : (tpw > 4 ? 4 : tpw);
    const int64_t want = (tiles + 4 * tpw - 1) / (4 * tpw);
    const int64_t blocks = want < 8192 ? want : 8192;
    if (tiles >= (int64_t)1 << 31) return hipErrorInvalidValue;  // tiles are numbered in 32 bits
    const bool two = hash_probe_class(js) == 2;
    auto kern = dim == 64 ? (two ? hash_bf16_kernel<64, 2> : hash_bf16_kernel<64, 3>)
                          : (two ? hash_bf16_kernel<128, 2> : hash_bf16_kernel<128, 3>);
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(256), 0, s, js, (const uint16_t*)planes, n_bits, diag);
    return hipGetLastError();
  }
  for (int i = 0; i < js.count; ++i) {
    const HashJob& j = js.j[i];
    const hipError_t e = dim == 64 ? launch_hash_f32<64>(j, planes, n_bits, diag, s)
                                   : launch_hash_f32<128>(j, planes, n_bits, diag, s);
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
