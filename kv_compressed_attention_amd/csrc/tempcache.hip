// TempCache merge on gfx950 (paperlayer.ai section 5 "TempCache", appendix A
// Lemma 5.1, appendix C representative and threshold ablations).
//
// Frames are merged one after another; per frame three kernels run:
//   tc_match    each new key j scans the previous frame's bucket ids (staged in
//               LDS) for candidates sharing its bucket, and keeps the candidate
//               of largest cosine if it passes tau;
//   tc_resolve  a candidate proposed to by several keys keeps the proposer of
//               largest cosine (ties: smaller j); records the group it extends;
//   tc_apply    numbers the unmatched keys as new groups in ascending j (block
//               scan) and updates the group rows: count, float32 value sum,
//               bf16/fp32 value mean rounded once, representative key and
//               bucket, ln(count); 16 lanes cooperate on each 128-dim row.
// Cosines are compared in float32 with a certified error bound; a comparison
// inside the bound is redone in float64 (where products of the stored values
// are exact) and counted in the diagnostics.

#include "common.h"
#include "kernels.h"

namespace fastar {

namespace {

template <typename T, int D>
struct Row;

template <int D>
struct Row<uint16_t, D> {
  static __device__ __forceinline__ void load(const uint16_t* p, float* o) {
#pragma unroll
    for (int c = 0; c < D / 8; ++c) {
      const uint4 u = reinterpret_cast<const uint4*>(p)[c];
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        o[8 * c + 2 * i] = __uint_as_float(w[i] << 16);
        o[8 * c + 2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      }
    }
  }
  // dot with a register row and squared norm of the memory row
  static __device__ __forceinline__ void dot(const uint16_t* p, const float* a, float& d, float& n2) {
    float s = 0.f, q = 0.f;
#pragma unroll
    for (int c = 0; c < D / 8; ++c) {
      const uint4 u = reinterpret_cast<const uint4*>(p)[c];
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float lo = __uint_as_float(w[i] << 16);
        const float hi = __uint_as_float(w[i] & 0xFFFF0000u);
        s = fmaf(a[8 * c + 2 * i], lo, s);
        s = fmaf(a[8 * c + 2 * i + 1], hi, s);
        q = fmaf(lo, lo, q);
        q = fmaf(hi, hi, q);
      }
    }
    d = s;
    n2 = q;
  }
};

template <int D>
struct Row<float, D> {
  static __device__ __forceinline__ void load(const float* p, float* o) {
#pragma unroll
    for (int c = 0; c < D / 4; ++c) {
      const float4 u = reinterpret_cast<const float4*>(p)[c];
      o[4 * c] = u.x;
      o[4 * c + 1] = u.y;
      o[4 * c + 2] = u.z;
      o[4 * c + 3] = u.w;
    }
  }
  static __device__ __forceinline__ void dot(const float* p, const float* a, float& d, float& n2) {
    float s = 0.f, q = 0.f;
#pragma unroll
    for (int c = 0; c < D / 4; ++c) {
      const float4 u = reinterpret_cast<const float4*>(p)[c];
      s = fmaf(a[4 * c], u.x, s);
      s = fmaf(a[4 * c + 1], u.y, s);
      s = fmaf(a[4 * c + 2], u.z, s);
      s = fmaf(a[4 * c + 3], u.w, s);
      q = fmaf(u.x, u.x, q);
      q = fmaf(u.y, u.y, q);
      q = fmaf(u.z, u.z, q);
      q = fmaf(u.w, u.w, q);
    }
    d = s;
    n2 = q;
  }
};

// bound on |fl32(cos) - cos|: dot and both norms of d exact products
// accumulated in float32, then rsqrt and two multiplies; twice the estimate
template <int D>
__device__ __forceinline__ float cos_err32() { return (float)(4 * D + 32) * 0x1p-24f; }
template <int D>
__device__ __forceinline__ double cos_err64() { return (double)(4 * D + 32) * 0x1p-53; }

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

template <typename T, int D>
__global__ __launch_bounds__(256) void tc_match_kernel(
    const T* __restrict__ rep_k, int cap, const int32_t* __restrict__ rep_bucket,
    const int32_t* __restrict__ frontier, int Tf, const T* __restrict__ knew, int64_t k_sh,
    int64_t k_st, int64_t frame_off, const int32_t* __restrict__ kbucket, int64_t kb_stride,
    const int32_t* __restrict__ ng_in, float tau, int32_t* __restrict__ target,
    float* __restrict__ tcos, fastar_diag_t* __restrict__ diag) {
  extern __shared__ int pb[];
  const int h = blockIdx.y;
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (ng_in[h] <= 0) {  // empty cache: nothing to match (uniform per block)
    if (j < Tf) {
      target[(int64_t)h * Tf + j] = -1;
      tcos[(int64_t)h * Tf + j] = 0.f;
    }
    return;
  }
  const int32_t* fr = frontier + (int64_t)h * Tf;
  for (int i = threadIdx.x; i < Tf; i += blockDim.x) {
    const int g = fr[i];
    pb[i] = g >= 0 ? rep_bucket[(int64_t)h * cap + g] : -1;
  }
  __syncthreads();
  if (j >= Tf) return;
  const int bj = kbucket[(int64_t)h * kb_stride + frame_off + j];
  const T* kj = knew + (int64_t)h * k_sh + (frame_off + j) * k_st;
  const T* rk = rep_k + (int64_t)h * cap * D;
  float a[D];
  Row<T, D>::load(kj, a);
  float nj2 = 0.f;
#pragma unroll
  for (int d = 0; d < D; ++d) nj2 = fmaf(a[d], a[d], nj2);
  const float rj = nj2 > 0.f ? rsqrtf(nj2) : 0.f;
  int best = -1;
  float c1 = -INFINITY, c2 = -INFINITY;
  for (int i = 0; i < Tf; ++i) {
    if (pb[i] != bj) continue;
    float dt, ni2;
    Row<T, D>::dot(rk + (int64_t)fr[i] * D, a, dt, ni2);
    const float c = (nj2 > 0.f && ni2 > 0.f) ? dt * rj * rsqrtf(ni2) : 0.f;
    if (c > c1) {
      c2 = c1;
      c1 = c;
      best = i;
    } else if (c > c2) {
      c2 = c;
    }
  }
  bool prop = false;
  float cb = c1;
  if (best >= 0) {
    const float e = cos_err32<D>();
    const bool amb = (c1 - c2 <= 2.f * e) || (fabsf(c1 - tau) <= e);
    if (!amb) {
      prop = c1 >= tau;
    } else {
      if (diag) atomicAdd(&diag->merge_fallbacks, 1u);
      double d1 = -INFINITY, d2 = -INFINITY;
      int b64 = -1;
      for (int i = 0; i < Tf; ++i) {
        if (pb[i] != bj) continue;
        const double c = cos64<T, D>(kj, rk + (int64_t)fr[i] * D);
        if (c > d1) {
          d2 = d1;
          d1 = c;
          b64 = i;
        } else if (c > d2) {
          d2 = c;
        }
      }
      const double e64 = cos_err64<D>();
      if ((d1 - d2 <= 2.0 * e64) || (fabs(d1 - (double)tau) <= e64)) {
        if (diag) atomicAdd(&diag->unresolved, 1u);
      }
      best = b64;
      prop = d1 >= (double)tau;
      cb = (float)d1;
    }
  }
  target[(int64_t)h * Tf + j] = prop ? best : -1;
  tcos[(int64_t)h * Tf + j] = cb;
}

template <typename T, int D>
__global__ __launch_bounds__(256) void tc_resolve_kernel(
    const T* __restrict__ rep_k, int cap, const int32_t* __restrict__ frontier, int Tf,
    const T* __restrict__ knew, int64_t k_sh, int64_t k_st, int64_t frame_off,
    const int32_t* __restrict__ target, const float* __restrict__ tcos,
    int32_t* __restrict__ mgroup, fastar_diag_t* __restrict__ diag) {
  extern __shared__ int sm[];
  int* tg = sm;
  float* tc = reinterpret_cast<float*>(sm + Tf);
  const int h = blockIdx.y;
  for (int i = threadIdx.x; i < Tf; i += blockDim.x) {
    tg[i] = target[(int64_t)h * Tf + i];
    tc[i] = tcos[(int64_t)h * Tf + i];
  }
  __syncthreads();
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= Tf) return;
  const int i = tg[j];
  if (i < 0) {
    mgroup[(int64_t)h * Tf + j] = -1;
    return;
  }
  const float e = cos_err32<D>();
  const float cj = tc[j];
  bool win = true, amb = false;
  for (int j2 = 0; j2 < Tf; ++j2) {
    if (j2 == j || tg[j2] != i) continue;
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
    for (int j2 = 0; j2 < Tf; ++j2) {
      if (j2 == j || tg[j2] != i) continue;
      const double d = cos64<T, D>(kh + (frame_off + j2) * k_st, prev);
      if (fabs(d - dj) <= 2.0 * e64) unres = true;
      if (d > dj || (d == dj && j2 < j)) win = false;
    }
    if (unres && diag) atomicAdd(&diag->unresolved, 1u);
  }
  mgroup[(int64_t)h * Tf + j] = win ? frontier[(int64_t)h * Tf + i] : -1;
}

template <typename T, int D>
__global__ __launch_bounds__(256) void tc_apply_kernel(
    T* __restrict__ rep_k, T* __restrict__ v_mean, float* __restrict__ v_sum,
    int32_t* __restrict__ count, float* __restrict__ log_count, int32_t* __restrict__ rep_bucket,
    int32_t* __restrict__ frontier, int cap, int Tf, const T* __restrict__ knew, int64_t k_sh,
    int64_t k_st, const T* __restrict__ vnew, int64_t v_sh, int64_t v_st, int64_t frame_off,
    const int32_t* __restrict__ kbucket, int64_t kb_stride, const int32_t* __restrict__ mgroup,
    const int32_t* __restrict__ ng_in, int32_t* __restrict__ ng_out,
    int32_t* __restrict__ group_of_new, fastar_diag_t* __restrict__ diag) {
  __shared__ int s_g[256];
  __shared__ int s_new[256];
  __shared__ int s_w[4];
  __shared__ int s_prior[4];
  const int h = blockIdx.y;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = lane_id();
  const int64_t j0 = (int64_t)blockIdx.x * 256;
  const int64_t j = j0 + tid;
  const bool valid = j < Tf;
  const int32_t* mg_h = mgroup + (int64_t)h * Tf;
  // new keys before this block
  int c = 0;
  for (int64_t jj = tid; jj < j0; jj += 256) c += mg_h[jj] < 0;
#pragma unroll
  for (int m = 1; m < FASTAR_WAVE; m <<= 1) c += shfl_xor_i(c, m);
  if (lane == 0) s_prior[wave] = c;
  const int mg = valid ? mg_h[j] : 0;
  const bool isnew = valid && mg < 0;
  const uint64_t bal = ballot64(isnew);
  if (lane == 0) s_w[wave] = __popcll(bal);
  __syncthreads();
  const int prior = s_prior[0] + s_prior[1] + s_prior[2] + s_prior[3];
  int rank = prior + __popcll(bal & lanemask_lt());
  for (int w = 0; w < wave; ++w) rank += s_w[w];
  const int ng0 = ng_in[h];
  int g = isnew ? ng0 + rank : mg;
  if (isnew && g >= cap) {
    g = -1;
    if (diag) atomicAdd(&diag->capacity_overflow, 1u);
  }
  if (valid) {
    if (group_of_new) group_of_new[(int64_t)h * kb_stride + frame_off + j] = g;
    frontier[(int64_t)h * Tf + j] = g;
  }
  if (blockIdx.x == gridDim.x - 1 && tid == 0) {
    const int total = prior + s_w[0] + s_w[1] + s_w[2] + s_w[3];
    const int ng1 = ng0 + total;
    ng_out[h] = ng1 < cap ? ng1 : cap;
  }
  s_g[tid] = valid ? g : -1;
  s_new[tid] = isnew ? 1 : 0;
  __syncthreads();
  // row updates, 16 lanes per row, EPL contiguous elements per lane
  constexpr int EPL = D / 16;
  const int sub = tid & 15;
  for (int rs = tid >> 4; rs < 256; rs += 16) {
    const int gg = s_g[rs];
    if (gg < 0) continue;
    const int64_t jj = j0 + rs;
    const int64_t gi = (int64_t)h * cap + gg;
    const T* kr = knew + (int64_t)h * k_sh + (frame_off + jj) * k_st + sub * EPL;
    const T* vr = vnew + (int64_t)h * v_sh + (frame_off + jj) * v_st + sub * EPL;
    T* rkr = rep_k + gi * D + sub * EPL;
    T* vmr = v_mean + gi * D + sub * EPL;
    float* vsr = v_sum + gi * D + sub * EPL;
    const int bkt = kbucket[(int64_t)h * kb_stride + frame_off + jj];
    if (s_new[rs]) {
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
}

__global__ void copy_i32_kernel(const int32_t* __restrict__ src, int32_t* __restrict__ dst, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src[i];
}

template <typename T, int D>
hipError_t merge_td(const fastar_cache_t& c, const fastar_tensor_t& kn, const fastar_tensor_t& vn,
                    const int32_t* kb, int F, float tau, int32_t* group_of_new, int32_t* rep_offsets,
                    int32_t* rep_perm, const MergeWs& ws, fastar_diag_t* diag, hipStream_t s) {
  const int H = c.heads, Tf = c.tokens_per_frame, cap = c.capacity;
  const int64_t kb_stride = (int64_t)F * Tf;
  const dim3 grid((unsigned)((Tf + 255) / 256), (unsigned)H);
  hipLaunchKernelGGL(copy_i32_kernel, dim3((H + 255) / 256), dim3(256), 0, s, c.n_groups, ws.ng, H);
  for (int f = 0; f < F; ++f) {
    const int64_t foff = (int64_t)f * Tf;
    const int32_t* ng_in = ws.ng + (int64_t)f * H;
    int32_t* ng_out = ws.ng + (int64_t)(f + 1) * H;
    hipLaunchKernelGGL((tc_match_kernel<T, D>), grid, dim3(256), Tf * sizeof(int), s,
                       (const T*)c.rep_k, cap, c.rep_bucket, c.frontier, Tf, (const T*)kn.data,
                       kn.stride_head, kn.stride_token, foff, kb, kb_stride, ng_in, tau,
                       ws.target, ws.tcos, diag);
    hipLaunchKernelGGL((tc_resolve_kernel<T, D>), grid, dim3(256), Tf * (sizeof(int) + sizeof(float)),
                       s, (const T*)c.rep_k, cap, c.frontier, Tf, (const T*)kn.data, kn.stride_head,
                       kn.stride_token, foff, ws.target, ws.tcos, ws.mgroup, diag);
    hipLaunchKernelGGL((tc_apply_kernel<T, D>), grid, dim3(256), 0, s, (T*)c.rep_k, (T*)c.v_mean,
                       c.v_sum, c.count, c.log_count, c.rep_bucket, c.frontier, cap, Tf,
                       (const T*)kn.data, kn.stride_head, kn.stride_token, (const T*)vn.data,
                       vn.stride_head, vn.stride_token, foff, kb, kb_stride, ws.mgroup, ng_in,
                       ng_out, group_of_new, diag);
  }
  const int32_t* ng_final = ws.ng + (int64_t)F * H;
  hipLaunchKernelGGL(copy_i32_kernel, dim3((H + 255) / 256), dim3(256), 0, s, ng_final, c.n_groups, H);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (rep_offsets && rep_perm)
    return launch_bucket_index(c.rep_bucket, H, cap, 1, c.n_bits, ng_final, rep_offsets, rep_perm,
                               ws.index_ws, s);
  return hipSuccess;
}

}  // namespace

hipError_t launch_tempcache_merge(const fastar_cache_t& c, const fastar_tensor_t& k_new,
                                  const fastar_tensor_t& v_new, const int32_t* k_new_bucket,
                                  int n_frames, float tau, int32_t* group_of_new,
                                  int32_t* rep_offsets, int32_t* rep_perm, const MergeWs& ws,
                                  fastar_diag_t* diag, hipStream_t s) {
  if (c.heads == 0) return hipSuccess;
  if (c.dtype == FASTAR_BF16)
    return c.dim == 64
               ? merge_td<uint16_t, 64>(c, k_new, v_new, k_new_bucket, n_frames, tau, group_of_new, rep_offsets, rep_perm, ws, diag, s)
               : merge_td<uint16_t, 128>(c, k_new, v_new, k_new_bucket, n_frames, tau, group_of_new, rep_offsets, rep_perm, ws, diag, s);
  return c.dim == 64
             ? merge_td<float, 64>(c, k_new, v_new, k_new_bucket, n_frames, tau, group_of_new, rep_offsets, rep_perm, ws, diag, s)
             : merge_td<float, 128>(c, k_new, v_new, k_new_bucket, n_frames, tau, group_of_new, rep_offsets, rep_perm, ws, diag, s);
}

}  // namespace fastar
